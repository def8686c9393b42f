"""Host-side tests of libtb's C ABI (no GPU needed).

They load the library, check that it exports every symbol the header
declares, compare tb_band_index with the oracle's band map bit for bit, and
check that invalid arguments are refused on the host before anything could
be enqueued (only argument combinations that fail validation are passed, so no
device is touched).
"""

import ctypes
import os
import re

import pytest

import oracle
from conftest import ROOT, BAND_FIXTURES, read_band_fixture

binding = pytest.importorskip("rank_factored_linear_amd.binding")
lib = binding.lib

HEADER = os.path.join(ROOT, "include", "tb.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tb_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("tb_band_index", "tb_linear_forward", "tb_reconstruct_weight", "tb_rel_frobenius_error"):
        assert required in names


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert names
    for name in names:
        assert hasattr(lib, name), name
        assert name in binding.EXPORTED, name


def test_band_index_matches_oracle_bit_exact():
    out = ctypes.c_int32()
    for L in range(1, 129):
        for G in range(1, L + 1):
            want = oracle.band_map(L, G)
            for l in range(L):
                assert lib.tb_band_index(L, G, l, ctypes.byref(out)) == 0
                assert out.value == want[l], (L, G, l)


@pytest.mark.parametrize("name", BAND_FIXTURES)
def test_band_index_golden(name):
    L, G, want = read_band_fixture(name)
    assert [binding.band_index(L, G, l) for l in range(L)] == want


def test_band_index_large_counts():
    # Far beyond the model sizes; checks the closed form's integer arithmetic.
    for L, G in ((1_000_003, 7), (2**31 - 1, 3), (2**31 - 1, 2**31 - 1), (65536, 1)):
        sizes = [L // G + (1 if b < L % G else 0) for b in range(G)] if G < 10 else None
        for l in (0, 1, L // 2, L - 2, L - 1):
            b = binding.band_index(L, G, l)
            if sizes is not None:
                start = sum(sizes[:b])
                assert start <= l < start + sizes[b]
            else:
                assert b == l  # G == L


@pytest.mark.parametrize("args", [(0, 1, 0), (5, 0, 0), (5, 6, 0), (5, 2, 5), (5, 2, -1), (-3, 1, 0)])
def test_band_index_invalid_leaves_output(args):
    out = ctypes.c_int32(-77)
    st = lib.tb_band_index(*args, ctypes.byref(out))
    assert st == binding.TB_ERR_INVALID_ARGUMENT
    assert out.value == -77
    assert lib.tb_last_error().decode()


def test_band_index_null_output():
    assert lib.tb_band_index(4, 2, 0, None) == binding.TB_ERR_INVALID_ARGUMENT


def test_status_strings():
    for code in range(4):
        assert lib.tb_status_string(code).decode()
    assert lib.tb_status_string(99).decode() == "unknown status"


FAKE = 0x100000  # 256-byte aligned non-NULL address; never dereferenced below


def _fwd(**kw):
    a = dict(x=FAKE, s=FAKE, w0=FAKE, u=FAKE, v=FAKE, y=FAKE, m=8, o=64, i=64, r=16, dt=binding.TB_BF16,
             ws=FAKE, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.tb_linear_forward(a["x"], a["s"], a["w0"], a["u"], a["v"], a["y"], a["m"], a["o"], a["i"], a["r"],
                                 a["dt"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(m=0), 1), (dict(o=0), 1), (dict(i=0), 1), (dict(r=-1), 1), (dict(dt=7), 1),
    (dict(x=None), 1), (dict(s=None, w0=None), 1), (dict(w0=None), 1), (dict(y=None), 1), (dict(ws=None), 1),
    (dict(u=None), 1), (dict(v=None), 1),
    (dict(i=60), 2), (dict(x=FAKE + 8), 2), (dict(w0=FAKE + 4), 2), (dict(u=FAKE + 2), 2),
    (dict(s=FAKE + 1), 2), (dict(y=FAKE + 1), 2), (dict(ws=FAKE + 16), 2), (dict(m=1 << 31), 2),
])
def test_forward_rejects_before_launch(kw, status):
    assert _fwd(**kw) == status
    assert lib.tb_last_error().decode()


@pytest.mark.parametrize("args,status", [
    ((FAKE, None, FAKE, 8, 64, 64, 1), 1),          # w
    ((None, FAKE, FAKE, 8, 64, 64, 1), 1),          # x
    ((FAKE, FAKE, None, 8, 64, 64, 1), 1),          # y
    ((FAKE, FAKE, FAKE, 0, 64, 64, 1), 1),          # m
    ((FAKE, FAKE, FAKE, 8, 64, 60, 1), 2),          # in_dim % 8
    ((FAKE, FAKE + 4, FAKE, 8, 64, 64, 1), 2),      # w alignment
    ((FAKE, FAKE, FAKE, 8, 64, 64, 9), 1),          # dtype
])
def test_dense_forward_rejects_before_launch(args, status):
    x, w, y, m, o, i, dt = args
    assert lib.tb_dense_forward(x, w, y, m, o, i, dt, FAKE, 1 << 20, None) == status
    assert lib.tb_dense_forward(FAKE, FAKE, FAKE, 8, 64, 64, 1, None, 1 << 20, None) == 1   # workspace
    assert lib.tb_last_error().decode()


def test_decomposition_rejects_before_launch():
    ptrs = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    sb = lib.tb_shared_block
    assert sb(None, 3, 64, 64, 1, FAKE, None) == 1
    assert sb(ptrs, 0, 64, 64, 1, FAKE, None) == 1
    assert sb(ptrs, binding.MAX_BAND_LAYERS + 1, 64, 64, 1, FAKE, None) == 1
    assert sb(ptrs, 3, 0, 64, 1, FAKE, None) == 1
    assert sb(ptrs, 3, 64, 64, 5, FAKE, None) == 1
    assert sb(ptrs, 3, 64, 64, 1, None, None) == 1
    bad = (ctypes.c_void_p * 3)(FAKE, None, FAKE)
    assert sb(bad, 3, 64, 64, 1, FAKE, None) == 1
    rs = lib.tb_row_scale
    assert rs(None, FAKE, 64, 64, 1, FAKE, None) == 1
    assert rs(FAKE, FAKE, 64, 0, 1, FAKE, None) == 1
    assert rs(FAKE, FAKE + 2, 64, 64, 1, FAKE, None) == 1
    lf = lib.tb_lowrank_factors
    args = [FAKE, FAKE, FAKE, 64, 48, 8, 1, FAKE, 16, 2, FAKE, FAKE, FAKE, 1 << 30, None]

    def call(**changes):
        a = list(args)
        for k, v in changes.items():
            a[int(k[1:])] = v
        return lf(*a)
    assert call(a5=17) == 1                    # rank > k
    assert call(a8=49) == 1                    # k > in_dim
    assert call(a5=-1) == 1
    assert call(a9=17) == 1                    # power iterations
    assert call(a0=None) == 1 and call(a7=None) == 1 and call(a12=None) == 1
    assert call(a10=None) == 1                 # u_out with rank > 0
    assert call(a2=FAKE + 2) == 1              # misaligned s
    assert call(a6=4) == 1                     # dtype
    assert call(a3=1 << 20, a4=1 << 12) == 2   # out * in >= 2^31
    assert call(a3=600, a4=600, a8=513, a5=8) == 2   # k above the widest probe
    lb = lib.tb_lowrank_factors_batch
    w3 = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    w0_bad = (ctypes.c_void_p * 3)(FAKE, None, FAKE)
    bargs = [w3, 3, w3, FAKE, 64, 48, 8, 1, FAKE, 16, 2, FAKE, FAKE, FAKE, 1 << 30, None]

    def bcall(**changes):
        a = list(bargs)
        for k, v in changes.items():
            a[int(k[1:])] = v
        return lb(*a)
    assert bcall(a0=None) == 1 and bcall(a2=None) == 1
    assert bcall(a1=0) == 1 and bcall(a1=binding.MAX_BAND_LAYERS + 1) == 1
    assert bcall(a2=w0_bad) == 1                # a NULL shared block
    assert bcall(a6=17) == 1 and bcall(a10=17) == 1
    rf = lib.tb_refine_shared_block
    p2 = (ctypes.c_void_p * 2)(FAKE, FAKE)
    n2 = (ctypes.c_void_p * 2)(FAKE, None)
    assert rf(None, p2, p2, p2, 2, 64, 48, 8, 1, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert rf(p2, p2, None, p2, 2, 64, 48, 8, 1, FAKE, FAKE, FAKE, 1 << 30, None) == 1   # u with rank > 0
    assert rf(p2, n2, p2, p2, 2, 64, 48, 8, 1, FAKE, FAKE, FAKE, 1 << 30, None) == 1     # a NULL scale
    assert rf(p2, p2, p2, p2, 0, 64, 48, 8, 1, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert rf(p2, p2, p2, p2, 2, 64, 48, 8, 1, FAKE, FAKE, FAKE, 16, None) == 1          # workspace too small
    assert rf(p2, p2, p2, p2, 2, 64, 48, 8, 1, FAKE, None, FAKE, 1 << 30, None) == 1
    out = ctypes.c_size_t(0)
    assert lib.tb_lowrank_factors_workspace_size(64, 48, 20, 16, ctypes.byref(out)) == 1
    assert lib.tb_lowrank_factors_workspace_size(64, 48, 8, 16, None) == 1
    assert lib.tb_last_error().decode()


def test_reconstruct_rejects_before_launch():
    f = lib.tb_reconstruct_weight
    assert f(None, FAKE, FAKE, FAKE, FAKE, 64, 64, 8, 1, 0, None) == 1
    assert f(FAKE, FAKE, None, FAKE, FAKE, 64, 64, 8, 1, 0, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 8, 1, 0, None) == 1
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 12, 8, 1, 0, None) == 2
    assert f(FAKE, FAKE + 2, FAKE, FAKE, FAKE, 64, 64, 8, 1, 0, None) == 2
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 8, 1, 5, None) == 1


def test_frobenius_rejects_before_launch():
    f = lib.tb_rel_frobenius_error
    ws = binding.FROBENIUS_WORKSPACE_BYTES
    assert f(None, FAKE, 4, 8, 0, FAKE, FAKE, ws, None) == 1
    assert f(FAKE, FAKE, 0, 8, 0, FAKE, FAKE, ws, None) == 1
    assert f(FAKE, FAKE, 4, 6, 0, FAKE, FAKE, ws, None) == 2
    assert f(FAKE, FAKE, 4, 8, 0, FAKE, FAKE, ws - 1, None) == 1
    assert f(FAKE, FAKE, 4, 8, 9, FAKE, FAKE, ws, None) == 1
    assert f(FAKE, FAKE + 4, 4, 8, 0, FAKE, FAKE, ws, None) == 2


def test_reconstruction_error_rejects_before_launch():
    f = lib.tb_reconstruction_error
    ws = binding.FROBENIUS_WORKSPACE_BYTES
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 64, 64, 8, 1, 0, FAKE, FAKE, ws, None]

    def call(**changes):
        a = list(args)
        for k, v in changes.items():
            a[int(k[1:])] = v
        return f(*a)
    assert call(a0=None) == 1                 # s
    assert call(a4=None) == 1                 # original
    assert call(a2=None) == 1                 # u with rank > 0
    assert call(a5=0) == 1                    # out_dim
    assert call(a6=12) == 2                   # in_dim % 8
    assert call(a4=FAKE + 4) == 2             # original alignment
    assert call(a8=7) == 1 and call(a9=7) == 1
    assert call(a12=ws - 1) == 1              # workspace too small
    assert call(a10=FAKE + 4) == 2            # result alignment
    assert lib.tb_last_error().decode()


def test_workspace_size_rejects_bad_arguments():
    out = ctypes.c_size_t(0)
    assert lib.tb_linear_forward_workspace_size(0, 64, 64, 0, 0, ctypes.byref(out)) == 1
    assert lib.tb_linear_forward_workspace_size(1, 64, 64, 0, 0, None) == 1
    assert lib.tb_linear_forward_workspace_size(1, 64, 63, 0, 0, ctypes.byref(out)) == 2


def _group(n=2, **kw):
    """A tb_projection array of n members with placeholder pointers; kw overrides member 0."""
    arr = (binding.Projection * max(n, 1))()
    for j in range(max(n, 1)):
        a = dict(x=FAKE, s=FAKE, w0=FAKE, u=FAKE, v=FAKE, y=FAKE, o=64, i=64, r=16)
        if j == 0:
            a.update(kw)
        arr[j] = binding.Projection(a["x"], a["s"], a["w0"], a["u"], a["v"], a["y"], a["o"], a["i"], a["r"])
    return arr


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(y=None), 1), (dict(u=None), 1), (dict(o=0), 1), (dict(r=-1), 1),
    (dict(i=60), 2), (dict(x=FAKE + 8), 2), (dict(s=FAKE + 1), 2),
])
def test_group_rejects_bad_member_before_launch(kw, status):
    arr = _group(3, **kw)
    assert lib.tb_linear_forward_group(3, arr, 8, binding.TB_BF16, FAKE, 1 << 24, None) == status
    assert lib.tb_last_error().decode()


def test_group_rejects_bad_call_before_launch():
    f = lib.tb_linear_forward_group
    arr = _group(2)
    assert f(0, arr, 8, binding.TB_BF16, FAKE, 1 << 24, None) == 1
    assert f(binding.MAX_GROUP + 1, arr, 8, binding.TB_BF16, FAKE, 1 << 24, None) == 1
    assert f(2, None, 8, binding.TB_BF16, FAKE, 1 << 24, None) == 1
    assert f(2, arr, 8, binding.TB_BF16, None, 1 << 24, None) == 1
    assert f(2, arr, 8, binding.TB_BF16, FAKE + 16, 1 << 24, None) == 2
    assert f(2, arr, 0, binding.TB_BF16, FAKE, 1 << 24, None) == 1
    assert f(2, arr, 8, 7, FAKE, 1 << 24, None) == 1
    out = ctypes.c_size_t(0)
    g = lib.tb_linear_forward_group_workspace_size
    assert g(0, arr, 8, binding.TB_BF16, ctypes.byref(out)) == 1
    assert g(2, arr, 8, binding.TB_BF16, None) == 1
    assert g(2, _group(2, i=63), 8, binding.TB_BF16, ctypes.byref(out)) == 2
