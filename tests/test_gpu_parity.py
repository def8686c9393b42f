"""GPU parity: libtb through its C ABI against the float64 oracle.

Every test calls the HIP kernels through ``rank_factored_linear_amd.binding``
(ctypes over tb.h) and compares with the oracle on the exact stored inputs.
Criteria (parity_util.check_forward / check_reconstruct): relative Frobenius
error <= 5e-3 (bf16 inputs, fp32 accumulate) or <= 1e-5 (fp32) over the
output, the same over every tile of 16 output features (rows of a rebuilt
weight one by one), and every element within a worst-case bound derived from
the arithmetic; band indices and rank-0 fp32 reconstruction bit-exact.
Outputs of up to 16 tokens are compared whole; larger ones on one output
feature and one token from every tile the kernels write.
"""

import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from rank_factored_linear_amd import inputs as gen
from parity_util import (BF16_TOL, F32_TOL, bits_to_device, check_forward, check_reconstruct, exact, f32_to_device,
                         stale_control_words, tile_sample, tol_for)

pytestmark = pytest.mark.gpu

tb = pytest.importorskip("rank_factored_linear_amd.binding")
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


def test_native_library_is_loaded():
    with open("/proc/self/maps") as f:
        maps = f.read()
    assert os.path.realpath(tb.LIB_PATH) in maps
    assert torch.cuda.is_available()
    _say("device:", torch.cuda.get_device_name(0))


# ---------------------------------------------------------------------------
# Tiny fp32 stack: oracle decomposition, GPU forward / reconstruct / error
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("rank", [16, 256])
def test_tiny_fp32_stack(rank):
    _say(f"tiny fp32 stack rank={rank}")
    weights, x = gen.tiny_stack()
    bun = oracle.decompose(weights, 2, rank)
    x32 = x.astype(np.float32)
    for l in range(gen.TINY_LAYERS):
        band = tb.band_index(gen.TINY_LAYERS, 2, l)
        assert band == bun["band"][l] == gen.TINY_LAYER_BAND[l]
        W0 = bun["W0"][band].astype(np.float32)
        s = bun["s"][l].astype(np.float32)
        U = bun["U"][l].astype(np.float32)
        V = bun["V"][l].astype(np.float32)
        y = tb.linear_forward(f32_to_device(x32), f32_to_device(s), f32_to_device(W0), f32_to_device(U), f32_to_device(V))
        check_forward(exact(y), x32, s, W0, U, V, bf16=False, what=f"tiny layer {l}")
        rec = tb.reconstruct_weight(f32_to_device(s), f32_to_device(W0), f32_to_device(U), f32_to_device(V))
        check_reconstruct(exact(rec), s, W0, U, V, bf16_out=False, what=f"tiny rebuild layer {l}")
        orig = f32_to_device(weights[l].astype(np.float32))
        e_gpu = float(tb.rel_frobenius_error(orig, rec).item())
        e_ref = oracle.relative_frobenius_error(exact(orig), exact(rec))
        assert abs(e_gpu - e_ref) <= 1e-9 + 1e-9 * e_ref
        if rank == 256:
            assert e_gpu < 1e-5  # a full-rank delta leaves only fp32 rounding


# ---------------------------------------------------------------------------
# Passthrough 26-layer bf16 stack: output equals the plain layer x W^T
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("family", gen.FAMILIES)
def test_passthrough_stack_bf16(family):
    for layer in (0, 13, 25):
        assert tb.band_index(26, 26, layer) == layer
        b = gen.bundle_bf16_host(2, family, gen.SHAPES_26, layer, layer, 0, passthrough=True)
        W = bits_to_device(b["W0"])
        s = bits_to_device(b["s"])
        Wd = exact(W)
        for M in (1, 8, 64):
            _say(f"passthrough {family} layer={layer} M={M}")
            x = bits_to_device(gen.activations_bf16_host(2, family, gen.SHAPES_26, layer, M))
            y = tb.linear_forward(x, s, W, None, None)
            check_forward(exact(y), exact(x), exact(s), Wd, np.zeros((Wd.shape[0], 0)), np.zeros((Wd.shape[1], 0)),
                          bf16=True, what=f"passthrough {family} layer {layer} M={M}")
        rec = tb.reconstruct_weight(s, W, None, None, out_dtype=torch.float32)
        assert np.array_equal(exact(rec), Wd)                    # rebuilt weight is the original
        assert float(tb.rel_frobenius_error(W.float(), rec).item()) == 0.0


# ---------------------------------------------------------------------------
# Banded 26-layer bf16 stack, rank 128, G in {1, 4}
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("M", [4, 2048])
@pytest.mark.parametrize("family", gen.FAMILIES)
def test_banded_stack_bf16(G, M, family):
    want_bands = oracle.band_map(26, G)
    for layer in (0, 6, 7, 19, 20, 25):
        band = tb.band_index(26, G, layer)
        assert band == want_bands[layer]
        _say(f"banded G={G} M={M} {family} layer={layer} band={band}")
        b = gen.bundle_bf16_host(3, family, gen.SHAPES_26, layer, band, 128)
        t = {k: bits_to_device(v) for k, v in b.items()}
        x = bits_to_device(gen.activations_bf16_host(3, family, gen.SHAPES_26, layer, M))
        y = tb.linear_forward(x, t["s"], t["W0"], t["U"], t["V"])
        tsel = np.arange(M) if M <= 64 else tile_sample(M, seed=layer, tile=32)
        check_forward(exact(y)[tsel], exact(x)[tsel], exact(t["s"]), exact(t["W0"]), exact(t["U"]), exact(t["V"]),
                      bf16=True, what=f"banded G={G} M={M} {family} layer {layer}")


# ---------------------------------------------------------------------------
# Large 60-layer bf16 stack, rank 256, drawn on the device; sampled outputs
# ---------------------------------------------------------------------------


def _large_case(G, layer, family, M):
    band = tb.band_index(60, G, layer)
    assert band == oracle.band_index(60, G, layer)
    W0 = gen.device_w0(torch, 4, family, gen.SHAPES_60, band)
    bun = gen.device_bundle(torch, 4, family, gen.SHAPES_60, layer, band, 256, with_w0=False)
    x = gen.device_activations(torch, 4, family, gen.SHAPES_60, layer, M)
    y = tb.linear_forward(x, bun["s"], W0, bun["U"], bun["V"])
    what = f"large G={G} layer {layer} M={M} {family}"
    if M <= 16:       # every output row
        return check_forward(exact(y), exact(x), exact(bun["s"]), exact(W0), exact(bun["U"]), exact(bun["V"]),
                             bf16=True, what=what)
    # One output feature from every 16-row tile and one token from every 64-token tile.
    oi = torch.from_numpy(tile_sample(W0.shape[0], seed=layer + 7)).to(DEV)
    ti = torch.from_numpy(tile_sample(M, seed=layer + 11, tile=64)).to(DEV)
    return check_forward(exact(y.index_select(0, ti).index_select(1, oi)), exact(x.index_select(0, ti)),
                         exact(bun["s"].index_select(0, oi)), exact(W0.index_select(0, oi)),
                         exact(bun["U"].index_select(0, oi)), exact(bun["V"]), bf16=True, what=what)


def _parity_layers(G, L=60):
    """Layer 0, the first layer of every band and layer L-1 (with G = L: 0, L/2 - 1 and L-1)."""
    if G == L:
        return [0, L // 2 - 1, L - 1]
    bands = oracle.band_map(L, G)
    firsts = [l for l in range(L) if l == 0 or bands[l] != bands[l - 1]]
    return sorted(set(firsts) | {L - 1})


LARGE_SAMPLE = [(6, l) for l in _parity_layers(6)] + [(60, l) for l in _parity_layers(60)]


@pytest.mark.parametrize("G,layer", LARGE_SAMPLE)
@pytest.mark.parametrize("M", [1, 16, 4096])
@pytest.mark.parametrize("family", gen.FAMILIES)
def test_large_stack_bf16(G, layer, M, family):
    _say(f"large G={G} layer={layer} M={M} {family}")
    err = _large_case(G, layer, family, M)
    assert err <= BF16_TOL, err
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Reconstruction path bf16 -> fp32 and relative Frobenius error, 60 layers G=6
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("rank", [256, 128, 0])
@pytest.mark.parametrize("family", gen.FAMILIES)
def test_reconstruct_large(rank, family):
    for layer in _parity_layers(6):
        band = tb.band_index(60, 6, layer)
        _say(f"reconstruct rank={rank} {family} layer={layer} band={band}")
        W0 = gen.device_w0(torch, 5, family, gen.SHAPES_60, band)
        bun = gen.device_bundle(torch, 5, family, gen.SHAPES_60, layer, band, rank, with_w0=False)
        U, V = (bun["U"], bun["V"]) if rank else (None, None)
        rec = tb.reconstruct_weight(bun["s"], W0, U, V, out_dtype=torch.float32)
        orig = gen.device_original(torch, W0, 5, family, layer)
        e_gpu = float(tb.rel_frobenius_error(orig, rec).item())
        # Oracle on sampled rows for the reconstruction ...
        osel = tile_sample(W0.shape[0], seed=layer + 3)     # one row from every 16-row tile
        oi = torch.from_numpy(osel).to(DEV)
        Us = exact(bun["U"].index_select(0, oi)) if rank else np.zeros((len(osel), 0))
        Vs = exact(bun["V"]) if rank else np.zeros((W0.shape[1], 0))
        ss, W0s = exact(bun["s"].index_select(0, oi)), exact(W0.index_select(0, oi))
        got = exact(rec.index_select(0, oi))
        if rank == 0:
            assert np.array_equal(oracle.reconstruct_weight(ss, W0s, Us, Vs), got)   # s * W0 of bf16 values is exact in fp32
        else:
            check_reconstruct(got, ss, W0s, Us, Vs, bf16_out=False, what=f"rebuild rank={rank} {family} layer {layer}")
        # ... and on the whole matrices for the error measure.
        e_ref = oracle.relative_frobenius_error(exact(orig), exact(rec))
        assert abs(e_gpu - e_ref) <= 1e-9 * max(e_ref, 1.0), (e_gpu, e_ref)
        del W0, bun, rec, orig
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Edge cases: ragged shapes, both dtypes, both kernels
# ---------------------------------------------------------------------------

EDGE_SHAPES = [  # (M, out, in, rank)
    (1, 1, 8, 0), (1, 5, 16, 1), (3, 17, 40, 4), (16, 64, 64, 32), (17, 100, 264, 12), (33, 130, 520, 40),
    (64, 64, 64, 8), (5, 48, 8192, 256), (2, 300, 1000, 300), (65, 130, 264, 12), (130, 257, 136, 20),
    (200, 300, 1000, 300), (257, 129, 72, 0), (96, 2048, 512, 64),
    # 16-byte aligned rows: the 256 x 256 kernel with ragged tiles and k tails,
    # the last one shared out by k-tiles over 128 workgroups.
    (300, 520, 200, 24), (513, 1000, 1032, 136), (1100, 700, 4104, 40), (700, 600, 1000, 264),
]


def _rand_case(M, O, I, R, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    mk = lambda *shape, sd=1.0: (torch.randn(*shape, generator=g) * sd).to(dtype).to(DEV)
    x = mk(M, I)
    W0 = mk(O, I, sd=0.02)
    s = (1.0 + 0.1 * torch.rand(O, generator=g)).to(dtype).to(DEV)
    U = mk(O, R, sd=0.01) if R else None
    V = mk(I, R, sd=0.01) if R else None
    return x, s, W0, U, V


def _parity(y, case, what=""):
    """check_forward on a GPU output and the exact values of its inputs (x, s, W0, U, V)."""
    x, s, W0, U, V = case
    R = 0 if U is None else U.shape[1]
    return check_forward(exact(y), exact(x), None if s is None else exact(s), exact(W0),
                         exact(U) if R else np.zeros((W0.shape[0], 0)), exact(V) if R else np.zeros((W0.shape[1], 0)),
                         bf16=x.dtype == torch.bfloat16, what=what)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_edge_shapes(shape, dtype):
    M, O, I, R = shape
    _say(f"edge forward {shape} {dtype}")
    x, s, W0, U, V = _rand_case(M, O, I, R, dtype, seed=sum(shape))
    # Guard bands around the output catch out-of-bounds stores.
    guard = 4096
    buf = torch.full((guard + M * O + guard,), 7.0, dtype=dtype, device=DEV)
    y = buf[guard:guard + M * O].view(M, O)
    tb.linear_forward(x, s, W0, U, V, out=y)
    _parity(y, (x, s, W0, U, V), what=f"edge {shape}")
    assert bool((buf[:guard] == 7.0).all()) and bool((buf[guard + M * O:] == 7.0).all())



# Decode calls with a small V (in * rank * 2 bytes around 512 KiB, rank up to
# 256, up to 32 tokens): ragged column blocks of T, k tails, several k-slices.
SMALL_V_SHAPES = [  # (out, in, rank)
    (6912, 1152, 128), (2048, 2048, 128), (2048, 2056, 128), (1000, 1000, 136), (3000, 520, 256),
    (260, 1032, 200), (130, 40, 8), (4096, 1024, 256), (4096, 1056, 256),
]


@pytest.mark.parametrize("M", [1, 4, 16, 17, 32])
@pytest.mark.parametrize("shape", SMALL_V_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_small_v(shape, M):
    O, I, R = shape
    _say(f"small V {shape} M={M}")
    x, s, W0, U, V = _rand_case(M, O, I, R, torch.bfloat16, seed=O + I + R + M)
    guard = 4096
    buf = torch.full((guard + M * O + guard,), 7.0, dtype=torch.bfloat16, device=DEV)
    y = buf[guard:guard + M * O].view(M, O)
    tb.linear_forward(x, s, W0, U, V, out=y)
    y2 = tb.linear_forward(x, s, W0, U, V)
    torch.cuda.synchronize()
    _parity(y, (x, s, W0, U, V), what=f"small V {shape} M={M}")
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert bool((buf[:guard] == 7.0).all()) and bool((buf[guard + M * O:] == 7.0).all())
    assert tb.workspace_error_word() == 0



# 17-64 tokens: the widest streaming tiles (96 rows with NT = 2, 64 rows with
# NT = 4), ragged row blocks and k tails, both dtypes.
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("M", [17, 32, 33, 48, 64])
@pytest.mark.parametrize("shape", [(8192, 5376, 256), (2100, 1032, 136), (21504, 1152, 128), (700, 4104, 40)],
                         ids=lambda s: "x".join(map(str, s)))
def test_forward_wide_rows_many_tokens(shape, M, dtype):
    O, I, R = shape
    _say(f"wide rows {shape} M={M} {dtype}")
    x, s, W0, U, V = _rand_case(M, O, I, R, dtype, seed=O + M)
    guard = 4096
    buf = torch.full((guard + M * O + guard,), 7.0, dtype=dtype, device=DEV)
    y = buf[guard:guard + M * O].view(M, O)
    tb.linear_forward(x, s, W0, U, V, out=y)
    torch.cuda.synchronize()
    _parity(y, (x, s, W0, U, V), what=f"wide rows {shape} M={M}")
    assert bool((buf[:guard] == 7.0).all()) and bool((buf[guard + M * O:] == 7.0).all())
    assert tb.workspace_error_word() == 0

@pytest.mark.parametrize("M", [1, 16, 32])
def test_forward_group_small_and_large_v(M):
    # One call with a member with a 288 KiB V and one with 2.6 MiB.
    members = [_rand_case(M, 6912, 1152, 128, torch.bfloat16, seed=M),
               _rand_case(M, 6912, 5376, 256, torch.bfloat16, seed=M + 1)]
    ys = tb.linear_forward_group(members)
    torch.cuda.synchronize()
    for mbr, y in zip(members, ys):
        _parity(y, mbr, what=f"group small and large V M={M}")
    assert tb.workspace_error_word() == 0


@pytest.mark.parametrize("shape", [(2048, 4096, 4104, 72), (4096, 4352, 4096, 64)], ids=["split_round", "rounds_and_split"])
def test_forward_split_rounds(shape):
    # 128 tiles of 256 x 256 split into two k-slices; and 272 tiles: one whole
    # round plus 16 remainder tiles split into k-slices.  Sampled outputs.
    M, O, I, R = shape
    _say(f"split rounds {shape}")
    x, s, W0, U, V = _rand_case(M, O, I, R, torch.bfloat16, seed=M + O)
    y = tb.linear_forward(x, s, W0, U, V)
    osel = torch.from_numpy(tile_sample(O, seed=5)).to(DEV)
    tsel = torch.from_numpy(tile_sample(M, seed=6, tile=64)).to(DEV)
    check_forward(exact(y.index_select(0, tsel).index_select(1, osel)), exact(x.index_select(0, tsel)),
                  exact(s.index_select(0, osel)), exact(W0.index_select(0, osel)), exact(U.index_select(0, osel)),
                  exact(V), bf16=True, what=f"split rounds {shape}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", [(17, 40, 4), (130, 264, 12), (64, 512, 256), (33, 72, 0), (1, 8, 3), (1, 8, 8),
                                   (130, 264, 24), (300, 520, 72), (257, 1032, 136), (128, 128, 64), (384, 8, 512),
                                   (130, 264, 200), (300, 520, 256), (257, 1032, 248), (1, 8, 256), (2100, 2104, 256),
                                   (4500, 4104, 64), (4500, 4104, 128), (4500, 4104, 192), (3000, 2056, 8),
                                   (2100, 4104, 136)],
                         ids=lambda s: "x".join(map(str, s)))
def test_reconstruct_edge_shapes(shape, dtype):
    O, I, R = shape
    _, s, W0, U, V = _rand_case(1, O, I, R, dtype, seed=O + I + R)
    Ud = exact(U) if R else np.zeros((O, 0))
    Vd = exact(V) if R else np.zeros((I, 0))
    want = oracle.reconstruct_weight(exact(s), exact(W0), Ud, Vd)
    for out_dtype in (torch.float32, torch.bfloat16):
        rec = tb.reconstruct_weight(s, W0, U, V, out_dtype=out_dtype)
        check_reconstruct(exact(rec), exact(s), exact(W0), Ud, Vd, bf16_out=out_dtype == torch.bfloat16,
                          what=f"rebuild {shape} {dtype} -> {out_dtype}")
        if R == 0 and out_dtype == torch.float32:
            # One multiply: exact for bf16 inputs; for fp32 inputs the float64
            # product (exact) rounded once to fp32.
            ref = want if dtype == torch.bfloat16 else want.astype(np.float32).astype(np.float64)
            assert np.array_equal(ref, exact(rec))


def test_frobenius_closed_forms():
    g = torch.Generator(device="cpu").manual_seed(3)
    for dtype in (torch.float32, torch.bfloat16):
        A = torch.randn(37, 64, generator=g).to(dtype).to(DEV)
        Z = torch.zeros_like(A)
        assert float(tb.rel_frobenius_error(A, A).item()) == 0.0
        assert float(tb.rel_frobenius_error(A, Z).item()) == pytest.approx(1.0, abs=1e-15)
        assert float(tb.rel_frobenius_error(Z, A).item()) == float("inf")
        assert float(tb.rel_frobenius_error(Z, Z).item()) == 0.0
        B = (A.double() * 2).to(dtype)
        assert float(tb.rel_frobenius_error(A, B).item()) == pytest.approx(1.0, rel=1e-12)
        assert float(tb.rel_frobenius_error(B, A).item()) == pytest.approx(0.5, rel=1e-12)
        want = oracle.relative_frobenius_error(exact(A), exact(B * 0.75))
        assert float(tb.rel_frobenius_error(A, (B * 0.75).to(dtype)).item()) == pytest.approx(want, rel=1e-12)
    big = torch.randn(1000, 4104, generator=g).to(DEV)
    other = big + 1e-3 * torch.randn(1000, 4104, generator=g).to(DEV)
    want = oracle.relative_frobenius_error(exact(big), exact(other))
    got = [float(tb.rel_frobenius_error(big, other).item()) for _ in range(3)]
    assert got[0] == pytest.approx(want, rel=1e-12)
    assert got[1] == got[0] and got[2] == got[0]          # fixed summation order
    # The arrival counters in the workspace's last 8 KB are back at zero.
    ws = tb._frob_ws[(torch.cuda.current_device(), torch.cuda.current_stream().cuda_stream)]
    torch.cuda.synchronize()
    assert int(ws[-8192:].count_nonzero().item()) == 0
    # Grids of one to a few workgroups (fewer than the 16 counter groups) and a ragged count.
    for rows in (1, 3, 200, 1037):
        A = torch.randn(rows, 8 * 37, generator=g).to(DEV)
        B = A + 1e-2 * torch.randn(rows, 8 * 37, generator=g).to(DEV)
        want = oracle.relative_frobenius_error(exact(A), exact(B))
        assert float(tb.rel_frobenius_error(A, B).item()) == pytest.approx(want, rel=1e-12)
    torch.cuda.synchronize()
    assert int(ws[-8192:].count_nonzero().item()) == 0


# ---------------------------------------------------------------------------
# Materialise-once mode: the weight rebuilt once, then tb_dense_forward
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", [(1, 2048, 5376), (16, 8192, 5376), (64, 2100, 2104), (65, 136, 264), (300, 1000, 1032),
                                   (4096, 5376, 2048)], ids=lambda s: "x".join(map(str, s)))
def test_dense_forward(shape, dtype):
    M, O, I = shape
    _say(f"dense forward {shape} {dtype}")
    x, _, W, _, _ = _rand_case(M, O, I, 0, dtype, seed=M + O + 3 * I)
    y = tb.dense_forward(x, W)
    tsel = torch.from_numpy(np.arange(M) if M <= 64 else tile_sample(M, seed=M, tile=64)).to(DEV)
    check_forward(exact(y.index_select(0, tsel)), exact(x.index_select(0, tsel)), None, exact(W),
                  np.zeros((O, 0)), np.zeros((I, 0)), bf16=dtype == torch.bfloat16, what=f"dense {shape}")
    # No scale is the unit scale: the rank-0 projection with s = 1, bit for bit.
    y1 = tb.linear_forward(x, torch.ones(O, dtype=dtype, device=DEV), W, None, None)
    y0 = tb.linear_forward(x, None, W, None, None)
    torch.cuda.synchronize()
    ib = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(y.view(ib), y1.view(ib)) and torch.equal(y.view(ib), y0.view(ib))


@pytest.mark.parametrize("M", [1, 16, 64, 300, 4096])
def test_materialise_once_matches_the_fused_projection(M):
    # The 60-layer q projection at rank 256: rebuild W in bf16 once, then y = x . W^T.
    O, I = gen.SHAPES_60["q_proj"]
    _say(f"materialise once M={M}")
    x, s, W0, U, V = _rand_case(M, O, I, 256, torch.bfloat16, seed=11 + M)
    W = tb.reconstruct_weight(s, W0, U, V, out_dtype=torch.bfloat16)
    y_dense = tb.dense_forward(x, W)
    y_fused = tb.linear_forward(x, s, W0, U, V)
    tsel = torch.from_numpy(np.arange(M) if M <= 64 else tile_sample(M, seed=M, tile=64)).to(DEV)
    osel = torch.from_numpy(tile_sample(O, seed=M + 1)).to(DEV)
    xs = exact(x.index_select(0, tsel))
    pick = lambda y: exact(y.index_select(0, tsel).index_select(1, osel))
    bundle = (exact(s.index_select(0, osel)), exact(W0.index_select(0, osel)), exact(U.index_select(0, osel)),
              exact(V))
    check_forward(pick(y_fused), xs, *bundle, bf16=True, what=f"fused M={M}")
    # The materialised weight adds one bf16 rounding per entry: the dense call against the exact projection by
    # the relative error, and element by element against the exact product with the stored weight.
    assert oracle.relative_frobenius_error(oracle.forward(xs, *bundle), pick(y_dense)) <= BF16_TOL
    check_forward(pick(y_dense), xs, None, exact(W.index_select(0, osel)), np.zeros((len(osel), 0)),
                  np.zeros((I, 0)), bf16=True, what=f"materialised M={M}")


# ---------------------------------------------------------------------------
# Reconstruction error without the rebuilt weight (tb_reconstruction_error)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("bundle", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", [(17, 40, 4), (130, 264, 12), (64, 512, 256), (33, 72, 0), (1, 8, 3), (300, 520, 72),
                                   (257, 1032, 136), (129, 136, 256), (2100, 2104, 64), (1000, 1000, 0), (1000, 1000, 200),
                                   (2100, 2104, 256), (4500, 1024, 248), (4500, 4104, 64), (2100, 4104, 136)],
                         ids=lambda s: "x".join(map(str, s)))
def test_reconstruction_error_small(shape, bundle):
    O, I, R = shape
    _, s, W0, U, V = _rand_case(1, O, I, R, bundle, seed=O * 7 + I + R)
    g = torch.Generator(device="cpu").manual_seed(O + R)
    Ud = exact(U) if R else np.zeros((O, 0))
    Vd = exact(V) if R else np.zeros((I, 0))
    rebuilt64 = oracle.reconstruct_weight(exact(s), exact(W0), Ud, Vd)
    for orig_dtype in (torch.float32, torch.bfloat16):
        # An original close to the bundle's weight (error ~ 5%), in the original's own dtype.
        orig = (torch.from_numpy(rebuilt64).float() + 0.05 * rebuilt64.std() * torch.randn(O, I, generator=g)).to(orig_dtype).to(DEV)
        e = float(tb.reconstruction_error(orig, s, W0, U if R else None, V if R else None).item())
        want = oracle.relative_frobenius_error(exact(orig), rebuilt64)
        # The kernel compares with the fp32 rounding of the rebuilt entries: |change| <= 2^-24 |W| per entry.
        assert abs(e - want) <= 1e-6 * max(want, 1e-3), (orig_dtype, e, want)
        if orig_dtype == torch.float32:
            rec = tb.reconstruct_weight(s, W0, U if R else None, V if R else None, out_dtype=torch.float32)
            composed = float(tb.rel_frobenius_error(orig, rec).item())
            assert e == pytest.approx(composed, rel=1e-12, abs=1e-15)
    ws = tb._error_workspace()
    torch.cuda.synchronize()
    assert int(ws[-8192:].count_nonzero().item()) == 0


@pytest.mark.parametrize("rank", [256, 64, 0])
@pytest.mark.parametrize("family", gen.FAMILIES)
def test_reconstruction_error_large(rank, family):
    # 60-layer shapes: equals rebuilding in fp32 and then measuring, for every band's first layer.
    for layer in _parity_layers(6)[::3]:
        band = tb.band_index(60, 6, layer)
        _say(f"reconstruction error rank={rank} {family} layer={layer}")
        W0 = gen.device_w0(torch, 5, family, gen.SHAPES_60, band)
        bun = gen.device_bundle(torch, 5, family, gen.SHAPES_60, layer, band, rank, with_w0=False)
        U, V = (bun["U"], bun["V"]) if rank else (None, None)
        orig = gen.device_original(torch, W0, 5, family, layer)
        fused = [float(tb.reconstruction_error(orig, bun["s"], W0, U, V).item()) for _ in range(2)]
        assert fused[0] == fused[1]                      # fixed summation order
        rec = tb.reconstruct_weight(bun["s"], W0, U, V, out_dtype=torch.float32)
        composed = float(tb.rel_frobenius_error(orig, rec).item())
        assert fused[0] == pytest.approx(composed, rel=1e-12)
        if family == "k_proj":                           # the float64 oracle on the whole matrix
            Ud = exact(U) if rank else np.zeros((W0.shape[0], 0))
            Vd = exact(V) if rank else np.zeros((W0.shape[1], 0))
            want = oracle.relative_frobenius_error(exact(orig), oracle.reconstruct_weight(exact(bun["s"]), exact(W0), Ud, Vd))
            assert abs(fused[0] - want) <= 1e-6 * want
        del W0, bun, rec, orig
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Determinism and workspace state
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("shape", [(16, 6912, 1152, 128), (4, 256, 1152, 128), (2048, 1152, 6912, 128), (1, 2048, 5376, 256)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bitwise_deterministic_and_workspace_clean(shape):
    M, O, I, R = shape
    x, s, W0, U, V = _rand_case(M, O, I, R, torch.bfloat16, seed=99)
    ys = [tb.linear_forward(x, s, W0, U, V).clone() for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(ys[0].view(torch.int16), y.view(torch.int16))
    ws = tb.workspace_for(0)
    ctrl = ws[:16].view(torch.int32).cpu().tolist()
    assert ctrl[2] == 0                      # no bounded wait timed out
    assert stale_control_words(ws[:tb.WORKSPACE_CONTROL_BYTES]) == 0   # every counter back at zero


GROUPS = {  # members (out, in, rank)
    "qkv60": [(8192, 5376, 256), (2048, 5376, 256), (2048, 5376, 256)],
    "gateup26": [(6912, 1152, 128), (6912, 1152, 128)],
    "q_and_o60": [(8192, 5376, 256), (5376, 8192, 256)],  # launch plans differ: one after another
    "ragged": [(17, 40, 4), (33, 72, 0), (130, 264, 12), (100, 264, 300)],
}


@pytest.mark.parametrize("M", [1, 4, 16, 64, 100])
@pytest.mark.parametrize("group", sorted(GROUPS))
def test_forward_group_matches_single_calls(group, M):
    # A grouped call computes each member as its own call would.  In one
    # launch the chip is shared out between the members, so a member's
    # k-slices (and its last bits) may differ from its own call's.  Prefill
    # members that differ in in_dim or rank run one after another, bit for
    # bit as their own calls.
    _say(f"group {group} M={M}")
    shapes = GROUPS[group]
    members = [_rand_case(M, O, I, R, torch.bfloat16, seed=31 * j + M) for j, (O, I, R) in enumerate(shapes)]
    ys = tb.linear_forward_group(members)
    ys2 = tb.linear_forward_group(members)
    singles = [tb.linear_forward(*mbr) for mbr in members]
    torch.cuda.synchronize()
    fused = len({(I, R) for _, I, R in shapes}) == 1
    for mbr, y, y2, y1 in zip(members, ys, ys2, singles):
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
        if M > 64 and not fused:
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16))
        else:
            assert oracle.relative_frobenius_error(exact(y1), exact(y)) <= BF16_TOL
        _parity(y, mbr, what=f"group {group} M={M}")
    assert tb.workspace_error_word() == 0



WIDE_GROUP = [(8192, 5376, 256), (17, 40, 4), (2048, 5376, 256), (130, 264, 12), (6912, 1152, 128), (100, 264, 300),
              (21504, 1152, 0), (33, 72, 0)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("M", [1, 16, 17, 32, 33, 64])
def test_group_stays_inside_its_workspace(M, dtype):
    # Eight members of very different sizes share the chip in one launch; a
    # guard band right after the queried workspace must stay untouched, and
    # every member must match its own call within the tolerance.
    _say(f"workspace guard M={M} {dtype}")
    members = [_rand_case(M, O, I, R, dtype, seed=7 * j + M) for j, (O, I, R) in enumerate(WIDE_GROUP)]
    dims = [(x, s_, W0, U, V, torch.empty((M, W0.shape[0]), dtype=dtype, device=DEV)) for x, s_, W0, U, V in members]
    need = ctypes.c_size_t(0)
    assert tb.lib.tb_linear_forward_group_workspace_size(len(dims), tb.projection_array(dims), M,
                                                          tb._dtype_code(dtype), ctypes.byref(need)) == 0
    guard = 1 << 20
    buf = torch.zeros(need.value + guard, dtype=torch.uint8, device=DEV)
    buf[need.value:] = 0xA5
    ys = tb.linear_forward_group(members, workspace=buf[:need.value])
    singles = [tb.linear_forward(*mbr) for mbr in members]
    torch.cuda.synchronize()
    assert bool((buf[need.value:] == 0xA5).all())
    assert stale_control_words(buf[:tb.WORKSPACE_CONTROL_BYTES]) == 0
    for y, y1 in zip(ys, singles):
        assert oracle.relative_frobenius_error(exact(y1), exact(y)) <= tol_for(dtype)
    for mbr, y in list(zip(members, ys))[1::2]:   # the small members against the oracle
        _parity(y, mbr, what=f"wide group member M={M}")

# Prefill groups whose members share in_dim and rank run as one x . V launch
# and one GEMM launch over every member's tiles: (tokens, members).
FUSED_PREFILL = {
    "qkv26_M2048": (2048, [(1024, 1152, 128), (256, 1152, 128), (256, 1152, 128)]),   # 128 x 128 kernel
    "gateup26_M2048": (2048, [(6912, 1152, 128), (6912, 1152, 128)]),                  # two whole rounds
    "split_across_members": (256, [(2048, 5376, 256), (8192, 5376, 256)]),            # every tile k-split
    "qkv60_M4096": (4096, [(8192, 5376, 256), (2048, 5376, 256), (2048, 5376, 256)]),  # three whole rounds
    "ragged_M300": (300, [(136, 264, 24), (72, 264, 24), (520, 264, 24)]),
    "unaligned_M100": (100, [(40, 40, 4), (17, 40, 4)]),                               # rank 4: x . V by the plain kernel
    "dense_M130": (130, [(264, 520, 0), (136, 520, 0)]),
}


@pytest.mark.parametrize("case", sorted(FUSED_PREFILL))
def test_fused_prefill_group(case):
    # Each member against the oracle (sampled rows and columns of the large
    # ones) and against its own call; a guard band after the queried
    # workspace stays untouched and the control words end clean.
    M, shapes = FUSED_PREFILL[case]
    _say(f"fused prefill group {case}")
    members = [_rand_case(M, O, I, R, torch.bfloat16, seed=11 * j + M) for j, (O, I, R) in enumerate(shapes)]
    dims = [(x, s_, W0, U, V, torch.empty((M, W0.shape[0]), dtype=torch.bfloat16, device=DEV))
            for x, s_, W0, U, V in members]
    need = ctypes.c_size_t(0)
    assert tb.lib.tb_linear_forward_group_workspace_size(len(dims), tb.projection_array(dims), M,
                                                          tb._dtype_code(torch.bfloat16), ctypes.byref(need)) == 0
    guard = 1 << 20
    buf = torch.zeros(need.value + guard, dtype=torch.uint8, device=DEV)
    buf[need.value:] = 0xA5
    ys = tb.linear_forward_group(members, workspace=buf[:need.value])
    ys2 = tb.linear_forward_group(members, workspace=buf[:need.value])
    singles = [tb.linear_forward(*mbr) for mbr in members]
    torch.cuda.synchronize()
    assert bool((buf[need.value:] == 0xA5).all())
    assert stale_control_words(buf[:tb.WORKSPACE_CONTROL_BYTES]) == 0
    for j, (mbr, y, y2, y1) in enumerate(zip(members, ys, ys2, singles)):
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
        assert oracle.relative_frobenius_error(exact(y1), exact(y)) <= BF16_TOL
        x, s_, W0, U, V = mbr
        if M * W0.shape[0] <= 1 << 20:
            _parity(y, mbr, what=f"{case} member {j}")
            continue
        O, R = W0.shape[0], 0 if U is None else U.shape[1]
        osel = torch.from_numpy(tile_sample(O, seed=j + 1)).to(DEV)
        tsel = torch.from_numpy(tile_sample(M, seed=j + 2, tile=64)).to(DEV)
        check_forward(exact(y.index_select(0, tsel).index_select(1, osel)), exact(x.index_select(0, tsel)),
                      exact(s_.index_select(0, osel)), exact(W0.index_select(0, osel)),
                      exact(U.index_select(0, osel)) if R else np.zeros((osel.numel(), 0)),
                      exact(V) if R else np.zeros((W0.shape[1], 0)), bf16=True, what=f"{case} member {j}")


def test_forward_group_fp32_and_clean_workspace():
    members = [_rand_case(8, O, I, R, torch.float32, seed=O) for (O, I, R) in GROUPS["ragged"]]
    ys = tb.linear_forward_group(members)
    for mbr, y in zip(members, ys):
        _parity(y, mbr, what="fp32 group")
    # Every member's control block is left clean.
    ws = tb.workspace_for(tb.WORKSPACE_CONTROL_BYTES)
    torch.cuda.synchronize()
    assert stale_control_words(ws[:tb.WORKSPACE_CONTROL_BYTES]) == 0


def test_stream_ordering_many_calls():
    # Back-to-back calls of different shapes on one stream reuse the
    # workspace; each must see clean control words.
    cases = [(1, 8192, 5376, 256), (16, 2048, 5376, 256), (4, 256, 1152, 128), (64, 1152, 6912, 0), (8, 21504, 5376, 256)]
    data = [_rand_case(*c, torch.bfloat16, seed=i) for i, c in enumerate(cases)]
    outs = [tb.linear_forward(*d) for d in data for _ in range(2)]
    torch.cuda.synchronize()
    for i, d in enumerate(data):
        for y in outs[2 * i: 2 * i + 2]:
            _parity(y, d, what=f"stream order case {i}")
    assert tb.workspace_error_word() == 0


@pytest.mark.parametrize("M", [1, 16, 64, 300])
def test_forward_replays_from_captured_graph(M):
    # A single call and a grouped call captured into a graph: every replay writes the eager results bit for
    # bit, with eager calls of another shape (their own workspace) between the replays.
    _say(f"graph capture M={M}")
    single = _rand_case(M, 2048, 5376, 256, torch.bfloat16, seed=5)
    group = [_rand_case(M, O, I, R, torch.bfloat16, seed=7 + j) for j, (O, I, R) in enumerate(GROUPS["qkv60"])]
    other = _rand_case(8, 256, 1152, 128, torch.bfloat16, seed=3)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):       # eager run on the capture stream sizes its workspace
        want1 = tb.linear_forward(*single).clone()
        wantg = [y.clone() for y in tb.linear_forward_group(group)]
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        y1 = tb.linear_forward(*single)
        yg = tb.linear_forward_group(group)
    torch.cuda.synchronize()
    for rep in range(3):
        tb.linear_forward(*other)
        for y in [y1] + yg:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), want1.view(torch.int16)), rep
        for a, b in zip(yg, wantg):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), rep
    assert tb.workspace_error_word() == 0
    with torch.cuda.stream(side):
        assert tb.workspace_error_word() == 0
    _parity(want1, single, what="graph replay")


# ---------------------------------------------------------------------------
# Timeout path of the bounded wait, forced from the host
# ---------------------------------------------------------------------------


def test_timed_out_wait_poisons_the_workspace_until_cleared():
    # A poll bound of 0 makes the decode streamers' wait for x . V give up at
    # once: every kernel still exits normally, word 2 is set and y is NaN.
    # While word 2 is set every forward call on that workspace writes NaN and
    # leaves the other control words alone; zeroing them makes it usable again.
    dec = _rand_case(16, 2048, 5376, 256, torch.bfloat16, seed=21)
    pre = _rand_case(300, 1000, 1032, 136, torch.bfloat16, seed=22)
    # 128 tiles of 256 x 256, each split into two k-slices that wait for each other.
    spl = _rand_case(2048, 4096, 4104, 72, torch.bfloat16, seed=24)
    grp = [_rand_case(4, O, I, R, torch.bfloat16, seed=23 + j) for j, (O, I, R) in enumerate(GROUPS["qkv60"])]
    need = max(tb.linear_forward_workspace_size(16, 2048, 5376, 256, torch.bfloat16),
               tb.linear_forward_workspace_size(300, 1000, 1032, 136, torch.bfloat16),
               tb.linear_forward_workspace_size(2048, 4096, 4104, 72, torch.bfloat16), 64 << 20)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    ctrl = ws[:tb.WORKSPACE_CONTROL_BYTES]
    err = lambda: int(ws[:16].view(torch.int32)[2].item())
    nan = lambda t: bool(torch.isnan(t.float()).all())
    _say("forced timeout: single call")
    tb.set_wait_polls(0)
    try:
        y = tb.linear_forward(*dec, workspace=ws)
        torch.cuda.synchronize()
    finally:
        tb.set_wait_polls()
    assert err() != 0 and nan(y)

    _say("poisoned workspace: decode, rank 0, dense, prefill and group calls")
    snapshot = ctrl.clone()
    outs = [tb.linear_forward(*dec, workspace=ws), tb.linear_forward(dec[0], dec[1], dec[2], None, None, workspace=ws),
            tb.dense_forward(dec[0], dec[2], workspace=ws), tb.linear_forward(*pre, workspace=ws),
            tb.linear_forward(pre[0], pre[1], pre[2], None, None, workspace=ws), tb.linear_forward(*spl, workspace=ws)]
    outs += tb.linear_forward_group(grp, workspace=ws)
    torch.cuda.synchronize()
    assert all(nan(o) for o in outs)
    assert torch.equal(ctrl, snapshot)

    _say("cleared workspace: correct again and left clean")
    ctrl.zero_()
    y = tb.linear_forward(*dec, workspace=ws)
    yp = tb.linear_forward(*pre, workspace=ws)
    torch.cuda.synchronize()
    _parity(y, dec, what="cleared workspace, decode")
    _parity(yp, pre, what="cleared workspace, prefill")
    assert stale_control_words(ctrl) == 0

    _say("forced timeout: k-split prefill tiles")
    tb.set_wait_polls(0)
    try:
        y = tb.linear_forward(*spl, workspace=ws)
        torch.cuda.synchronize()
    finally:
        tb.set_wait_polls()
    assert err() != 0 and nan(y)
    ctrl.zero_()
    y = tb.linear_forward(*spl, workspace=ws)
    torch.cuda.synchronize()
    x, s_, W0, U, V = spl
    osel = torch.from_numpy(tile_sample(W0.shape[0], seed=3)).to(DEV)
    tsel = torch.from_numpy(tile_sample(x.shape[0], seed=4, tile=64)).to(DEV)
    check_forward(exact(y.index_select(0, tsel).index_select(1, osel)), exact(x.index_select(0, tsel)),
                  exact(s_.index_select(0, osel)), exact(W0.index_select(0, osel)), exact(U.index_select(0, osel)),
                  exact(V), bf16=True, what="cleared workspace, k-split prefill")
    assert stale_control_words(ctrl) == 0

    _say("forced timeout: grouped launch")
    tb.set_wait_polls(0)
    try:
        ys = tb.linear_forward_group(grp, workspace=ws)
        torch.cuda.synchronize()
    finally:
        tb.set_wait_polls()
    assert err() != 0 and all(nan(y) for y in ys)
    ctrl.zero_()
    ys = tb.linear_forward_group(grp, workspace=ws)
    torch.cuda.synchronize()
    for mbr, y in zip(grp, ys):
        _parity(y, mbr, what="cleared workspace, group")
    assert stale_control_words(ctrl) == 0
