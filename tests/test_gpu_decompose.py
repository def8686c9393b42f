"""GPU parity of the analytic decomposition (tb_shared_block, tb_row_scale,
tb_lowrank_factors) through the C ABI against the float64 oracle.

The shared block is compared bit for bit with the oracle's float64 mean
rounded to fp32 (same summation order); the row scale to a few fp32 ulps.
The low-rank factors follow the randomized SVD on the same probe as
oracle.randomized_factors: U V^T is compared where it is well defined (a
spectral gap at the rank, or a residual of exact low rank), the
approximation error otherwise, and the exact truncated SVD when the probe
spans the whole input space.
"""

import numpy as np
import pytest
import torch

import oracle
from rank_factored_linear_amd import inputs as gen
from parity_util import check_forward, exact, f32_to_device

pytestmark = pytest.mark.gpu

tb = pytest.importorskip("rank_factored_linear_amd.binding")
DEV = "cuda"


def _say(*a):
    print(*a, flush=True)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(a), 1e-300))


def _residual64(w, W0, s):
    """The residual the GPU factors, from the GPU's own fp32 W0 and s (float64)."""
    return exact(w) - exact(s)[:, None] * exact(W0)


def _with_spectrum(O, I, sigma, rng):
    P = np.linalg.qr(rng.normal(size=(O, len(sigma))))[0]
    Q = np.linalg.qr(rng.normal(size=(I, len(sigma))))[0]
    return (P * sigma[None, :]) @ Q.T


def _band(n, O, I, dtype, seed, lowrank=None):
    """n layers a_l B + low-rank_l + noise (the tiny stack's recipe at another size)."""
    r = np.random.default_rng(seed)
    B = r.normal(0.0, 0.02, (O, I))
    ws = []
    for l in range(n):
        a = r.uniform(0.95, 1.05)
        w = a * B + r.normal(0.0, 1e-3, (O, I))
        if lowrank:
            w = w + r.normal(0.0, 0.05, (O, lowrank)) @ r.normal(0.0, 0.05, (I, lowrank)).T
        ws.append(torch.from_numpy(w.astype(np.float32)).to(dtype).to(DEV))
    return ws


# ---------------------------------------------------------------------------
# Shared block and row scale
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("n,shape", [(1, (17, 40)), (2, (130, 264)), (3, (1000, 1032)), (7, (257, 129)),
                                     (15, (2048, 1152))], ids=lambda v: str(v))
def test_shared_block_bit_exact(n, shape, dtype):
    ws = _band(n, *shape, dtype, seed=n + shape[0])
    W0 = tb.shared_block(ws)
    want = oracle.shared_block([exact(w) for w in ws]).astype(np.float32)
    assert np.array_equal(W0.cpu().numpy(), want)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("shape", [(17, 40), (130, 264), (2048, 5376), (3, 100000)], ids=lambda v: "x".join(map(str, v)))
def test_row_scale(shape, dtype):
    ws = _band(3, *shape, dtype, seed=shape[0])
    W0 = tb.shared_block(ws)
    W0[1].zero_()                          # a zero row of W0: s = 0 (minimum-norm reading)
    for w in ws:
        s = tb.row_scale(w, W0).cpu().numpy().astype(np.float64)
        want = oracle.row_scale(exact(w), exact(W0))
        assert s[1] == 0.0 and want[1] == 0.0
        # float64 sums in another order, rounded once to fp32: within two fp32 ulps.
        assert np.all(np.abs(s - want) <= 2 * 2.0 ** -23 * np.abs(want) + 1e-30)


def test_passthrough_band_gives_zero_delta():
    # G = L: W0 = W exactly, s = 1 exactly, the residual is zero and so are U and V.
    w = _band(1, 300, 520, torch.float32, seed=4)[0]
    W0 = tb.shared_block([w])
    assert torch.equal(W0, w)
    s = tb.row_scale(w, W0)
    assert torch.equal(s, torch.ones_like(s))
    omega = torch.randn((520, 24), generator=torch.Generator().manual_seed(1)).to(DEV)
    U, V = tb.lowrank_factors(w, W0, s, 16, omega, 2)
    torch.cuda.synchronize()
    assert int(U.count_nonzero()) == 0 and int(V.count_nonzero()) == 0


# ---------------------------------------------------------------------------
# Low-rank factors
# ---------------------------------------------------------------------------


def _case(O, I, seed, sigma=None, dtype=torch.float32):
    """A band of two layers; with sigma, layer 0's residual gets that spectrum added on top."""
    r = np.random.default_rng(seed)
    ws = _band(2, O, I, torch.float32, seed=seed)
    if sigma is not None:
        extra = _with_spectrum(O, I, sigma, r)
        ws[0] = (ws[0].double() + torch.from_numpy(extra).to(DEV)).float()
    ws = [w.to(dtype) for w in ws]
    W0 = tb.shared_block(ws)
    s = tb.row_scale(ws[0], W0)
    return ws[0], W0, s


@pytest.mark.parametrize("O,I,rank", [(64, 40, 8), (300, 130, 24), (130, 300, 130), (600, 400, 40), (340, 700, 20)], ids=lambda v: str(v))
def test_full_probe_is_the_exact_truncated_svd(O, I, rank):
    # k = min(out, in): the probe spans the input space, so the result is the
    # Eckart-Young optimum, here with a gap after the rank.
    sigma = np.concatenate([np.linspace(2.0, 1.0, rank), 0.05 * np.linspace(1.0, 0.1, min(O, I) - rank)])
    w, W0, s = _case(O, I, seed=O + rank, sigma=sigma)
    k = min(O, I)
    omega = torch.randn((I, k), generator=torch.Generator().manual_seed(O)).to(DEV)
    U, V = tb.lowrank_factors(w, W0, s, rank, omega, 0)
    E = _residual64(w, W0, s)
    Ue, Ve = oracle.truncated_factors(E, rank)
    assert _rel(Ue @ Ve.T, exact(U) @ exact(V).T) <= 1e-5
    # Columns by decreasing singular value, U absorbing them.
    assert np.allclose(np.linalg.norm(exact(U), axis=0), np.linalg.norm(Ue, axis=0), rtol=1e-5)


@pytest.mark.parametrize("q", [0, 2])
def test_exact_low_rank_residual_is_recovered(q):
    # With the scale the weight was built from, the residual has rank 12 <= k
    # (up to the fp32 rounding of the weight): the probe spans its range at any q.
    O, I = 1000, 1032
    r = np.random.default_rng(8)
    W0 = torch.from_numpy(r.normal(0, 0.02, (O, I)).astype(np.float32)).to(DEV)
    s_true = r.uniform(0.9, 1.1, O)
    low = r.normal(0, 0.05, (O, 12)) @ r.normal(0, 0.05, (I, 12)).T
    s = torch.from_numpy(s_true.astype(np.float32)).to(DEV)
    w = torch.from_numpy((exact(s)[:, None] * exact(W0) + low).astype(np.float32)).to(DEV)
    omega = torch.randn((I, 32), generator=torch.Generator().manual_seed(9)).to(DEV)
    U, V = tb.lowrank_factors(w, W0, s, 16, omega, q)
    E = _residual64(w, W0, s)
    assert _rel(E, exact(U) @ exact(V).T) <= 2e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("O,I,rank,p,q", [(256, 512, 16, 16, 2), (1000, 1032, 64, 16, 2), (1032, 1000, 64, 8, 0),
                                          (2048, 5376, 256, 16, 2)], ids=lambda v: str(v))
def test_matches_the_oracle_randomized_svd_with_a_gap(O, I, rank, p, q, dtype):
    # A spectral gap after the rank: U V^T is well defined and must match the
    # oracle's randomized SVD on the same probe.
    n = min(O, I)
    sigma = np.concatenate([np.linspace(1.0, 0.5, rank), 0.02 * np.linspace(1.0, 0.01, n - rank)])
    w, W0, s = _case(O, I, seed=O + I + rank, sigma=sigma, dtype=dtype)
    _say(f"randomized gap {O}x{I} r={rank} k={rank + p} q={q} {dtype}")
    omega = torch.randn((I, rank + p), generator=torch.Generator().manual_seed(rank)).to(DEV)
    U, V = tb.lowrank_factors(w, W0, s, rank, omega, q)
    E = _residual64(w, W0, s)
    Uo, Vo = oracle.randomized_factors(E, rank, exact(omega), q)
    assert _rel(Uo @ Vo.T, exact(U) @ exact(V).T) <= 1e-4
    err_gpu, err_orc = _rel(E, exact(U) @ exact(V).T), _rel(E, Uo @ Vo.T)
    assert abs(err_gpu - err_orc) <= 1e-5 * max(err_orc, 1e-3)


@pytest.mark.parametrize("O,I,rank,q", [(256, 512, 16, 2), (1152, 6912, 128, 2), (5376, 2048, 64, 1)],
                         ids=lambda v: str(v))
def test_matches_the_oracle_error_without_a_gap(O, I, rank, q):
    # Weight-like residuals (a band of noisy scaled blocks plus a low-rank
    # part): the rank-r subspace is not sharply defined, but the error each
    # reaches on the same probe is, to first order.
    ws = _band(3, O, I, torch.float32, seed=O + rank, lowrank=rank // 2)
    W0 = tb.shared_block(ws)
    s = tb.row_scale(ws[1], W0)
    k = rank + 16
    omega = torch.randn((I, k), generator=torch.Generator().manual_seed(O)).to(DEV)
    _say(f"randomized no gap {O}x{I} r={rank} q={q}")
    U, V = tb.lowrank_factors(ws[1], W0, s, rank, omega, q)
    E = _residual64(ws[1], W0, s)
    Uo, Vo = oracle.randomized_factors(E, rank, exact(omega), q)
    err_gpu, err_orc = _rel(E, exact(U) @ exact(V).T), _rel(E, Uo @ Vo.T)
    assert abs(err_gpu - err_orc) <= 1e-4 * err_orc, (err_gpu, err_orc)
    # Never below the Eckart-Young optimum.
    opt = np.sqrt(np.sum(np.linalg.svd(E, compute_uv=False)[rank:] ** 2)) / np.linalg.norm(E)
    assert err_gpu >= opt * (1 - 1e-5)


def test_decompose_tiny_stack_matches_the_oracle_pipeline():
    weights, _ = gen.tiny_stack()
    wd = [f32_to_device(w) for w in weights]
    rank, p, q, seed = 16, 16, 2, 7
    bun = tb.decompose(wd, 2, rank, oversampling=p, power_iters=q, seed=seed)
    g = torch.Generator(device="cpu").manual_seed(seed)
    for l in range(gen.TINY_LAYERS):
        band = bun["band"][l]
        assert band == gen.TINY_LAYER_BAND[l]
        members = [exact(wd[j]) for j in range(gen.TINY_LAYERS) if gen.TINY_LAYER_BAND[j] == band]
        assert np.array_equal(bun["W0"][band].cpu().numpy(), oracle.shared_block(members).astype(np.float32))
        s_want = oracle.row_scale(exact(wd[l]), exact(bun["W0"][band]))
        assert np.all(np.abs(exact(bun["s"][l]) - s_want) <= 2 * 2.0 ** -23 * np.abs(s_want))
        omega = torch.randn((gen.TINY_IN, rank + p), generator=g, dtype=torch.float32)
        E = _residual64(wd[l], bun["W0"][band], bun["s"][l])
        Uo, Vo = oracle.randomized_factors(E, rank, exact(omega), q)
        got = exact(bun["U"][l]) @ exact(bun["V"][l]).T
        assert abs(_rel(E, got) - _rel(E, Uo @ Vo.T)) <= 1e-4 * _rel(E, Uo @ Vo.T)
        # The rebuilt weight: W0, s, U, V through the forward path's reconstruction.
        rec = tb.reconstruct_weight(bun["s"][l], bun["W0"][band], bun["U"][l], bun["V"][l])
        e_gpu = oracle.relative_frobenius_error(exact(wd[l]), exact(rec))
        e_orc = oracle.relative_frobenius_error(exact(wd[l]), oracle.reconstruct_weight(
            exact(bun["s"][l]), exact(bun["W0"][band]), Uo, Vo))
        assert abs(e_gpu - e_orc) <= 1e-3 * e_orc


def test_batch_matches_single_calls():
    # A band of eight layers in one batched call against one call per layer
    # (a gap after the rank: U V^T is well defined).
    ws = _band(8, 1000, 1032, torch.bfloat16, seed=21, lowrank=16)
    W0 = tb.shared_block(ws)
    S = torch.stack([tb.row_scale(w, W0) for w in ws])
    om = torch.randn((8, 1032, 32), generator=torch.Generator().manual_seed(5)).to(DEV)
    U, V = tb.lowrank_factors_batch(ws, W0, S, 16, om, 2)
    for l in range(8):
        u1, v1 = tb.lowrank_factors(ws[l], W0, S[l].contiguous(), 16, om[l].contiguous(), 2)
        assert _rel(exact(u1) @ exact(v1).T, exact(U[l]) @ exact(V[l]).T) <= 1e-5, l


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("n,O,I,rank", [(3, 130, 264, 8), (5, 1000, 1032, 64), (2, 300, 520, 0)], ids=lambda v: str(v))
def test_refine_shared_block(n, O, I, rank, dtype):
    r = np.random.default_rng(n + O + rank)
    ws = [torch.from_numpy(r.normal(0, 0.02, (O, I)).astype(np.float32)).to(dtype).to(DEV) for _ in range(n)]
    ss = [torch.from_numpy(r.uniform(0.5, 1.5, O).astype(np.float32)).to(DEV) for _ in range(n)]
    for t in ss:
        t[3] = 0.0                       # a row with all-zero scales keeps its previous value
    Us = [torch.from_numpy(r.normal(0, 0.01, (O, rank)).astype(np.float32)).to(DEV) for _ in range(n)]
    Vs = [torch.from_numpy(r.normal(0, 0.01, (I, rank)).astype(np.float32)).to(DEV) for _ in range(n)]
    prev = torch.from_numpy(r.normal(0, 0.02, (O, I)).astype(np.float32)).to(DEV)
    W0 = tb.refine_shared_block(ws, ss, Us if rank else [None] * n, Vs if rank else [None] * n, prev)
    want = oracle.refine_shared_block([exact(w) for w in ws], [exact(t) for t in ss],
                                      [exact(u) for u in Us], [exact(v) for v in Vs], exact(prev))
    assert torch.equal(W0[3], prev[3])
    assert _rel(want, exact(W0)) <= 1e-6


def test_als_tiny_stack_matches_the_oracle():
    # With a probe as wide as the input (k = min(out, in)) the randomized SVD is
    # the exact one, so two ALS rounds follow the oracle's exact-SVD ALS.
    weights, _ = gen.tiny_stack()
    wd = [f32_to_device(w) for w in weights]
    got = tb.als_decompose(wd, 2, 16, 2, oversampling=gen.TINY_OUT)
    want = oracle.als_decompose(weights, 2, 16, 2)
    for l in range(gen.TINY_LAYERS):
        band = got["band"][l]
        assert _rel(want["W0"][band], exact(got["W0"][band])) <= 1e-5
        rec = tb.reconstruct_weight(got["s"][l], got["W0"][band], got["U"][l], got["V"][l])
        e_gpu = oracle.relative_frobenius_error(weights[l], exact(rec))
        e_orc = oracle.relative_frobenius_error(weights[l], oracle.reconstruct_weight(
            want["s"][l], want["W0"][band], want["U"][l], want["V"][l]))
        assert abs(e_gpu - e_orc) <= 1e-4 * e_orc, (l, e_gpu, e_orc)


@pytest.mark.parametrize("tie", ["all", "attn"])
def test_decompose_model_tie_families(tie):
    # A 4-layer model with all seven families ("The theta bundle", Projection
    # families).  Families that share go through decompose() with the seed it
    # is given; under tie_families="attn" the MLP layers stay dense and their
    # forward is x . W^T against the oracle.
    r = np.random.default_rng(3)
    L, G, rank = 4, 2, 8
    shapes = {"q_proj": (96, 64), "k_proj": (32, 64), "v_proj": (32, 64), "o_proj": (64, 96),
              "gate_proj": (160, 64), "up_proj": (160, 64), "down_proj": (64, 160)}
    model = {}
    for fam, (O, I) in shapes.items():
        B = r.normal(0.0, 0.02, (O, I))
        model[fam] = [torch.from_numpy((r.uniform(0.9, 1.1) * B + r.normal(0.0, 1e-3, (O, I))).astype(np.float32))
                      .to(torch.bfloat16).to(DEV) for _ in range(L)]
    got = tb.decompose_model(model, G, rank, tie_families=tie, seed=5)
    want = oracle.decompose_model({f: [exact(w) for w in ws] for f, ws in model.items()}, G, 0, tie_families=tie)
    x = torch.from_numpy(r.normal(size=(8, 160)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    for j, (fam, ws) in enumerate(model.items()):
        bun = got[fam]
        if tie == "attn" and fam in tb.MLP_FAMILIES:
            assert bun["band"] == list(range(L))
            for l in range(L):
                assert bun["W0"][l] is ws[l] and bun["s"][l] is None and bun["U"][l] is None
                xi = x[:, : ws[l].shape[1]].contiguous()
                y = tb.linear_forward(xi, None, bun["W0"][l], None, None)
                wb = want[fam]
                check_forward(exact(y), exact(xi), wb["s"][l], wb["W0"][l], wb["U"][l], wb["V"][l], True,
                              f"{fam} layer {l}")
            continue
        again = tb.decompose(ws, G, rank, seed=5 + j)       # the same call, deterministic kernels
        for l in range(L):
            band = bun["band"][l]
            assert band == want[fam]["band"][l]
            assert np.array_equal(bun["W0"][band].cpu().numpy(), want[fam]["W0"][band].astype(np.float32))
            for k in ("s", "U", "V"):
                assert torch.equal(bun[k][l], again[k][l]), (fam, l, k)
