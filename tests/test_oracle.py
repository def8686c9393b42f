"""Pins for the float64 oracle, independent of the oracle's own formulas.

Each check below compares the oracle with something other than itself: the
hand-worked examples under tests/golden (each cites the page it follows), a
library routine that solves the same problem another way (numpy.array_split,
numpy.linalg.lstsq), closed forms, invariants, and brute-force loops on tiny
inputs.  The checks are written as functions of the implementation so that the
mutation tests at the bottom can show that a plausible mistake in the oracle
(a misplaced remainder, a swapped ratio, a transposed factor, singular values
on the wrong side, the wrong norm in the denominator) fails at least one pin.
"""

import json
import os
import types

import numpy as np
import pytest

import oracle
from oracle import theta_bundle as tb
from conftest import GOLDEN, BAND_FIXTURES, read_band_fixture

from rank_factored_linear_amd import inputs


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# Pin checks, parameterised by implementation
# ---------------------------------------------------------------------------


def check_band_map(impl) -> None:
    # Golden fixtures (hand-written from the pages and the workload statements).
    for name in BAND_FIXTURES:
        L, G, want = read_band_fixture(name)
        assert impl.band_map(L, G) == want, name
        assert [impl.band_index(L, G, l) for l in range(L)] == want, name
    # A library routine that splits a sequence the same way.
    for L in range(1, 129):
        for G in range(1, L + 1):
            parts = np.array_split(np.arange(L), G)
            want = [b for b, p in enumerate(parts) for _ in p]
            assert impl.band_map(L, G) == want, (L, G)
            assert impl.band_sizes(L, G) == [len(p) for p in parts], (L, G)


def check_forward(impl) -> None:
    g = _golden("forward_hand_example.json")
    args = [np.array(g[k], dtype=np.float64) for k in ("x", "s", "W0", "U", "V")]
    assert np.array_equal(impl.forward(*args), np.array(g["y"], dtype=np.float64))
    # Brute force: materialise every weight entry, then every output, by loops.
    r = np.random.default_rng(5)
    M, O, I, R = 3, 5, 4, 2
    x, s, W0 = r.normal(size=(M, I)), r.normal(size=O), r.normal(size=(O, I))
    U, V = r.normal(size=(O, R)), r.normal(size=(I, R))
    want = np.zeros((M, O))
    for m in range(M):
        for o in range(O):
            acc = 0.0
            for i in range(I):
                w = s[o] * W0[o, i]
                for j in range(R):
                    w += U[o, j] * V[i, j]
                acc += x[m, i] * w
            want[m, o] = acc
    got = impl.forward(x, s, W0, U, V)
    assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def check_reconstruct(impl) -> None:
    g = _golden("forward_hand_example.json")
    got = impl.reconstruct_weight(*[np.array(g[k], dtype=np.float64) for k in ("s", "W0", "U", "V")])
    assert np.array_equal(got, np.array(g["weight"], dtype=np.float64))
    r = np.random.default_rng(6)
    O, I, R = 4, 6, 3
    s, W0, U, V = r.normal(size=O), r.normal(size=(O, I)), r.normal(size=(O, R)), r.normal(size=(I, R))
    want = np.zeros((O, I))
    for o in range(O):
        for i in range(I):
            want[o, i] = s[o] * W0[o, i] + sum(U[o, j] * V[i, j] for j in range(R))
    assert np.max(np.abs(impl.reconstruct_weight(s, W0, U, V) - want)) <= 1e-13


def check_frobenius(impl) -> None:
    g = _golden("frobenius_hand_example.json")
    assert impl.relative_frobenius_error(np.array(g["original"], float), np.array(g["reconstructed"], float)) == pytest.approx(g["error"], abs=1e-15)
    A = np.random.default_rng(7).normal(size=(5, 7))
    assert impl.relative_frobenius_error(A, A) == 0.0
    assert impl.relative_frobenius_error(A, np.zeros_like(A)) == pytest.approx(1.0, abs=1e-15)
    for eps in (1e-3, -0.25, 2.0):
        assert impl.relative_frobenius_error(A, (1 + eps) * A) == pytest.approx(abs(eps), rel=1e-12)
    # The original's norm is the denominator: err(A, 2A) = 1, err(2A, A) = 1/2.
    assert impl.relative_frobenius_error(A, 2 * A) == pytest.approx(1.0, rel=1e-14)
    assert impl.relative_frobenius_error(2 * A, A) == pytest.approx(0.5, rel=1e-14)
    assert impl.relative_frobenius_error(3.5 * A, 3.5 * (A + 0.1)) == pytest.approx(
        impl.relative_frobenius_error(A, A + 0.1), rel=1e-12)


def check_row_scale(impl) -> None:
    r = np.random.default_rng(8)
    O, I = 6, 9
    W, W0 = r.normal(size=(O, I)), r.normal(size=(O, I))
    s = impl.row_scale(W, W0)
    # Each s[o] is the least-squares solution of W0[o] * s = W[o] (a library solver).
    for o in range(O):
        sol = np.linalg.lstsq(W0[o][:, None], W[o], rcond=None)[0][0]
        assert s[o] == pytest.approx(sol, rel=1e-12, abs=1e-14)
        # Normal equations: the residual row is orthogonal to the W0 row.
        assert abs(np.dot(W[o] - s[o] * W0[o], W0[o])) <= 1e-12 * np.dot(W0[o], W0[o])
    # An exact multiple is recovered: W = c * W0 row by row.
    c = r.uniform(0.5, 2.0, size=O)
    assert np.allclose(impl.row_scale(c[:, None] * W0, W0), c, rtol=1e-14, atol=0)


def check_truncated_factors(impl) -> None:
    r = np.random.default_rng(9)
    O, I = 12, 8
    P = np.linalg.qr(r.normal(size=(O, I)))[0]            # O x I orthonormal columns
    Q = np.linalg.qr(r.normal(size=(I, I)))[0]            # I x I orthogonal
    sigma = np.array([9.0, 7.0, 5.0, 3.0, 2.0, 1.0, 0.5, 0.25])
    Rm = P @ np.diag(sigma) @ Q.T                           # known spectrum
    for k in range(0, I + 1):
        U, V = impl.truncated_factors(Rm, k)
        assert U.shape == (O, k) and V.shape == (I, k)
        best = P[:, :k] @ np.diag(sigma[:k]) @ Q[:, :k].T   # Eckart-Young optimum
        assert np.max(np.abs(U @ V.T - best)) <= 1e-12
        # U absorbs the singular values: V has orthonormal columns, U = R V.
        assert np.allclose(V.T @ V, np.eye(k), atol=1e-12)
        assert np.allclose(U, Rm @ V, atol=1e-12)
        assert np.sum((Rm - U @ V.T) ** 2) == pytest.approx(np.sum(sigma[k:] ** 2), abs=1e-11)


def check_randomized_factors(impl) -> None:
    r = np.random.default_rng(11)
    # 1. A probe as wide as the input space covers the column space: the exact
    #    truncated SVD (Eckart-Young optimum of a known spectrum) at every rank.
    O, I = 12, 8
    P = np.linalg.qr(r.normal(size=(O, I)))[0]
    Q = np.linalg.qr(r.normal(size=(I, I)))[0]
    sigma = np.array([9.0, 7.0, 5.0, 3.0, 2.0, 1.0, 0.5, 0.25])
    Rm = P @ np.diag(sigma) @ Q.T
    om = r.normal(size=(I, I))
    for q in (0, 1):
        for k in range(0, I + 1):
            U, V = impl.randomized_factors(Rm, k, om, q)
            assert U.shape == (O, k) and V.shape == (I, k)
            best = P[:, :k] @ np.diag(sigma[:k]) @ Q[:, :k].T
            assert np.max(np.abs(U @ V.T - best)) <= 1e-12
            assert np.allclose(np.linalg.norm(U, axis=0), sigma[:k], rtol=1e-12, atol=0)
    # 2. A residual of exact rank k = 16 over eight decades: the k-column probe
    #    spans its range, so every rank <= 16 is exact, with or without power
    #    iterations (without oversampling, or without re-orthonormalising the
    #    power iterations, the weak directions are lost).
    O, I, k = 60, 40, 16
    P = np.linalg.qr(r.normal(size=(O, k)))[0]
    Q = np.linalg.qr(r.normal(size=(I, k)))[0]
    sigma = 10.0 ** (-np.arange(k) / 2)
    Rm = P @ np.diag(sigma) @ Q.T
    om = r.normal(size=(I, k))
    for q in (0, 3):
        for rank in (1, 8, 12, 16):
            U, V = impl.randomized_factors(Rm, rank, om, q)
            best = P[:, :rank] @ np.diag(sigma[:rank]) @ Q[:, :rank].T
            assert np.max(np.abs(U @ V.T - best)) <= 1e-12, (q, rank)
    # 3. Halko et al. (2009), Theorem 10.5: E||A - Q Q^T A||_F^2 <= (1 + r/(p-1)) tail^2
    #    for target rank r and oversampling p; cutting Q Q^T A to rank r adds at
    #    most tail^2 (orthogonal pieces; B = Q^T A has singular values <= A's).
    #    Averaged over 20 probes, with 20% for the sample mean.  Every draw is at
    #    least the Eckart-Young optimum.
    O, I, rank, p = 200, 150, 10, 6
    P = np.linalg.qr(r.normal(size=(O, I)))[0]
    Q = np.linalg.qr(r.normal(size=(I, I)))[0]
    sigma = 1.0 / np.arange(1, I + 1)
    Rm = P @ np.diag(sigma) @ Q.T
    tail2 = float(np.sum(sigma[rank:] ** 2))
    errs = []
    for d in range(20):
        U, V = impl.randomized_factors(Rm, rank, np.random.default_rng(100 + d).normal(size=(I, rank + p)), 0)
        e2 = float(np.sum((Rm - U @ V.T) ** 2))
        assert e2 >= tail2 * (1 - 1e-12)
        errs.append(e2)
        # 5. U absorbs the singular values: V orthonormal, U's columns orthogonal
        #    with non-increasing norms.
        assert np.allclose(V.T @ V, np.eye(rank), atol=1e-12)
        G = U.T @ U
        assert np.max(np.abs(G - np.diag(np.diag(G)))) <= 1e-12 * G[0, 0]
        assert np.all(np.diff(np.diag(G)) <= 1e-15)
    assert np.mean(errs) <= 1.2 * (2 + rank / (p - 1)) * tail2
    # 4. Power iterations close the gap to the optimum.
    for d in range(5):
        U, V = impl.randomized_factors(Rm, rank, np.random.default_rng(200 + d).normal(size=(I, rank + p)), 6)
        assert np.sqrt(np.sum((Rm - U @ V.T) ** 2)) <= 1.0001 * np.sqrt(tail2)


def check_refine_shared_block(impl) -> None:
    r = np.random.default_rng(12)
    O, I, R, n = 5, 7, 2, 3
    Ws = [r.normal(size=(O, I)) for _ in range(n)]
    ss = [r.uniform(0.5, 1.5, size=O) for _ in range(n)]
    Us = [r.normal(size=(O, R)) for _ in range(n)]
    Vs = [r.normal(size=(I, R)) for _ in range(n)]
    prev = r.normal(size=(O, I))
    ss[1][2] = 0.0
    W0 = impl.refine_shared_block(Ws, ss, Us, Vs, prev)
    for o in range(O):
        # Normal equations of min_x sum_l |(W_l - U_l V_l^T)[o] - s_l[o] x|^2 ...
        g = sum(ss[l][o] * (Ws[l] - ss[l][o] * W0 - Us[l] @ Vs[l].T)[o] for l in range(n))
        assert np.max(np.abs(g)) <= 1e-12
        # ... and a library least-squares solve of the stacked system.
        A = np.vstack([ss[l][o] * np.eye(I) for l in range(n)])
        b = np.concatenate([(Ws[l] - Us[l] @ Vs[l].T)[o] for l in range(n)])
        assert np.allclose(W0[o], np.linalg.lstsq(A, b, rcond=None)[0], rtol=1e-12, atol=1e-13)
    # A row whose scales are all zero keeps its previous value.
    zs = [s.copy() for s in ss]
    for s in zs:
        s[4] = 0.0
    assert np.array_equal(impl.refine_shared_block(Ws, zs, Us, Vs, prev)[4], prev[4])
    # Consistent data W_l = diag(s_l) B + U_l V_l^T: the block is recovered exactly.
    B = r.normal(size=(O, I))
    Wc = [np.diag(ss[l]) @ B + Us[l] @ Vs[l].T for l in range(n)]
    assert np.max(np.abs(impl.refine_shared_block(Wc, ss, Us, Vs, prev) - B)) <= 1e-12
    # ALS with no rounds is the analytic decomposition; passthrough is a fixed point.
    w, _ = inputs.tiny_stack()
    a0, d0 = impl.als_decompose(w, 2, 4, 0), impl.decompose(w, 2, 4)
    assert all(np.array_equal(x, y) for x, y in zip(a0["W0"], d0["W0"]))
    a2 = impl.als_decompose(w, 4, 0, 2)
    for l in range(4):
        assert np.max(np.abs(a2["W0"][a2["band"][l]] - w[l])) <= 1e-15 and np.allclose(a2["s"][l], 1.0, atol=1e-15)


def _als_stack():
    """Four 12 x 9 layers in two bands: a per-band block under per-row scales, a rank-3 term and noise."""
    r = np.random.default_rng(13)
    O, I = 12, 9
    B = [r.normal(size=(O, I)) for _ in range(2)]
    return [r.uniform(0.6, 1.4, size=O)[:, None] * B[l // 2] + r.normal(size=(O, 3)) @ r.normal(size=(3, I))
            + 0.3 * r.normal(size=(O, I)) for l in range(4)]


def check_als_decompose(impl) -> None:
    # Invariants of the bundle returned after one and two rounds, each checked
    # with numbers the oracle does not compute itself.
    Ws, G, rank = _als_stack(), 2, 2
    for iters in (1, 2):
        prev = impl.als_decompose(Ws, G, rank, iters - 1)
        cur = impl.als_decompose(Ws, G, rank, iters)
        assert cur["band"] == [0, 0, 1, 1]
        for l, w in enumerate(Ws):
            w0 = cur["W0"][cur["band"][l]]
            s, U, V = cur["s"][l], cur["U"][l], cur["V"][l]
            # (a) s is the row-wise least-squares fit against the RETURNED block:
            #     the residual row is orthogonal to the block row.
            for o in range(w.shape[0]):
                assert abs(np.dot(w[o] - s[o] * w0[o], w0[o])) <= 1e-11 * np.dot(w0[o], w0[o]), (iters, l, o)
            # (b) U V^T is the Eckart-Young cut of the RETURNED residual: its error
            #     is the sum of the residual's smallest squared singular values,
            #     taken here from the eigenvalues of the Gram matrix (another
            #     library routine than the oracle's SVD); V is orthonormal and U = E V.
            E = w - s[:, None] * w0
            lam = np.sort(np.linalg.eigvalsh(E.T @ E))[::-1]
            tail = float(np.sum(np.clip(lam[rank:], 0.0, None)))
            assert np.sum((E - U @ V.T) ** 2) == pytest.approx(tail, rel=1e-9, abs=1e-12), (iters, l)
            assert np.allclose(V.T @ V, np.eye(rank), atol=1e-12) and np.allclose(U, E @ V, atol=1e-11)
        # (c) Each returned block solves the block least-squares problem for the
        #     PREVIOUS round's scales and factors: the normal equations
        #     sum_l s_l[o] (W_l - s_l[o] W0 - U_l V_l^T)[o] = 0 hold row by row.
        for b in range(G):
            members = [l for l in range(len(Ws)) if cur["band"][l] == b]
            w0 = cur["W0"][b]
            for o in range(w0.shape[0]):
                g = sum(prev["s"][l][o] * (Ws[l] - prev["s"][l][o] * w0 - prev["U"][l] @ prev["V"][l].T)[o]
                        for l in members)
                assert np.max(np.abs(g)) <= 1e-11, (iters, b, o)
        # A round changes the block (the pins above are not met trivially).
        assert max(np.max(np.abs(a - c)) for a, c in zip(prev["W0"], cur["W0"])) > 1e-3


def check_decompose(impl) -> None:
    r = np.random.default_rng(10)
    # Passthrough (G = L): W0 = W, s = 1 exactly, delta 0 and error exactly 0.
    Ws = [r.normal(0, 0.02, size=(6, 10)) for _ in range(3)]
    for rank in (0, 2):
        bun = impl.decompose(Ws, 3, rank)
        for l in range(3):
            assert np.array_equal(bun["W0"][bun["band"][l]], Ws[l])
            assert np.array_equal(bun["s"][l], np.ones(6))
            assert np.array_equal(bun["U"][l] @ bun["V"][l].T, np.zeros((6, 10)))
        assert impl.decomposition_error(Ws, bun) == [0.0, 0.0, 0.0]
    # Hand-worked band means for the 26-layer G=4 map.
    g = _golden("band_mean_26_g4.json")
    Ws = [float(l) * np.ones((2, 3)) for l in range(26)]
    bun = impl.decompose(Ws, 4, 0)
    assert [float(w[0, 0]) for w in bun["W0"]] == g["band_means"]
    for l in range(26):
        mean_b = g["band_means"][bun["band"][l]]
        assert np.allclose(bun["s"][l], l / mean_b, rtol=1e-15, atol=0)
    assert max(impl.decomposition_error(Ws, bun)) <= 1e-15
    # A pure-scale band W_l = c_l B: s = c_l / mean(c), zero error at rank 0.
    B = r.normal(size=(5, 7))
    cs = [0.7, 1.1, 1.3]
    bun = impl.decompose([c * B for c in cs], 1, 0)
    for l, c in enumerate(cs):
        assert np.allclose(bun["s"][l], c / np.mean(cs), rtol=1e-13, atol=0)
    assert max(impl.decomposition_error([c * B for c in cs], bun)) <= 1e-14


def check_decompose_model(impl) -> None:
    # "The theta bundle", Projection families: with tie_families="attn" only
    # q/k/v/o share a block; the MLP stays dense.  Attention families are
    # pure-scale bands W_l = c_l B (closed form at rank 0: W0 = mean(c) B,
    # s_l = c_l / mean(c)); MLP families are unstructured.
    r = np.random.default_rng(11)
    L, G = 4, 2
    shapes = {"q_proj": (6, 8), "k_proj": (4, 8), "v_proj": (4, 8), "o_proj": (8, 6),
              "gate_proj": (10, 8), "up_proj": (10, 8), "down_proj": (8, 10)}
    cs = [0.8, 1.2, 0.9, 1.1]
    model = {}
    for fam, (O, I) in shapes.items():
        if fam in ("q_proj", "k_proj", "v_proj", "o_proj"):
            B = r.normal(size=(O, I))
            model[fam] = [c * B for c in cs]
        else:
            model[fam] = [r.normal(size=(O, I)) for _ in range(L)]
    bands = [b for b, p in enumerate(np.array_split(np.arange(L), G)) for _ in p]
    x = r.normal(size=(3, 10))
    for tie in ("all", "attn"):
        got = impl.decompose_model(model, G, 0, tie_families=tie)
        assert sorted(got) == sorted(shapes), tie
        for fam, ws in model.items():
            bun = got[fam]
            dense = tie == "attn" and fam in ("gate_proj", "up_proj", "down_proj")
            for l, w in enumerate(ws):
                rebuilt = impl.reconstruct_weight(bun["s"][l], bun["W0"][bun["band"][l]], bun["U"][l], bun["V"][l])
                if dense:
                    # A plain dense layer: its own weight, unscaled, no delta.
                    assert bun["band"][l] == l and bun["U"][l].shape[1] == 0
                    assert np.array_equal(rebuilt, w), (tie, fam, l)
                    xi = x[:, : w.shape[1]]
                    assert np.array_equal(impl.forward(xi, bun["s"][l], bun["W0"][l], bun["U"][l], bun["V"][l]),
                                          xi @ w.T), (tie, fam, l)
                    continue
                members = [j for j in range(L) if bands[j] == bands[l]]
                assert bun["band"][l] == bands[l], (tie, fam, l)
                assert np.allclose(bun["W0"][bands[l]], np.mean([ws[j] for j in members], axis=0),
                                   rtol=1e-14, atol=1e-15), (tie, fam, l)
                if fam in ("q_proj", "k_proj", "v_proj", "o_proj"):
                    mc = np.mean([cs[j] for j in members])
                    assert np.allclose(bun["s"][l], cs[l] / mc, rtol=1e-13, atol=0), (tie, fam, l)
                    assert np.max(np.abs(rebuilt - w)) <= 1e-13 * np.max(np.abs(w)), (tie, fam, l)
                else:
                    # A shared block of unstructured layers cannot be exact at rank 0.
                    assert impl.relative_frobenius_error(w, rebuilt) > 0.1, (tie, fam, l)
    for bad in ("mlp", "none", ""):
        with pytest.raises(ValueError):
            impl.decompose_model(model, G, 0, tie_families=bad)
    with pytest.raises(ValueError):
        impl.decompose_model({"lm_head": model["q_proj"]}, G, 0)


ALL_CHECKS = [check_band_map, check_forward, check_reconstruct, check_frobenius,
              check_row_scale, check_truncated_factors, check_randomized_factors, check_refine_shared_block,
              check_als_decompose, check_decompose, check_decompose_model]


# ---------------------------------------------------------------------------
# The oracle passes every pin
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pinned(check):
    check(tb)


def test_band_map_properties_bruteforce():
    for L in range(1, 129):
        for G in range(1, L + 1):
            bm = oracle.band_map(L, G)
            sizes = oracle.band_sizes(L, G)
            assert len(bm) == L and bm[0] == 0 and bm[-1] == G - 1
            assert all(b2 - b1 in (0, 1) for b1, b2 in zip(bm, bm[1:]))     # contiguous
            assert max(sizes) - min(sizes) <= 1                            # near-equal
            assert sizes == sorted(sizes, reverse=True)                    # earlier take the rest
            assert sum(sizes) == L
    assert oracle.band_map(26, 1) == [0] * 26
    assert oracle.band_map(26, 26) == list(range(26))


def test_band_invalid_arguments():
    for L, G in ((0, 1), (5, 0), (5, 6), (5, -1)):
        with pytest.raises(ValueError):
            oracle.band_map(L, G)
    with pytest.raises(ValueError):
        oracle.band_index(5, 2, 5)
    with pytest.raises(ValueError):
        oracle.band_index(5, 2, -1)


def test_bf16_decoding():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 0.0, -0.0, (2 - 2.0 ** -7) * 2.0 ** 127, 2.0 ** -133, 3.140625]
    got = oracle.bf16_bits_to_f64(bits)
    assert list(got) == want
    assert np.signbit(got[4])


def test_passthrough_forward_bit_identical():
    # At passthrough (s = 1, rank 0) the projection is the plain layer x W^T,
    # and the float64 factored form reproduces np.matmul exactly.
    r = np.random.default_rng(11)
    x, W = r.normal(size=(8, 64)), r.normal(0, 0.02, size=(48, 64))
    y = oracle.forward(x, np.ones(48), W, np.zeros((48, 0)), np.zeros((64, 0)))
    assert np.array_equal(y, x @ W.T)


def test_factored_equals_materialised():
    r = np.random.default_rng(12)
    x, s, W0 = r.normal(size=(7, 40)), r.uniform(0.9, 1.1, 30), r.normal(0, 0.02, (30, 40))
    U, V = r.normal(0, 0.01, (30, 5)), r.normal(0, 0.01, (40, 5))
    a = oracle.forward(x, s, W0, U, V)
    b = oracle.forward_dense(x, oracle.reconstruct_weight(s, W0, U, V))
    assert oracle.relative_frobenius_error(b, a) <= 1e-13
    # Linearity in x.
    x2 = r.normal(size=x.shape)
    lin = oracle.forward(2.0 * x - 3.0 * x2, s, W0, U, V)
    assert np.allclose(lin, 2.0 * a - 3.0 * oracle.forward(x2, s, W0, U, V), rtol=0, atol=1e-12)


def test_row_scale_zero_row_reading():
    W0 = np.array([[0.0, 0.0], [1.0, 2.0]])
    W = np.array([[3.0, 4.0], [2.0, 4.0]])
    assert list(oracle.row_scale(W, W0)) == [0.0, 2.0]


def test_frobenius_zero_cases():
    Z = np.zeros((3, 3))
    assert oracle.relative_frobenius_error(Z, Z) == 0.0
    assert oracle.relative_frobenius_error(Z, np.eye(3)) == float("inf")


def test_mean_error_unweighted():
    assert oracle.mean_error([0.0, 0.5, 1.0]) == 0.5
    with pytest.raises(ValueError):
        oracle.mean_error([])


def test_truncated_factors_rank_bounds():
    R = np.ones((3, 5))
    with pytest.raises(ValueError):
        oracle.truncated_factors(R, 4)
    with pytest.raises(ValueError):
        oracle.truncated_factors(R, -1)


def test_tiny_stack_full_rank_zero_error():
    # A full-rank delta absorbs the whole residual: zero error on tiny inputs.
    weights, _ = inputs.tiny_stack()
    bun = oracle.decompose(weights, 2, min(weights[0].shape))
    assert max(oracle.decomposition_error(weights, bun)) <= 1e-12
    assert bun["band"] == list(inputs.TINY_LAYER_BAND)


def test_tiny_stack_rank16_error_is_small_but_nonzero():
    # Gross-bug detector only: the residual is band noise plus the rank-8 term
    # and the N(0, 1e-3) noise; a rank-16 delta absorbs the structured part.
    weights, _ = inputs.tiny_stack()
    bun = oracle.decompose(weights, 2, 16)
    err = oracle.mean_error(oracle.decomposition_error(weights, bun))
    assert 1e-3 < err < 0.2
    err0 = oracle.mean_error(oracle.decomposition_error(weights, oracle.decompose(weights, 2, 0)))
    assert err0 > err


def test_byte_accounting_of_gemma3_projections():
    # "Quality", section "Reconstruction error": 1778.91 MB of fp32 projection
    # weights.  With MLP width 4096 (the page's up_proj 4096x1152) the seven
    # families over 26 layers give exactly that; the measured 26-layer stack
    # uses width 6912 instead.
    shapes = dict(inputs.SHAPES_26)
    for f in ("gate_proj", "up_proj"):
        shapes[f] = (4096, 1152)
    shapes["down_proj"] = (1152, 4096)
    total = 26 * sum(o * i for o, i in shapes.values()) * 4
    assert total == 1_778_909_184
    assert round(total / 1e6, 2) == 1778.91


def test_oracle_imports_nothing_from_the_product():
    here = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
    for fn in os.listdir(here):
        if fn.endswith(".py"):
            text = open(os.path.join(here, fn)).read()
            assert "rank_factored_linear_amd" not in text.replace("``rank_factored_linear_amd``", "")


# ---------------------------------------------------------------------------
# Mutation tests: planted mistakes in copies of the oracle must fail a pin
# ---------------------------------------------------------------------------


def _mutant(**overrides):
    m = types.SimpleNamespace(**{k: getattr(tb, k) for k in dir(tb) if not k.startswith("__")})
    for k, v in overrides.items():
        setattr(m, k, v)
    return m


def _remainder_last_sizes(L, G):
    q, rem = divmod(L, G)
    return [q] * (G - rem) + [q + 1] * rem


def _remainder_last_map(L, G):
    return [b for b, n in enumerate(_remainder_last_sizes(L, G)) for _ in range(n)]


def _floor_map(L, G):
    return [l * G // L for l in range(L)]


def _swapped_row_scale(weight, W0):
    return np.array([np.dot(W0[o], W0[o]) / np.dot(weight[o], W0[o]) for o in range(W0.shape[0])])


def _input_dot_row_scale(weight, W0):  # normalises by the weight row instead of the W0 row
    return np.array([np.dot(weight[o], W0[o]) / np.dot(weight[o], weight[o]) for o in range(W0.shape[0])])


def _v_absorbs(residual, rank):
    P, sg, Qt = np.linalg.svd(residual, full_matrices=False)
    return P[:, :rank], Qt[:rank, :].T * sg[:rank][None, :]


def _wrong_transposed_forward(x, s, W0, U, V):   # delta uses (x V) without U^T's transpose
    return (x @ W0.T) * s[None, :] + (x @ V) @ U.T[:, ::-1][::-1, :]


def _scale_after_delta(x, s, W0, U, V):
    return ((x @ W0.T) + (x @ V) @ U.T) * s[None, :]


def _recon_transposed(s, W0, U, V):
    return (W0.T * s).T + U @ V.T[:, ::-1]


def _frob_wrong_den(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b)) if np.linalg.norm(a - b) else 0.0


def _frob_squared(a, b):
    num = np.sum((a - b) ** 2)
    return float(num / np.sum(a * a)) if num else 0.0


def _rand_v_absorbs(residual, rank, omega, power_iters):
    U, V = tb.randomized_factors(residual, rank, omega, power_iters)
    norms = np.linalg.norm(U, axis=0)
    return U / np.where(norms > 0, norms, 1.0)[None, :], V * norms[None, :]


def _rand_sigma_dropped(residual, rank, omega, power_iters):
    U, V = tb.randomized_factors(residual, rank, omega, power_iters)
    norms = np.linalg.norm(U, axis=0)
    return U / np.where(norms > 0, norms, 1.0)[None, :], V


def _rand_no_oversampling(residual, rank, omega, power_iters):
    return tb.randomized_factors(residual, rank, omega[:, :rank], power_iters)


def _rand_plain_powers(residual, rank, omega, power_iters):
    Y = residual @ omega
    for _ in range(power_iters):
        Y = residual @ (residual.T @ Y)
    Q = np.linalg.qr(Y)[0]
    P, sg, Qt = np.linalg.svd(Q.T @ residual, full_matrices=False)
    return Q @ (P[:, :rank] * sg[:rank][None, :]), Qt[:rank].T


def _refine_by_sum_of_scales(weights, s_list, U_list, V_list, W0_prev):
    num = sum(sl[:, None] * (w - U @ V.T) for w, sl, U, V in zip(weights, s_list, U_list, V_list))
    den = sum(s_list)
    out = np.array(W0_prev, dtype=np.float64)
    rows = den != 0
    out[rows] = num[rows] / den[rows][:, None]
    return out


def _refine_without_delta(weights, s_list, U_list, V_list, W0_prev):
    return tb.refine_shared_block(weights, s_list, [0 * U for U in U_list], V_list, W0_prev)


def _als_variant(weights, num_bands, rank, iters, *, s_from_old_block=False, keep_factors=False,
                 block_from_first_round=False, refit_before_block=False):
    """als_decompose with one planted mistake (each keyword plants one)."""
    weights = [np.asarray(w, dtype=np.float64) for w in weights]
    bun = tb.decompose(weights, num_bands, rank)
    first = {k: list(bun[k]) for k in ("s", "U", "V")}
    bands = bun["band"]

    def refit_layers(blocks_for_s, blocks_for_delta):
        for l, w in enumerate(weights):
            s = tb.row_scale(w, blocks_for_s[bands[l]])
            if not keep_factors:
                bun["U"][l], bun["V"][l] = tb.truncated_factors(w - np.diag(s) @ blocks_for_delta[bands[l]], rank)
            bun["s"][l] = s

    for _ in range(iters):
        if refit_before_block:
            refit_layers(bun["W0"], bun["W0"])
        old = list(bun["W0"])
        src = first if block_from_first_round else bun
        for b in range(num_bands):
            members = [l for l in range(len(weights)) if bands[l] == b]
            bun["W0"][b] = tb.refine_shared_block([weights[l] for l in members], [src["s"][l] for l in members],
                                                  [src["U"][l] for l in members], [src["V"][l] for l in members],
                                                  bun["W0"][b])
        if not refit_before_block:
            refit_layers(old if s_from_old_block else bun["W0"], bun["W0"])
    return bun


def _als(**plant):
    return lambda weights, num_bands, rank, iters: _als_variant(weights, num_bands, rank, iters, **plant)


def _model_ties_everything(weights_by_family, num_bands, rank, tie_families="all"):
    if tie_families not in ("all", "attn"):
        raise ValueError(tie_families)
    return tb.decompose_model(weights_by_family, num_bands, rank, "all")


def _model_ties_the_mlp(weights_by_family, num_bands, rank, tie_families="all"):
    if tie_families not in ("all", "attn"):
        raise ValueError(tie_families)
    if tie_families == "all":
        return tb.decompose_model(weights_by_family, num_bands, rank, "all")
    swapped = {("gate_proj" if f == "q_proj" else "q_proj" if f == "gate_proj" else f): w
               for f, w in weights_by_family.items()}
    got = tb.decompose_model(swapped, num_bands, rank, "attn")
    return {("gate_proj" if f == "q_proj" else "q_proj" if f == "gate_proj" else f): b for f, b in got.items()}


MUTANTS = [
    ("tie_families='attn' decomposes the MLP too", check_decompose_model,
     dict(decompose_model=_model_ties_everything)),
    ("tie_families='attn' keeps q dense and shares gate", check_decompose_model,
     dict(decompose_model=_model_ties_the_mlp)),
    ("ALS: s refit against the previous block", check_als_decompose, dict(als_decompose=_als(s_from_old_block=True))),
    ("ALS: U, V not refit", check_als_decompose, dict(als_decompose=_als(keep_factors=True))),
    ("ALS: block refit from the first round's factors", check_als_decompose,
     dict(als_decompose=_als(block_from_first_round=True))),
    ("ALS: layers refit before the block", check_als_decompose, dict(als_decompose=_als(refit_before_block=True))),
    ("band remainder to the last bands", check_band_map,
     dict(band_sizes=_remainder_last_sizes, band_map=_remainder_last_map,
          band_index=lambda L, G, l: _remainder_last_map(L, G)[l])),
    ("band by floor(l*G/L)", check_band_map,
     dict(band_map=_floor_map, band_index=lambda L, G, l: _floor_map(L, G)[l])),
    ("s ratio swapped", check_row_scale, dict(row_scale=_swapped_row_scale)),
    ("s normalised by the weight row", check_row_scale, dict(row_scale=_input_dot_row_scale)),
    ("V absorbs the singular values", check_truncated_factors, dict(truncated_factors=_v_absorbs)),
    ("ALS: block normalised by the sum of scales", check_refine_shared_block,
     dict(refine_shared_block=_refine_by_sum_of_scales)),
    ("ALS: delta left out of the block update", check_refine_shared_block,
     dict(refine_shared_block=_refine_without_delta)),
    ("randomized: V absorbs the singular values", check_randomized_factors, dict(randomized_factors=_rand_v_absorbs)),
    ("randomized: singular values dropped", check_randomized_factors, dict(randomized_factors=_rand_sigma_dropped)),
    ("randomized: probe without oversampling", check_randomized_factors,
     dict(randomized_factors=_rand_no_oversampling)),
    ("randomized: power iterations not re-orthonormalised", check_randomized_factors,
     dict(randomized_factors=_rand_plain_powers)),
    ("delta factor reversed", check_forward, dict(forward=_wrong_transposed_forward)),
    ("scale applied to the delta too", check_forward, dict(forward=_scale_after_delta)),
    ("reconstruct with a permuted V", check_reconstruct, dict(reconstruct_weight=_recon_transposed)),
    ("Frobenius normalised by the rebuilt weight", check_frobenius, dict(relative_frobenius_error=_frob_wrong_den)),
    ("Frobenius without the square root", check_frobenius, dict(relative_frobenius_error=_frob_squared)),
]


@pytest.mark.parametrize("name,check,overrides", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, check, overrides):
    with pytest.raises(AssertionError):
        check(_mutant(**overrides))


def test_als_variant_without_a_plant_passes():
    # The harness that plants the ALS mistakes computes the oracle's rounds
    # when nothing is planted, so each caught mutant differs by its plant only.
    check_als_decompose(_mutant(als_decompose=_als()))
    w = _als_stack()
    a, b = tb.als_decompose(w, 2, 2, 2), _als()(w, 2, 2, 2)
    assert all(np.array_equal(p, q) for p, q in zip(a["W0"], b["W0"]))
