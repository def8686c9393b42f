"""Helpers for GPU-vs-oracle parity tests: exact value transfer and tolerances."""

import numpy as np
import torch

import oracle

# Relative Frobenius error of the GPU projection against the float64 oracle:
# 5e-3 for bf16 inputs with fp32 accumulation, 1e-5 for fp32 inputs.
BF16_TOL = 5e-3
F32_TOL = 1e-5


def bits_to_device(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def f32_to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def exact(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bf16 or fp32 tensor (any device)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    if t.dtype == torch.float64:
        return t.numpy().copy()
    raise TypeError(t.dtype)


def tol_for(dtype) -> float:
    return BF16_TOL if dtype == torch.bfloat16 else F32_TOL


def sample_rows(n: int, k: int, seed: int) -> np.ndarray:
    """k distinct indices in [0, n) including the first and last (sorted)."""
    if n <= k:
        return np.arange(n)
    r = np.random.default_rng(seed)
    pick = set(r.choice(n, size=k - 2, replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(pick))


# ---------------------------------------------------------------------------
# Element-wise and per-tile parity
# ---------------------------------------------------------------------------
#
# Every output element is held to a worst-case bound derived from the
# arithmetic the kernels do, in addition to the relative Frobenius error over
# the whole output and over each tile of 16 output features:
#   * fp32 sums of n products: |computed - exact| <= gamma(n) * sum |terms|,
#     gamma(n) = n u / (1 - n u) with u = 2^-23 (this covers any summation
#     order, k-slice partials combined in any order, and rounding toward zero
#     as well as to nearest);
#   * the rounding of the output to bf16: 2^-8 of the value (8 significant
#     bits, round to nearest even); fp32 output adds no rounding beyond the
#     sums above;
#   * for bf16, T = x V is rounded to bf16 before it meets U: 2^-8 of each
#     |T_j| times |U_oj|, i.e. 2^-8 D with D = |x V| |U|^T (the error of the
#     fp32 sum that T is rounded from is in the gamma term).
# The magnitude of every sum comes from the oracle's own forward applied to
# |x|, |s|, |W0|, |U|, |V|: F = |s| (|x| |W0|^T) + (|x| |V|) |U|^T.
U_SUM = 2.0 ** -23
BF16_U = 2.0 ** -8
TILE = 16


def gamma(n: int) -> float:
    return n * U_SUM / (1.0 - n * U_SUM)


def _tile_errors(want: np.ndarray, got: np.ndarray, axis_len: int, width: int = TILE) -> np.ndarray:
    """Relative Frobenius error of each block of `width` consecutive columns (all rows)."""
    errs = []
    for c0 in range(0, axis_len, width):
        errs.append(oracle.relative_frobenius_error(want[:, c0:c0 + width], got[:, c0:c0 + width]))
    return np.array(errs)


def _check_elements(want, got, bound, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = np.abs(got - want)
    bad = diff > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        rows = [(tuple(int(v) for v in i), float(want[tuple(i)]), float(got[tuple(i)]), float(bound[tuple(i)]))
                for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside the bound, e.g. (index, want, got, bound) "
                             f"{rows}")


def check_forward(got: np.ndarray, x, s, W0, U, V, bf16: bool, what: str = "") -> float:
    """Parity of a projection's output `got` [m, out] (exact float64 values of the GPU result) with the oracle on
    the exact inputs (float64 arrays; s None means unit scale, U/V [*, 0] for rank 0): the global relative
    Frobenius error, the same per tile of 16 output features (10x the global tolerance for fp32, where the
    tolerance is far below the bf16 rounding that makes a per-tile bound rigorous), and every element within
    its worst-case bound.  Returns the global error."""
    x, W0, U, V = (np.asarray(a, dtype=np.float64) for a in (x, W0, U, V))
    s = np.ones(W0.shape[0]) if s is None else np.asarray(s, dtype=np.float64)
    want = oracle.forward(x, s, W0, U, V)
    tol = BF16_TOL if bf16 else F32_TOL
    err = oracle.relative_frobenius_error(want, got)
    assert err <= tol, f"{what}: relative error {err:.3e} > {tol:.0e}"
    tiles = _tile_errors(want, got, want.shape[1])
    tile_tol = tol if bf16 else 10 * tol
    worst = int(np.argmax(tiles))
    assert tiles[worst] <= tile_tol, f"{what}: tile of columns {worst * TILE}.. has relative error {tiles[worst]:.3e}"
    aU = np.abs(U)
    F = oracle.forward(np.abs(x), np.abs(s), np.abs(W0), aU, np.abs(V))
    g = gamma(W0.shape[1] + U.shape[1] + 64)
    if bf16:
        D = np.abs(x @ V) @ aU.T
        bound = BF16_U * np.abs(want) + 1.01 * (g * F + BF16_U * D) + 1e-30
    else:
        bound = 1.01 * g * F + 1e-30
    _check_elements(want, got, bound, what)
    return err


def check_reconstruct(got: np.ndarray, s, W0, U, V, bf16_out: bool, what: str = "") -> float:
    """Parity of a rebuilt weight (rows of it) with the oracle's diag(s) W0 + U V^T: global and per-tile
    relative Frobenius error and the element-wise bound (fp32 sums of the rank products and the scaled
    block; the bf16 rounding of the output when it is bf16)."""
    s, W0, U, V = (np.asarray(a, dtype=np.float64) for a in (s, W0, U, V))
    want = oracle.reconstruct_weight(s, W0, U, V)
    tol = BF16_TOL if bf16_out else F32_TOL
    err = oracle.relative_frobenius_error(want, got)
    assert err <= tol, f"{what}: relative error {err:.3e} > {tol:.0e}"
    rows = _tile_errors(want.T, got.T, want.shape[0], width=1)     # each row of the weight on its own
    row_tol = tol if bf16_out else 10 * tol
    assert rows.max() <= row_tol, f"{what}: row {int(np.argmax(rows))} has relative error {rows.max():.3e}"
    F = oracle.reconstruct_weight(np.abs(s), np.abs(W0), np.abs(U), np.abs(V))
    g = gamma(U.shape[1] + 4)
    bound = (BF16_U * np.abs(want) if bf16_out else 0.0) + 1.01 * g * F + 1e-30
    _check_elements(want, got, bound, what)
    return err


def tile_sample(n: int, seed: int, tile: int = TILE) -> np.ndarray:
    """One index in every block of `tile` consecutive indices (a random offset per block), plus the first and
    the last index: every tile of an output the kernels write is looked at."""
    r = np.random.default_rng(seed)
    pick = {min(b + int(r.integers(tile)), n - 1) for b in range(0, n, tile)} | {0, n - 1}
    return np.array(sorted(pick))


# ---------------------------------------------------------------------------
# Forward workspace control words
# ---------------------------------------------------------------------------
# The library's control block layout (64 KiB per group member): word 2 is the
# sticky error flag, word 3 the parity of the decode x . V exchange, words
# 1088 .. 15295 the two exchange halves; every other word (the arrival, done
# and finish counters) must be zero between calls.
CTRL_BLOCK_WORDS = 16384
CTRL_PARITY_WORD = 3
CTRL_EXCHANGE = (64 + 1024, CTRL_BLOCK_WORDS - 17 * 64)


def stale_control_words(ctrl_bytes) -> int:
    """Number of control words that should be zero between calls and are not (the parity word and the
    exchange halves, which legitimately carry the last call's state, are left out)."""
    import torch
    words = ctrl_bytes.view(torch.int32).view(-1, CTRL_BLOCK_WORDS).clone()
    words[:, CTRL_PARITY_WORD] = 0
    words[:, CTRL_EXCHANGE[0]:CTRL_EXCHANGE[1]] = 0
    return int(words.count_nonzero().item())
