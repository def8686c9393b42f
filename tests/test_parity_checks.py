"""The element-wise parity check used by the GPU tests, exercised on the CPU.

A float32 simulation of what the kernels compute (fp32 sums, T = x V rounded
to bf16, one bf16 rounding of y) must pass parity_util.check_forward, and the
same output with a plausible kernel bug planted in one place must fail it:
the rank-r delta dropped in one tile of 16 output features (a few percent of
|y| there, small against the whole output), or one element off by 5% of the
output's RMS.
"""

import numpy as np
import pytest

from parity_util import check_forward, check_reconstruct, tile_sample


def _bf16(a):
    """Round float32 values to bfloat16 (nearest, ties to even), returned as float64."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _case(M, O, I, R, seed):
    r = np.random.default_rng(seed)
    x = _bf16(r.normal(size=(M, I)))
    W0 = _bf16(r.normal(0, 0.02, size=(O, I)))
    s = _bf16(r.uniform(0.9, 1.1, size=O))
    U = _bf16(r.normal(0, 0.01, size=(O, R)))
    V = _bf16(r.normal(0, 0.01, size=(I, R)))
    return x, s, W0, U, V


def _kernel_like(x, s, W0, U, V, drop_tail_rows=None):
    f = lambda a: np.asarray(a, dtype=np.float32)
    A = f(x) @ f(W0).T * f(s)[None, :]
    T = _bf16(f(x) @ f(V))
    D = f(T) @ f(U).T
    if drop_tail_rows is not None:
        D[:, drop_tail_rows] = 0.0
    return _bf16(A + D)


@pytest.mark.parametrize("M", [1, 16])
def test_check_accepts_kernel_arithmetic_and_rejects_a_dropped_tail(M):
    x, s, W0, U, V = _case(M, 2048, 1024, 128, seed=M)
    check_forward(_kernel_like(x, s, W0, U, V), x, s, W0, U, V, bf16=True, what="fp32 simulation")
    bad = _kernel_like(x, s, W0, U, V, drop_tail_rows=slice(1024, 1040))
    with pytest.raises(AssertionError):
        check_forward(bad, x, s, W0, U, V, bf16=True)
    one = _kernel_like(x, s, W0, U, V)
    one[0, 700] += 0.05 * np.sqrt(np.mean(one ** 2))
    with pytest.raises(AssertionError):
        check_forward(one, x, s, W0, U, V, bf16=True)


def test_check_fp32_and_rebuild():
    r = np.random.default_rng(3)
    x = r.normal(size=(8, 512)).astype(np.float32)
    s = r.uniform(0.9, 1.1, 256).astype(np.float32)
    W0 = r.normal(0, 0.02, (256, 512)).astype(np.float32)
    U = r.normal(0, 0.01, (256, 16)).astype(np.float32)
    V = r.normal(0, 0.01, (512, 16)).astype(np.float32)
    y = (x @ W0.T) * s[None, :] + (x @ V) @ U.T
    check_forward(y.astype(np.float64), x, s, W0, U, V, bf16=False)
    y[:, 32:48] -= ((x @ V) @ U.T)[:, 32:48]
    with pytest.raises(AssertionError):
        check_forward(y.astype(np.float64), x, s, W0, U, V, bf16=False)
    W = (s[:, None] * W0 + U @ V.T).astype(np.float32)
    check_reconstruct(W.astype(np.float64), s, W0, U, V, bf16_out=False)
    W[100] = s[100] * W0[100]
    with pytest.raises(AssertionError):
        check_reconstruct(W.astype(np.float64), s, W0, U, V, bf16_out=False)


def test_tile_sample_covers_every_tile():
    for n in (1, 15, 16, 17, 1000, 21504):
        idx = tile_sample(n, seed=n)
        assert idx[0] == 0 and idx[-1] == n - 1 and np.all(np.diff(idx) > 0)
        assert set(range(0, n, 16)) <= {i // 16 * 16 for i in idx}
