"""tb_linear_forward_no_alloc: the forward call whose workspace is the
library's static device scratch, against tb_linear_forward (the same
computation with a caller-provided workspace) and the float64 oracle.

The scratch is shared by every call on the GPU and keeps the last call's
contents, so each test makes two calls in a row, the second smaller than the
first.
"""

import numpy as np
import pytest
import torch

from parity_util import check_forward, exact

pytestmark = pytest.mark.gpu

tb = pytest.importorskip("rank_factored_linear_amd.binding")
DEV = "cuda"


def _case(M, O, I, R, dtype, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    mk = lambda *shape, sd=1.0: (torch.randn(*shape, generator=g) * sd).to(dtype).to(DEV)
    x = mk(M, I)
    W0 = mk(O, I, sd=0.02)
    s = (1.0 + 0.1 * torch.rand(O, generator=g)).to(dtype).to(DEV)
    U = mk(O, R, sd=0.01) if R else None
    V = mk(I, R, sd=0.01) if R else None
    return x, s, W0, U, V


def _parity(y, case, what):
    x, s, W0, U, V = case
    R = 0 if U is None else U.shape[1]
    check_forward(exact(y), exact(x), exact(s), exact(W0), exact(U) if R else np.zeros((W0.shape[0], 0)),
                  exact(V) if R else np.zeros((W0.shape[1], 0)), bf16=x.dtype == torch.bfloat16, what=what)


def _same_bits(a, b):
    ib = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(ib), b.view(ib))


CALL_PAIRS = {
    # decode: a 60-layer q projection at 16 tokens, then a 26-layer one at 4 tokens
    "decode": [(16, 8192, 5376, 256, torch.bfloat16), (4, 1024, 1152, 128, torch.bfloat16)],
    # prefill: the 60-layer k projection at 2048 tokens (~82 MiB of scratch), then a ragged 300-token one
    "prefill": [(2048, 2048, 5376, 256, torch.bfloat16), (300, 1000, 1032, 136, torch.bfloat16)],
    # fp32 decode, then a rank-0 one
    "fp32": [(17, 700, 4104, 40, torch.float32), (3, 130, 264, 0, torch.float32)],
}


@pytest.mark.parametrize("pair", sorted(CALL_PAIRS))
def test_no_alloc_matches_the_workspace_entry_point(pair):
    for j, (M, O, I, R, dtype) in enumerate(CALL_PAIRS[pair]):
        print(f"no-alloc {pair} call {j}: M={M} O={O} I={I} R={R} {dtype}", flush=True)
        case = _case(M, O, I, R, dtype, seed=M + O + j)
        y_ws = tb.linear_forward(*case)
        out = torch.empty((M, O), dtype=dtype, device=DEV)
        y = tb.linear_forward_no_alloc(*case, out=out)
        torch.cuda.synchronize()
        assert y.data_ptr() == out.data_ptr()
        assert _same_bits(y, y_ws), f"{pair} call {j}: differs from tb_linear_forward"
        _parity(y, case, what=f"no-alloc {pair} call {j}")


def test_no_alloc_refuses_a_call_beyond_its_scratch():
    # 131072 tokens at rank 512: T = x V alone takes 128 MiB.
    M, O, I, R = 131072, 256, 64, 512
    assert tb.linear_forward_workspace_size(M, O, I, R, torch.bfloat16) > tb.NO_ALLOC_SCRATCH_BYTES
    x, s, W0, U, V = _case(M, O, I, R, torch.bfloat16, seed=1)
    out = torch.full((M, O), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tb.TBError) as e:
        tb.linear_forward_no_alloc(x, s, W0, U, V, out=out)
    assert e.value.status == tb.TB_ERR_UNSUPPORTED and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())           # nothing was enqueued


def test_no_alloc_timed_out_call_leaves_the_next_one_correct():
    # A poll bound of 0 makes the call's wait for x . V give up (its y is NaN);
    # the next call clears the control words first and is correct.
    big = _case(16, 2048, 5376, 256, torch.bfloat16, seed=3)
    small = _case(4, 256, 1152, 128, torch.bfloat16, seed=4)
    tb.set_wait_polls(0)
    try:
        y = tb.linear_forward_no_alloc(*big)
        torch.cuda.synchronize()
    finally:
        tb.set_wait_polls()
    assert bool(torch.isnan(y.float()).all())
    for case, what in ((small, "after a timeout, smaller"), (big, "after a timeout, again")):
        y = tb.linear_forward_no_alloc(*case)
        torch.cuda.synchronize()
        assert _same_bits(y, tb.linear_forward(*case))
        _parity(y, case, what=what)


def test_no_alloc_replays_from_a_captured_graph():
    # Captured once, replayed three times with eager calls of another shape in between.
    case = _case(16, 2048, 5376, 256, torch.bfloat16, seed=5)
    other = _case(4, 1024, 1152, 128, torch.bfloat16, seed=6)
    want = tb.linear_forward(*case).clone()
    out = torch.empty_like(want)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tb.linear_forward_no_alloc(*case, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        tb.linear_forward_no_alloc(*case, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        y_other = tb.linear_forward_no_alloc(*other)
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same_bits(out, want), rep
        assert _same_bits(y_other, tb.linear_forward(*other)), rep
