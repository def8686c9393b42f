"""Host-only checks of the Python binding's argument validation.

The C ABI takes raw pointers and cannot see buffer sizes, so the binding must
reject every mis-sized operand or output before anything crosses the ABI.
These tests use CPU tensors: the shape and dtype checks run before the device
checks, so a wrong shape is reported as such (and nothing could be launched
from here anyway).
"""

import pytest
import torch

tb = pytest.importorskip("rank_factored_linear_amd.binding")

BF = torch.bfloat16


def _case(M=4, O=16, I=32, R=8, dtype=BF):
    z = lambda *s: torch.zeros(*s, dtype=dtype)
    return z(M, I), z(O), z(O, I), z(O, R), z(I, R)


def _raises(fn, *words):
    with pytest.raises(tb.TBError) as e:
        fn()
    assert e.value.status == tb.TB_ERR_INVALID_ARGUMENT, str(e.value)
    for w in words:
        assert w in str(e.value), str(e.value)


def test_well_formed_cpu_call_fails_only_on_the_device():
    x, s, W0, U, V = _case()
    _raises(lambda: tb.linear_forward(x, s, W0, U, V), "GPU")


@pytest.mark.parametrize("bad", ["x_in", "W0_in", "s_len", "U_rows", "U_rank", "V_rows", "V_rank", "U_only",
                                 "dtype_mix", "out_shape", "out_dtype"])
def test_linear_forward_rejects_mis_sized_operands(bad):
    x, s, W0, U, V = _case()
    out = None
    word = {"x_in": "W0", "W0_in": "W0", "s_len": "s", "U_rows": "U", "U_rank": "V", "V_rows": "V", "V_rank": "V",
            "U_only": "together", "dtype_mix": "bfloat16", "out_shape": "out", "out_dtype": "out"}[bad]
    if bad == "x_in":
        x = torch.zeros(4, 40, dtype=BF)
    elif bad == "W0_in":
        W0 = torch.zeros(16, 40, dtype=BF)
    elif bad == "s_len":
        s = torch.zeros(15, dtype=BF)
    elif bad == "U_rows":
        U = torch.zeros(17, 8, dtype=BF)
    elif bad == "U_rank":
        U = torch.zeros(16, 9, dtype=BF)
    elif bad == "V_rows":
        V = torch.zeros(33, 8, dtype=BF)
    elif bad == "V_rank":
        V = torch.zeros(32, 7, dtype=BF)
    elif bad == "U_only":
        V = None
    elif bad == "dtype_mix":
        s = torch.zeros(16, dtype=torch.float32)
    elif bad == "out_shape":
        out = torch.zeros(4, 17, dtype=BF)
    elif bad == "out_dtype":
        out = torch.zeros(4, 16, dtype=torch.float32)
    _raises(lambda: tb.linear_forward(x, s, W0, U, V, out=out), word)


def test_dense_forward_rejects_mis_sized_operands():
    x, _, W, _, _ = _case()
    _raises(lambda: tb.dense_forward(x, torch.zeros(16, 31, dtype=BF)), "W0")
    _raises(lambda: tb.dense_forward(x, W, out=torch.zeros(3, 16, dtype=BF)), "out")


def test_group_checks_every_member():
    good = _case()
    x, s, W0, U, V = _case(O=24, I=40, R=4)
    bad_members = [
        (x, s, W0, U, torch.zeros(40, 5, dtype=BF)),          # V's rank differs from U's
        (torch.zeros(4, 48, dtype=BF), s, W0, U, V),           # x's in_dim differs from W0's
        (x, torch.zeros(23, dtype=BF), W0, U, V),              # s too short
        (torch.zeros(5, 40, dtype=BF), s, W0, U, V),           # token count differs from member 0
    ]
    words = ["V", "W0", "s", "token count"]
    for bad, word in zip(bad_members, words):
        _raises(lambda: tb.linear_forward_group([good, bad]), word)
    _raises(lambda: tb.linear_forward_group([good], outs=[torch.zeros(4, 15, dtype=BF)]), "out")
    _raises(lambda: tb.linear_forward_group([good] * 9), "1..8")


def test_reconstruct_and_errors_reject_mis_sized_operands():
    _, s, W0, U, V = _case()
    _raises(lambda: tb.reconstruct_weight(torch.zeros(15, dtype=BF), W0, U, V), "s")
    _raises(lambda: tb.reconstruct_weight(s, W0, U, torch.zeros(31, 8, dtype=BF)), "V")
    _raises(lambda: tb.reconstruct_weight(s, W0, U, V, out=torch.zeros(16, 33)), "out")
    orig = torch.zeros(16, 32)
    _raises(lambda: tb.reconstruction_error(torch.zeros(16, 31), s, W0, U, V), "original")
    _raises(lambda: tb.reconstruction_error(orig, s, W0, torch.zeros(16, 9, dtype=BF), V), "V")
    _raises(lambda: tb.reconstruction_error(orig, torch.zeros(17, dtype=BF), W0, U, V), "s")
    _raises(lambda: tb.rel_frobenius_error(orig, torch.zeros(16, 40)), "reconstructed")
    _raises(lambda: tb.rel_frobenius_error(orig, orig.to(BF)), "reconstructed")
    # The result is one float64 on the device: an fp32 or a larger out is refused.
    _raises(lambda: tb.rel_frobenius_error(orig, orig, out=torch.zeros((), dtype=torch.float32)), "float64")
    _raises(lambda: tb.rel_frobenius_error(orig, orig, out=torch.zeros(2, dtype=torch.float64)), "float64")
    _raises(lambda: tb.reconstruction_error(orig, s, W0, U, V, out=torch.zeros(1, dtype=torch.float32)), "float64")


def test_decomposition_wrappers_reject_mis_sized_operands():
    w = torch.zeros(16, 32)
    _raises(lambda: tb.shared_block([w, torch.zeros(16, 31)]), "weights[1]")
    _raises(lambda: tb.row_scale(w, torch.zeros(16, 31)), "W0")
    _raises(lambda: tb.row_scale(w, w, out=torch.zeros(15)), "out")
    _raises(lambda: tb.lowrank_factors(w, w, torch.zeros(15), 4, torch.zeros(32, 8), 0), "s")
    _raises(lambda: tb.lowrank_factors(w, w, torch.zeros(16), 4, torch.zeros(31, 8), 0), "omega")
    S, om = torch.zeros(2, 16), torch.zeros(2, 32, 8)
    _raises(lambda: tb.lowrank_factors_batch([w, w], [w], S, 4, om, 0), "one shared block")
    _raises(lambda: tb.lowrank_factors_batch([w, w], w, torch.zeros(2, 15), 4, om, 0), "S")
    _raises(lambda: tb.lowrank_factors_batch([w, w], w, S, 4, torch.zeros(3, 32, 8), 0), "omega")
    U, V = torch.zeros(16, 4), torch.zeros(32, 4)
    _raises(lambda: tb.refine_shared_block([w], [torch.zeros(16)], [U], [torch.zeros(32, 5)], w), "V[0]")
    _raises(lambda: tb.refine_shared_block([w], [torch.zeros(16)], [U], [V], w, out=torch.zeros(16, 31)), "out")


def test_decompose_model_rejects_bad_arguments():
    ws = [torch.zeros(16, 32, dtype=BF) for _ in range(2)]
    _raises(lambda: tb.decompose_model({"q_proj": ws}, 1, 0, tie_families="mlp"), "tie_families")
    _raises(lambda: tb.decompose_model({"q_proj": ws}, 1, 0, tie_families=""), "tie_families")
    _raises(lambda: tb.decompose_model({"lm_head": ws}, 1, 0), "lm_head")


def test_decompose_model_keeps_the_mlp_dense_without_a_launch():
    # tie_families="attn" with MLP families only: nothing is decomposed, so
    # this runs on host tensors; each layer's bundle is its own weight.
    ws = {f: [torch.zeros(16, 32, dtype=BF) for _ in range(3)] for f in tb.MLP_FAMILIES}
    got = tb.decompose_model(ws, 1, 8, tie_families="attn")
    for f in tb.MLP_FAMILIES:
        assert got[f]["band"] == [0, 1, 2]
        assert all(a is b for a, b in zip(got[f]["W0"], ws[f]))
        assert got[f]["s"] == [None] * 3 and got[f]["U"] == [None] * 3 and got[f]["V"] == [None] * 3
