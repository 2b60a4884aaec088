"""The whole-tensor parity comparison itself (CPU only, no GPU): given the
oracle's own outputs rounded to bf16 it passes the gates, and a planted
mistake of the kind a head remap or tile order bug would make (two query
heads swapped, a wrong KV head's gradient, one corrupted row in the ragged
last block) fails them.  The planted mistakes go into the host copies that
stand in for the library's outputs."""
import numpy as np
import pytest

import oracle
from flash_attention_transformers_amd import workloads as W

import harness as H


def _bf16(a):
    return W.bf16_bits_to_f32(W.round_to_bf16_bits(np.asarray(a, np.float32)))


def _fake_outputs(w, inp, backward=True):
    v = inp.vals
    o, lse = oracle.attention_forward(v["q"], v["k"], v["v"], w.causal, w.scale)
    g = {"o": _bf16(o), "lse": lse.astype(np.float32)}
    if backward:
        dq, dk, dv, _ = oracle.attention_backward(v["q"], v["k"], v["v"], v["do"], w.causal, w.scale)
        g.update(dq=_bf16(dq), dk=_bf16(dk), dv=_bf16(dv))
    return g


W_BWD = W.Workload("harness_gqa", 2, 4, 2, 70, 90, 64, True, "bf16", 5, True)
W_FWD = W.Workload("harness_rows", 1, 2, 1, 2 * H.ROW_BLOCK + 37, 40, 64, False, "bf16", 6, False)


def test_exact_outputs_pass():
    inp = W.make_inputs(W_BWD)
    res = H.compare_full(W_BWD, inp, _fake_outputs(W_BWD, inp), True, threads=4)
    H.assert_gates(W_BWD, res, True)
    assert res["o_max_abs"] < 4e-3 and res["dk"] < 4e-3, res


def test_swapped_query_heads_fail():
    inp = W.make_inputs(W_BWD)
    g = _fake_outputs(W_BWD, inp)
    g["o"][1, [0, 1]] = g["o"][1, [1, 0]]
    res = H.compare_full(W_BWD, inp, g, True, threads=4)
    with pytest.raises(AssertionError):
        H.assert_gates(W_BWD, res, True)


def test_wrong_kv_head_gradient_fails():
    inp = W.make_inputs(W_BWD)
    g = _fake_outputs(W_BWD, inp)
    g["dk"][0, 1] = g["dk"][0, 0]
    res = H.compare_full(W_BWD, inp, g, True, threads=4)
    assert res["dk"] > H.TOL["bf16"]["grad_rel_l2"], res
    assert res["dv"] < 4e-3, res


def test_forward_row_blocks_cover_the_ragged_end():
    inp = W.make_inputs(W_FWD)
    g = _fake_outputs(W_FWD, inp, backward=False)
    res = H.compare_full(W_FWD, inp, g, False, threads=4)
    H.assert_gates(W_FWD, res, False)
    g["o"][0, 1, -1] += 0.5
    res = H.compare_full(W_FWD, inp, g, False, threads=4)
    assert res["o_max_abs"] > 0.4, res
    g = _fake_outputs(W_FWD, inp, backward=False)
    g["lse"][0, 0, H.ROW_BLOCK] += 0.01
    res = H.compare_full(W_FWD, inp, g, False, threads=4)
    assert res["lse_max_abs"] > 0.009, res
