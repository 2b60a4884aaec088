"""mattn_bwd_noalloc: the backward with its workspace in the library's static
scratch array instead of a caller-provided buffer, for callers that cannot
allocate.  Called through the C ABI and compared with mattn_bwd on the same
inputs: the same kernels run, so the results must be the same bits.  Two
calls in a row, the second with a smaller problem, so the second runs on a
scratch array that still holds the first call's values."""
import ctypes

import numpy as np
import pytest

import flash_attention_transformers_amd as fa
from flash_attention_transformers_amd import workloads as W

import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    fa.load_library()
    return torch.device("cuda:0")


def _noalloc(lib, t, o, lse, dq, dk, dv, w, stream):
    vp = ctypes.c_void_p
    return lib.mattn_bwd_noalloc(
        vp(t["q"].data_ptr()), vp(t["k"].data_ptr()), vp(t["v"].data_ptr()), vp(o.data_ptr()),
        vp(lse.data_ptr()), vp(t["do"].data_ptr()), vp(dq.data_ptr()), vp(dk.data_ptr()),
        vp(dv.data_ptr()), w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, int(w.causal),
        ctypes.c_float(w.scale), 0 if w.dtype == "bf16" else 1, vp(stream))


# Largest first: split dK/dV partials fill much of the scratch; then smaller
# problems (causal GQA, fp32) over the values the first call left there.
CASES = [
    W.Workload("noalloc_cross_split", 1, 10, 10, 32760, 257, 128, False, "bf16", 52, True),
    W.Workload("noalloc_gqa_causal", 2, 8, 2, 700, 700, 128, True, "bf16", 41, True),
    W.Workload("noalloc_f32_small", 1, 4, 2, 150, 90, 64, False, "f32", 43, True),
]


def test_noalloc_matches_bwd_on_consecutive_calls(dev):
    import torch

    lib = fa.load_library()
    stream = torch.cuda.current_stream(dev).cuda_stream
    for w in CASES:
        H.say(f"[noalloc] {w}")
        need = fa.mattn_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D)
        assert need <= fa.MATTN_SCRATCH_BYTES
        t = W.to_torch(W.make_inputs(w), dev)
        o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=w.causal, scale=w.scale)
        ref = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=w.causal, scale=w.scale)
        outs = [torch.full_like(x, float("nan")) for x in ref]
        st = _noalloc(lib, t, o, lse, *outs, w, stream)
        assert st == fa.MATTN_OK, fa.mattn_strerror(st)
        torch.cuda.synchronize()
        for n, a, b in zip(("dq", "dk", "dv"), outs, ref):
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (w.name, n)


def test_noalloc_rejects_a_problem_beyond_the_scratch(dev):
    import torch

    lib = fa.load_library()
    # Dlt of 2^25 - 1 rows (128 MiB) plus split partials: over 128 MiB.
    B, Hq, Hkv, Sq, Skv, D = 1, 1, 1, (1 << 25) - 1, 100, 64
    assert fa.mattn_bwd_workspace_size(B, Hq, Hkv, Sq, Skv, D) > fa.MATTN_SCRATCH_BYTES
    x = torch.full((64,), float("nan"), device=dev)
    p = ctypes.c_void_p(x.data_ptr())  # never dereferenced: the call is rejected first
    st = lib.mattn_bwd_noalloc(p, p, p, p, p, p, p, p, p, B, Hq, Hkv, Sq, Skv, D, 0,
                               ctypes.c_float(0.088), 0, ctypes.c_void_p(0))
    assert st == fa.MATTN_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(x).all()
