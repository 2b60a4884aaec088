"""The bf16 dK/dV kernel forms dS = P (dP - D) from P rounded to fp16 (the
value its P-wave hands to the dS-wave), where the dQ kernel uses P in fp32
and the dV product takes P rounded to bf16.  This CPU check emulates the
kernels' roundings in float32 (bf16 inputs, fp32 products and sums, P and
dS rounded as the MFMA operands are, outputs rounded to bf16) for three ways
of forming dS: from bf16 P, from fp16 P (the kernel's) and from fp32 P, and
compares each dK with the float64 oracle: all must sit well inside the 2e-2
gate, the fp16-P form within a few percent of the fp32-P form, and the
bf16-P form (the kernel's former hand-off) within a small factor of it.
The measured errors are printed (pytest -s)."""
import numpy as np
import pytest

import oracle
from flash_attention_transformers_amd import workloads as W


def _bf16(a):
    return W.bf16_bits_to_f32(W.round_to_bf16_bits(np.asarray(a, np.float32)))


def _dk_emulated(q, k, v, do, lse, dlt, causal, scale, p_for_ds):
    """dK of one head under the kernel's roundings, with dS formed from P
    rounded as `p_for_ds` says ("bf16", "f16" round to nearest even, "f32");
    q, k, v, do float32 with bf16 values, lse and dlt float32."""
    c = np.float32(scale * np.log2(np.e))
    s = (q @ k.T).astype(np.float32)
    p = np.exp2(s * c - (lse * np.float32(np.log2(np.e)))[:, None]).astype(np.float32)
    if causal:
        Sq, Skv = s.shape
        vis = np.arange(Skv)[None, :] <= np.arange(Sq)[:, None] + (Skv - Sq)
        p = np.where(vis, p, np.float32(0))
    pr = {"bf16": _bf16(p), "f16": p.astype(np.float16).astype(np.float32), "f32": p}[p_for_ds]
    dp = (do @ v.T).astype(np.float32)
    ds = _bf16(pr * (dp - dlt[:, None]))
    return _bf16(np.float32(scale) * (ds.T @ q))


@pytest.mark.parametrize("shape", [(1, 2, 2, 512, 512, 128, True), (1, 2, 2, 256, 2048, 128, False),
                                   (1, 2, 2, 1024, 1024, 64, True)])
def test_ds_from_rounded_p_costs_little(shape):
    B, Hq, Hkv, Sq, Skv, D, causal = shape
    w = W.Workload("r9", B, Hq, Hkv, Sq, Skv, D, causal, "bf16", 97, True)
    v = W.make_inputs(w).vals
    scale = w.scale
    modes = ("bf16", "f16", "f32")
    num = {m: 0.0 for m in modes}
    den = 0.0
    for h in range(Hq):
        q, k, vv, do = v["q"][0, h], v["k"][0, h], v["v"][0, h], v["do"][0, h]
        o, lse = oracle.forward_head(q, k, vv, causal, scale)
        _, rdk, _, _ = oracle.backward_head(q, k, vv, do, causal, scale)
        # D as the kernels form it: from the bf16 O the forward stores.
        dlt = np.sum(do.astype(np.float32) * _bf16(o), axis=1, dtype=np.float32)
        for m in modes:
            e = _dk_emulated(q, k, vv, do, lse.astype(np.float32), dlt, causal, scale, m) - rdk
            num[m] += float(np.sum(e * e))
        den += float(np.sum(rdk * rdk))
    err = {m: (num[m] / den) ** 0.5 for m in modes}
    print(f"\n[R9] {shape}: dK relL2 with dS from bf16 P {err['bf16']:.3e}, "
          f"from fp16 P {err['f16']:.3e}, from fp32 P {err['f32']:.3e}")
    assert max(err.values()) < 1e-2
    assert err["f16"] < 1.05 * err["f32"]
    assert err["bf16"] < 1.6 * err["f32"]
