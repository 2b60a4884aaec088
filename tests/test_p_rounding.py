"""The bf16 dK/dV kernel forms dS = P (dP - D) from P already rounded to bf16
(the value it hands to the PV-style product), where the dQ kernel uses P in
fp32.  This CPU check emulates the kernels' roundings in float32 (bf16
inputs, fp32 products and sums, P and dS rounded to bf16 as MFMA operands,
outputs rounded to bf16) for both ways of forming dS, and compares each dK
with the float64 oracle: both must sit well inside the 2e-2 gate, and the
bf16-P form must not cost more than a small factor over the fp32-P form.
The measured errors are printed (pytest -s)."""
import numpy as np
import pytest

import oracle
from flash_attention_transformers_amd import workloads as W


def _bf16(a):
    return W.bf16_bits_to_f32(W.round_to_bf16_bits(np.asarray(a, np.float32)))


def _dk_emulated(q, k, v, do, lse, dlt, causal, scale, p_bf16_for_ds):
    """dK of one head under the kernel's roundings; q, k, v, do float32 with
    bf16 values, lse and dlt float32."""
    c = np.float32(scale * np.log2(np.e))
    s = (q @ k.T).astype(np.float32)
    p = np.exp2(s * c - (lse * np.float32(np.log2(np.e)))[:, None]).astype(np.float32)
    if causal:
        Sq, Skv = s.shape
        vis = np.arange(Skv)[None, :] <= np.arange(Sq)[:, None] + (Skv - Sq)
        p = np.where(vis, p, np.float32(0))
    pb = _bf16(p)
    dp = (do @ v.T).astype(np.float32)
    ds = _bf16((pb if p_bf16_for_ds else p) * (dp - dlt[:, None]))
    return _bf16(np.float32(scale) * (ds.T @ q))


@pytest.mark.parametrize("shape", [(1, 2, 2, 512, 512, 128, True), (1, 2, 2, 256, 2048, 128, False),
                                   (1, 2, 2, 1024, 1024, 64, True)])
def test_ds_from_bf16_p_costs_little(shape):
    B, Hq, Hkv, Sq, Skv, D, causal = shape
    w = W.Workload("r9", B, Hq, Hkv, Sq, Skv, D, causal, "bf16", 97, True)
    v = W.make_inputs(w).vals
    scale = w.scale
    num = {True: 0.0, False: 0.0}
    den = 0.0
    for h in range(Hq):
        q, k, vv, do = v["q"][0, h], v["k"][0, h], v["v"][0, h], v["do"][0, h]
        o, lse = oracle.forward_head(q, k, vv, causal, scale)
        _, rdk, _, _ = oracle.backward_head(q, k, vv, do, causal, scale)
        # D as the kernels form it: from the bf16 O the forward stores.
        dlt = np.sum(do.astype(np.float32) * _bf16(o), axis=1, dtype=np.float32)
        for mode in (True, False):
            e = _dk_emulated(q, k, vv, do, lse.astype(np.float32), dlt, causal, scale, mode) - rdk
            num[mode] += float(np.sum(e * e))
        den += float(np.sum(rdk * rdk))
    err_bf16_p = (num[True] / den) ** 0.5
    err_f32_p = (num[False] / den) ** 0.5
    print(f"\n[R9] {shape}: dK relL2 with dS from bf16 P {err_bf16_p:.3e}, from fp32 P {err_f32_p:.3e}")
    assert err_bf16_p < 1e-2 and err_f32_p < 1e-2
    assert err_bf16_p < 1.6 * err_f32_p
