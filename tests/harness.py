"""Shared helpers for the GPU parity tests: run libmattn on seeded inputs and
compare with the float64 oracle.  Tolerances are fixed here, once."""
from __future__ import annotations

import sys

import numpy as np

import oracle
from flash_attention_transformers_amd import workloads as W

# Gates (bf16 I/O with fp32 accumulation, and the float32 path).
TOL = {
    "bf16": dict(o_max_abs=2e-2, o_rel_l2=2e-2, grad_rel_l2=2e-2, lse_max_abs=1e-3),
    "f32": dict(o_max_abs=1e-4, o_rel_l2=1e-4, grad_rel_l2=1e-4, lse_max_abs=1e-4),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def max_abs(a, r) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - r))) if np.size(r) else 0.0


def rel_l2(a, r) -> float:
    den = np.linalg.norm(r)
    return float(np.linalg.norm(np.asarray(a, np.float64) - r) / (den if den > 0 else 1.0))


def to_np(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_gpu(w: W.Workload, inp: W.Inputs, dev, backward: bool):
    import torch

    import flash_attention_transformers_amd as fa

    t = W.to_torch(inp, dev)
    o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=w.causal, scale=w.scale)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=w.causal, scale=w.scale)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return out


def check_full(w: W.Workload, dev, backward: bool = True):
    """Whole-tensor parity for sizes the oracle finishes in seconds."""
    say(f"[parity full] {w}")
    inp = W.make_inputs(w)
    g = run_gpu(w, inp, dev, backward)
    v = inp.vals
    ro, rlse = oracle.attention_forward(v["q"], v["k"], v["v"], w.causal, w.scale)
    tol = TOL[w.dtype]
    res = {"o_max_abs": max_abs(to_np(g["o"]), ro), "o_rel_l2": rel_l2(to_np(g["o"]), ro),
           "lse_max_abs": max_abs(to_np(g["lse"]), rlse)}
    if backward:
        rdq, rdk, rdv, _ = oracle.attention_backward(v["q"], v["k"], v["v"], v["do"], w.causal, w.scale)
        res.update(dq=rel_l2(to_np(g["dq"]), rdq), dk=rel_l2(to_np(g["dk"]), rdk),
                   dv=rel_l2(to_np(g["dv"]), rdv))
    say(f"    {res}")
    assert res["o_max_abs"] <= tol["o_max_abs"], res
    assert res["o_rel_l2"] <= tol["o_rel_l2"], res
    assert res["lse_max_abs"] <= tol["lse_max_abs"], res
    if backward:
        for n in ("dq", "dk", "dv"):
            assert res[n] <= tol["grad_rel_l2"], (n, res)
    return res


def check_sampled(w: W.Workload, dev, kv_heads, rows_per_head=None, backward=True):
    """Full-size parity on sampled outputs: every query head of the sampled
    (b, kv-head) pairs; optionally only some query rows (forward only)."""
    say(f"[parity sampled] {w} kv_heads={kv_heads} rows={None if rows_per_head is None else len(rows_per_head)}")
    inp = W.make_inputs(w)
    g = run_gpu(w, inp, dev, backward)
    G = w.Hq // w.Hkv
    v = inp.vals
    tol = TOL[w.dtype]
    go, glse = g["o"].float().cpu().numpy(), g["lse"].cpu().numpy()
    errs = {"o_max_abs": 0.0, "lse_max_abs": 0.0}
    o_num = o_den = 0.0
    grad_sq = {"dq": [0.0, 0.0], "dk": [0.0, 0.0], "dv": [0.0, 0.0]}
    if backward:
        gdq, gdk, gdv = (g[n].float().cpu().numpy() for n in ("dq", "dk", "dv"))
    for b, kvh in kv_heads:
        dk_ref = np.zeros((w.Skv, w.D))
        dv_ref = np.zeros((w.Skv, w.D))
        for r in range(G):
            h = kvh * G + r
            q, k, vv = v["q"][b, h], v["k"][b, kvh], v["v"][b, kvh]
            rows = rows_per_head
            ro, rlse = oracle.forward_head(q, k, vv, w.causal, w.scale, rows)
            sel = slice(None) if rows is None else np.asarray(rows)
            d = go[b, h][sel].astype(np.float64) - ro
            errs["o_max_abs"] = max(errs["o_max_abs"], float(np.abs(d).max()))
            o_num += float(np.sum(d * d))
            o_den += float(np.sum(ro * ro))
            errs["lse_max_abs"] = max(errs["lse_max_abs"], max_abs(glse[b, h][sel], rlse))
            if backward:
                rdq, rdk, rdv, _ = oracle.backward_head(q, k, vv, v["do"][b, h], w.causal, w.scale)
                dk_ref += rdk
                dv_ref += rdv
                e = gdq[b, h].astype(np.float64) - rdq
                grad_sq["dq"][0] += float(np.sum(e * e))
                grad_sq["dq"][1] += float(np.sum(rdq * rdq))
        if backward:
            for n, gg, rr in (("dk", gdk[b, kvh], dk_ref), ("dv", gdv[b, kvh], dv_ref)):
                e = gg.astype(np.float64) - rr
                grad_sq[n][0] += float(np.sum(e * e))
                grad_sq[n][1] += float(np.sum(rr * rr))
    errs["o_rel_l2"] = float(np.sqrt(o_num / o_den))
    if backward:
        for n in grad_sq:
            errs[n] = float(np.sqrt(grad_sq[n][0] / grad_sq[n][1]))
    say(f"    {errs}")
    assert errs["o_max_abs"] <= tol["o_max_abs"], errs
    assert errs["o_rel_l2"] <= tol["o_rel_l2"], errs
    assert errs["lse_max_abs"] <= tol["lse_max_abs"], errs
    if backward:
        for n in ("dq", "dk", "dv"):
            assert errs[n] <= tol["grad_rel_l2"], (n, errs)
    return errs
