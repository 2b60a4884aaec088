"""Shared helpers for the GPU parity tests: run libmattn on seeded inputs and
compare with the float64 oracle.  Tolerances are fixed here, once.

Whole-tensor comparisons split the oracle's work over (batch, KV head)
groups, or over blocks of query rows for forward-only workloads, and run the
pieces on a pool of host threads (the BLAS products and numpy's elementwise
loops release the interpreter lock; BLAS runs single-threaded inside each
piece).  Every element of every output is compared; the pieces only bound
memory and spread the work over the host cores.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np

import oracle
from flash_attention_transformers_amd import workloads as W

# Gates (bf16 I/O with fp32 accumulation, and the float32 path).
TOL = {
    "bf16": dict(o_max_abs=2e-2, o_rel_l2=2e-2, grad_rel_l2=2e-2, lse_max_abs=1e-3),
    "f32": dict(o_max_abs=1e-4, o_rel_l2=1e-4, grad_rel_l2=1e-4, lse_max_abs=1e-4),
}

# Results of every parity comparison in this session, printed at its end by
# conftest.pytest_terminal_summary.
RESULTS = []

ROW_BLOCK = 1024  # query rows per piece of a forward-only comparison


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


def oracle_threads() -> int:
    """Host threads for the oracle: the machine's cores, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


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


def gpu_to_host(g) -> dict:
    """Device outputs as float32 host arrays (bf16 values are exact in fp32)."""
    return {n: t.float().cpu().numpy() for n, t in g.items()}


class _Acc:
    """Running error statistics over pieces: max-abs of O and LSE, and the
    numerator and denominator of each relative L2 norm."""

    def __init__(self):
        self.o_max = 0.0
        self.lse_max = 0.0
        self.sq = {n: [0.0, 0.0] for n in ("o", "dq", "dk", "dv")}

    def add_sq(self, name, got, ref):
        e = np.asarray(got, np.float64) - ref
        self.sq[name][0] += float(np.sum(e * e))
        self.sq[name][1] += float(np.sum(ref * ref))

    def add_fwd(self, go, ro, glse, rlse):
        if ro.size:
            self.o_max = max(self.o_max, float(np.max(np.abs(np.asarray(go, np.float64) - ro))))
            self.lse_max = max(self.lse_max, float(np.max(np.abs(np.asarray(glse, np.float64) - rlse))))
        self.add_sq("o", go, ro)

    def merge(self, other: "_Acc"):
        self.o_max = max(self.o_max, other.o_max)
        self.lse_max = max(self.lse_max, other.lse_max)
        for n in self.sq:
            self.sq[n][0] += other.sq[n][0]
            self.sq[n][1] += other.sq[n][1]

    def result(self, backward: bool) -> dict:
        def rel(n):
            num, den = self.sq[n]
            return float(np.sqrt(num / den)) if den > 0 else float(np.sqrt(num))

        res = {"o_max_abs": self.o_max, "o_rel_l2": rel("o"), "lse_max_abs": self.lse_max}
        if backward:
            res.update(dq=rel("dq"), dk=rel("dk"), dv=rel("dv"))
        return res


def _group_piece(w: W.Workload, v, g, b: int, kvh: int) -> _Acc:
    """Every output of one (batch, KV head) group: O, LSE and dQ of each of
    its query heads, and dK, dV of the KV head (the in-group sum)."""
    G = w.Hq // w.Hkv
    acc = _Acc()
    k, vv = v["k"][b, kvh], v["v"][b, kvh]
    dk_ref = np.zeros((w.Skv, w.D))
    dv_ref = np.zeros((w.Skv, w.D))
    for r in range(G):
        h = kvh * G + r
        q = v["q"][b, h]
        ro, rlse = oracle.forward_head(q, k, vv, w.causal, w.scale)
        acc.add_fwd(g["o"][b, h], ro, g["lse"][b, h], rlse)
        rdq, rdk, rdv, _ = oracle.backward_head(q, k, vv, v["do"][b, h], w.causal, w.scale)
        acc.add_sq("dq", g["dq"][b, h], rdq)
        dk_ref += rdk
        dv_ref += rdv
    acc.add_sq("dk", g["dk"][b, kvh], dk_ref)
    acc.add_sq("dv", g["dv"][b, kvh], dv_ref)
    return acc


def _rows_piece(w: W.Workload, v, g, b: int, h: int, r0: int, r1: int) -> _Acc:
    """O and LSE of query rows [r0, r1) of one head."""
    G = w.Hq // w.Hkv
    rows = np.arange(r0, r1)
    ro, rlse = oracle.forward_head(v["q"][b, h], v["k"][b, h // G], v["v"][b, h // G], w.causal,
                                   w.scale, rows)
    acc = _Acc()
    acc.add_fwd(g["o"][b, h][r0:r1], ro, g["lse"][b, h][r0:r1], rlse)
    return acc


def compare_full(w: W.Workload, inp: W.Inputs, g: dict, backward: bool,
                 threads: int = None) -> dict:
    """Whole-tensor error statistics of host outputs `g` (o, lse and, with
    `backward`, dq, dk, dv as arrays) against the oracle on the same inputs:
    O max-abs and relative L2, LSE max-abs, and the relative L2 of each
    gradient over the whole flattened tensor."""
    from threadpoolctl import threadpool_limits

    v = inp.vals
    if backward:
        jobs = [(_group_piece, (w, v, g, b, kvh)) for b in range(w.B) for kvh in range(w.Hkv)]
    else:
        jobs = [(_rows_piece, (w, v, g, b, h, r0, min(w.Sq, r0 + ROW_BLOCK)))
                for b in range(w.B) for h in range(w.Hq) for r0 in range(0, w.Sq, ROW_BLOCK)]
    total = _Acc()
    n = threads or oracle_threads()
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=n) as ex:
            for acc in ex.map(lambda j: j[0](*j[1]), jobs):
                total.merge(acc)
    return total.result(backward)


def assert_gates(w: W.Workload, res: dict, backward: bool):
    tol = TOL[w.dtype]
    assert res["o_max_abs"] <= tol["o_max_abs"], res
    assert res["o_rel_l2"] <= tol["o_rel_l2"], res
    assert res["lse_max_abs"] <= tol["lse_max_abs"], res
    if backward:
        for n in ("dq", "dk", "dv"):
            assert res[n] <= tol["grad_rel_l2"], (n, res)


def check_full(w: W.Workload, dev, backward: bool = True):
    """Whole-tensor parity: every element of O, LSE and (with `backward`)
    dQ, dK, dV against the oracle."""
    say(f"[parity full] {w}")
    inp = W.make_inputs(w)
    g = gpu_to_host(run_gpu(w, inp, dev, backward))
    res = compare_full(w, inp, g, backward)
    say(f"    {res}")
    RESULTS.append((w.name, "full", res))
    assert_gates(w, res, backward)
    return res


def check_sampled(w: W.Workload, dev, kv_heads, rows_per_head=None, backward=True):
    """Full-size parity on sampled outputs: every query head of the sampled
    (b, kv-head) pairs; optionally only some query rows (forward only)."""
    say(f"[parity sampled] {w} kv_heads={kv_heads} rows={None if rows_per_head is None else len(rows_per_head)}")
    inp = W.make_inputs(w)
    g = run_gpu(w, inp, dev, backward)
    G = w.Hq // w.Hkv
    v = inp.vals
    go, glse = g["o"].float().cpu().numpy(), g["lse"].cpu().numpy()
    acc = _Acc()
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
            acc.add_fwd(go[b, h][sel], ro, glse[b, h][sel], rlse)
            if backward:
                rdq, rdk, rdv, _ = oracle.backward_head(q, k, vv, v["do"][b, h], w.causal, w.scale)
                dk_ref += rdk
                dv_ref += rdv
                acc.add_sq("dq", gdq[b, h], rdq)
        if backward:
            acc.add_sq("dk", gdk[b, kvh], dk_ref)
            acc.add_sq("dv", gdv[b, kvh], dv_ref)
    errs = acc.result(backward)
    say(f"    {errs}")
    RESULTS.append((w.name, "sampled", errs))
    assert_gates(w, errs, backward)
    return errs
