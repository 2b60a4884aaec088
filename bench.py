"""Benchmark of the fused attention hot path on one MI355X.

One step = mattn_fwd + the backward (the dQ kernel, which also forms
D = sum(dO*O) for bf16, then the dK/dV kernel) over one batch of seeded
synthetic input that is already resident in HBM.  The backward is enqueued as
its stages (mattn_bwd_stages, the same kernels mattn_bwd issues, in the same
order on the same stream).  The timed region holds exactly `steps` steps and
nothing else, run as 3 consecutive groups with HIP events between them; the
figure is the median of the group means (the LingBot report's timing
protocol: groups of event timings, median of the group means).  The forward
alone is timed the same way to split the step into forward and backward, and
a second pass with events between the kernels gives the per-kernel times.
Clocks (sclk, mclk) are read before and after.

With the default workload the same run also measures, each with its own
warm-up and 3 groups: the DiT self-attention forward, the two DiT
cross-attention shapes and the decoder shape, the latter three warm and with
inputs rotated through more than 1 GiB (beyond the 256 MB last-level cache),
each against its roofline; they appear under "workloads" in the same line.

Default workload: GQA causal training attention, B=4, Hq=32, Hkv=8, S=4096,
D=128, bf16 (the long-sequence configuration that exercises every step of the
path, including the grouped-KV head map and the group-summed backward).

Prints ONE JSON line.  `value` is credited TFLOP/s of the whole step:
(4*B*Hq*Sq*Skv*D forward + 2.5x that backward, halved for causal) / step time.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-extra]
    python bench.py --copy-probe   # plain 1 GiB device copy, to calibrate HBM byte counters
    python bench.py --gemm-probe   # library bf16 GEMM rate: what a plain contraction reaches here

The roofline object describes the kernel with the largest share of the step.
Algorithmic work per launch, with F = 4*B*Hq*Sq*Skv*D (halved when causal):
forward F (QK^T and PV); dK/dV 2F (S, dP, dV, dK); dQ 1.5F (S, dP, dQ).  The
two backward kernels each recompute S and dP, so together they execute 3.5F
against the 2.5F credited to the backward.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
F32_PEAK_TFLOPS = 157.3    # MI355X fp32 matrix / packed vector peak
PROFILES = os.path.join(ROOT, "profiles")


KERNEL_SOURCES = {
    "fwd_bf16_kernel": "fwd_bf16.hip", "bwd_dkdv_kernel": "bwd_bf16.hip",
    "bwd_dq_kernel": "bwd_bf16.hip", "fwd_f32_kernel": "attn_f32.hip",
    "dkdv_f32_kernel": "attn_f32.hip", "dq_f32_kernel": "attn_f32.hip",
    "kvcache_fwd_kernel": "kvcache_bf16.hip",
}
HBM_PEAK_GBS = 8000.0


def _traffic_from_profile(kernel: str, workload: str):
    """Per-launch HBM bytes of `kernel` from the committed rocprofv3 counter
    summary, or None if absent or if the kernel's source (or the shared
    header) changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel source sha256: ([0-9a-f]{64})", text)
    m_b = re.search(r"HBM bytes per launch \(calibrated\): ([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_sha(kernel):
        return None
    return float(m_b.group(1))


def roofline_kernel(stage: str, dtype: str) -> str:
    """Kernel name (as rocprofv3 and the profile summaries call it) of a stage."""
    if dtype == "bf16":
        return {"fwd": "fwd_bf16_kernel", "dkdv": "bwd_dkdv_kernel", "dq": "bwd_dq_kernel"}[stage]
    return {"fwd": "fwd_f32_kernel", "dkdv": "dkdv_f32_kernel", "dq": "dq_f32_kernel"}[stage]


def kernel_source_sha(kernel: str) -> str:
    csrc = os.path.join(ROOT, "flash_attention_transformers_amd", "csrc")
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "common.hpp", "grp_layout.hpp"):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def copy_probe(steps: int):
    """Plain device-to-device copy of 1 GiB, `steps` times: the reference for
    scaling FETCH_SIZE / WRITE_SIZE (each launch reads and writes 1 GiB)."""
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_launch": n, "launches": steps}), flush=True)


def gemm_probe(steps: int):
    """Rate of torch's bf16 matrix product (the vendor GEMM library) on square
    operands: the rate a plain dense contraction reaches on this GPU at its
    sustained clock, a practical reference beside the nominal MFMA peak."""
    import torch

    out = {}
    for n in (8192, 16384):
        g = torch.Generator(device="cuda:0").manual_seed(0)
        a = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
        b = torch.randn(n, n, device="cuda:0", dtype=torch.bfloat16, generator=g)
        for _ in range(3):
            c = a @ b
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out[f"gemm_bf16_{n}_tflops"] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
        del a, b, c
    out["peak_tflops"] = BF16_PEAK_TFLOPS
    print(json.dumps(out), flush=True)


def cpu_baseline(w, budget_s: float = 12.0):
    """Time the float64 oracle on the host cores on a bounded sample of the
    same workload: whole KV-head groups (all their query heads), forward and
    backward, until the time budget is spent.  Rate = credited FLOP of the
    sample / time."""
    import numpy as np

    import oracle
    from flash_attention_transformers_amd import workloads as W

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    G = w.Hq // w.Hkv
    small = w.with_shape(B=1, Hq=G, Hkv=1)  # one KV-head group at full sequence length
    inp = W.make_inputs(small, seed=w.seed)
    v = inp.vals
    groups = 0
    t0 = time.perf_counter()
    while True:
        for r in range(G):
            q, k, vv, do = v["q"][0, r], v["k"][0, 0], v["v"][0, 0], v["do"][0, r]
            oracle.forward_head(q, k, vv, w.causal, w.scale)
            if w.backward:
                oracle.backward_head(q, k, vv, do, w.causal, w.scale)
        groups += 1
        el = time.perf_counter() - t0
        if el >= budget_s or groups >= w.B * w.Hkv:
            break
    flop_per_group = small.fwd_flop() * (3.5 if w.backward else 1.0)
    return {
        "value": groups * flop_per_group / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{groups} of {w.B * w.Hkv} (batch, kv-head) groups, each with its {G} query "
                  f"head(s) at Sq={w.Sq}, Skv={w.Skv}, D={w.D}, causal={w.causal}, "
                  f"{'forward+backward' if w.backward else 'forward'}, float64, "
                  f"{el:.1f} s; rate credited like the GPU (causal halved)",
    }


def cpu_baseline_paged(w, budget_s: float = 12.0):
    """The paged oracle on the host cores, one whole sequence at a time (all
    its query heads), until the time budget is spent."""
    import oracle
    from flash_attention_transformers_amd import workloads as W

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    inp = W.make_paged_inputs(w)
    v = inp.vals
    done, flop = 0, 0.0
    t0 = time.perf_counter()
    while done < w.B:
        b = done
        oracle.kvcache_forward(v["q"][b:b + 1], v["k_cache"], v["v_cache"],
                               inp.block_table[b:b + 1], inp.seqlens[b:b + 1], w.causal, w.scale)
        one = dataclasses.replace(w, B=1, seqlens=(w.seqlens[b],))
        flop += one.fwd_flop()
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {
        "value": flop / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(cores),
        "kind": "oracle",
        "sample": f"{done} of {w.B} sequences (all {w.Hq} query heads, Sq={w.Sq}, their effective "
                  f"cached keys), forward, float64, {el:.1f} s; rate credited like the GPU",
    }


def main_paged(args, w):
    """Forward over the paged KV cache: one mattn_fwd_kvcache call per step
    (the attention kernel plus, for split caches, the merge kernel)."""
    import torch

    import flash_attention_transformers_amd as fa
    from flash_attention_transformers_amd import workloads as W

    dev = torch.device("cuda:0")
    fa.load_library()
    inp = W.make_paged_inputs(w)
    t = W.paged_to_torch(inp, dev)
    del inp
    q = t["q"]
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    n = fa.mattn_fwd_kvcache_workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.D, w.page_size,
                                            w.pages_per_seq)
    ws = torch.empty(n, dtype=torch.uint8, device=dev) if n > 0 else None
    stream = torch.cuda.current_stream(dev)

    def step():
        fa.mattn_fwd_kvcache(q, t["k_cache"], t["v_cache"], t["block_table"], t["seqlens"], o, lse,
                             ws, w.causal, w.scale, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / args.steps
    # Per-call span (attention kernel plus merge): a second pass with events
    # around each call.
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in evs:
        e[0].record(stream)
        step()
        e[1].record(stream)
    torch.cuda.synchronize()
    call_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / args.steps
    flop = w.fwd_flop()
    value = flop / (ms_step * 1e-3) / 1e12
    qo_bytes = 2.0 * 2 * w.B * w.Hq * w.Sq * w.D + 4.0 * w.B * w.Hq * w.Sq
    moved = w.kv_bytes() + qo_bytes
    achieved = moved / (call_ms * 1e-3) / 1e9
    line = {
        "metric": "attention TFLOPS fwd and fwd+bwd at 1 MI355X; % of bf16 MFMA peak",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) paged cache, shuffled block table, resident in HBM)",
        "config": {
            "workload": f"{w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Sq={w.Sq} D={w.D} "
                        f"page_size={w.page_size} seqlens={list(w.seqlens)} causal={int(w.causal)}; "
                        f"step = forward over the paged KV cache",
            "global_batch": w.B, "seq_len": w.Sq, "parallelism": "single GPU",
        },
        "pct_of_peak": round(100 * value / BF16_PEAK_TFLOPS, 3),
        "kernel_ms": {"kvcache": round(call_ms, 4)},
        "wall_s_timed_region": round(wall, 4),
        "roofline": {
            "kernel": "kvcache_fwd_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": _traffic_from_profile("kvcache_fwd_kernel", w.name),
            "bytes_per_launch": moved,
        },
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_paged(w)
    print(json.dumps(line), flush=True)


def read_clocks():
    """Current GPU clocks in MHz (sclk and mclk), read in-process through
    amdsmi: no child program may be started once the GPU is initialised.
    Either may be None where the interface is unavailable."""
    out = {"sclk_mhz": None, "mclk_mhz": None}
    try:
        import amdsmi
        import torch

        handle = torch.cuda._get_amdsmi_handler(torch.device("cuda:0"))
        for key, typ in (("sclk_mhz", amdsmi.AmdSmiClkType.GFX), ("mclk_mhz", amdsmi.AmdSmiClkType.MEM)):
            info = amdsmi.amdsmi_get_clock_info(handle, typ)
            val = info.get("cur_clk", info.get("clk"))
            out[key] = int(val) if isinstance(val, (int, float)) else None
    except Exception:  # pragma: no cover - interface missing
        pass
    return out


def time_groups(fn, steps: int, stream, groups: int = 3, during=None):
    """Run fn(i) for i in [0, steps) as `groups` consecutive groups inside
    one synchronized region, with HIP events recorded on `stream` between
    the groups.  Returns (mean ms per call of each group, wall seconds).
    `during`, if given, is called once every call is enqueued and before the
    synchronize, while the GPU still works through them."""
    import torch

    groups = max(1, min(groups, steps))
    bounds = [steps * g // groups for g in range(groups + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for g in range(groups):
        for i in range(bounds[g], bounds[g + 1]):
            fn(i)
        evs[g + 1].record(stream)
    if during is not None:
        during()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    means = [evs[g].elapsed_time(evs[g + 1]) / (bounds[g + 1] - bounds[g]) for g in range(groups)]
    return means, wall


def median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def algo_bytes(w):
    """Algorithmic HBM bytes (each tensor read or written once): forward reads
    q, k, v and writes o and lse; the backward reads q, k, v, o, dO and lse
    and writes dq, dk and dv (the per-row D workspace excluded)."""
    e = 2 if w.dtype == "bf16" else 4
    q = w.B * w.Hq * w.Sq * w.D * e
    kv = w.B * w.Hkv * w.Skv * w.D * e
    lse = w.B * w.Hq * w.Sq * 4
    return 2 * q + 2 * kv + lse, 4 * q + 4 * kv + lse


class DenseRun:
    """Device buffers of one workload (R copies when rotating inputs through
    more memory than the last-level cache holds) and the calls of one step."""

    def __init__(self, w, dev, stream, copies: int = 1):
        import torch

        import flash_attention_transformers_amd as fa
        from flash_attention_transformers_amd import workloads as W

        self.fa, self.w, self.stream = fa, w, stream
        inp = W.make_inputs(w)
        base = W.to_torch(inp, dev)
        del inp
        self.sets = []
        # One workspace serves every copy: each step rewrites what it reads.
        ws = fa.bwd_workspace(base["q"], base["k"]) if w.backward else None
        for r in range(copies):
            t = {n: (x if r == 0 else x.clone()) for n, x in base.items()}
            t["o"] = torch.empty_like(t["q"])
            t["lse"] = torch.empty(t["q"].shape[:3], dtype=torch.float32, device=dev)
            if w.backward:
                t["dq"], t["dk"], t["dv"] = (torch.empty_like(t["q"]), torch.empty_like(t["k"]),
                                             torch.empty_like(t["v"]))
                t["ws"] = ws
            self.sets.append(t)
        # The stages mattn_bwd enqueues: bf16 forms D inside the dQ kernel.
        if not w.backward:
            self.stages, self.names = [], ["fwd"]
        elif w.dtype == "bf16":
            self.stages, self.names = [fa.MATTN_BWD_DQ, fa.MATTN_BWD_DKDV], ["fwd", "dq", "dkdv"]
        else:
            self.stages = [fa.MATTN_BWD_PREPROCESS, fa.MATTN_BWD_DQ, fa.MATTN_BWD_DKDV]
            self.names = ["fwd", "pre", "dq", "dkdv"]

    def footprint(self) -> int:
        """Bytes of one copy of the inputs and outputs (the shared workspace aside)."""
        return sum(x.numel() * x.element_size() for n, x in self.sets[0].items() if n != "ws")

    def fwd(self, i: int):
        t, w = self.sets[i % len(self.sets)], self.w
        self.fa.mattn_fwd(t["q"], t["k"], t["v"], t["o"], t["lse"], w.causal, w.scale, self.stream)

    def step(self, i: int, ev=None):
        t, w = self.sets[i % len(self.sets)], self.w
        if ev is not None:
            ev[0].record(self.stream)
        self.fwd(i)
        if ev is not None:
            ev[1].record(self.stream)
        for j, st in enumerate(self.stages):
            self.fa.mattn_bwd_stages(t["q"], t["k"], t["v"], t["o"], t["lse"], t["do"], t["dq"],
                                     t["dk"], t["dv"], t["ws"], st, w.causal, w.scale, self.stream)
            if ev is not None:
                ev[2 + j].record(self.stream)

    def kernel_ms(self, steps: int):
        """Per-kernel spans: `steps` steps with an event between kernels."""
        import torch

        nev = 2 + len(self.stages)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
        for i in range(steps):
            self.step(i, evs[i])
        torch.cuda.synchronize()
        return {n: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / steps
                for i, n in enumerate(self.names)}


def sclk_now():
    """The GPU's current shader clock in MHz (amdsmi through torch), or None."""
    import torch

    try:
        return int(torch.cuda.clock_rate(0))
    except Exception:  # pragma: no cover
        return None


def measure(run: DenseRun, steps: int, warmup: int, clocks=None):
    """Warm up, then the step and the forward alone, each as 3 groups; the
    median of the group means is the figure.  With `clocks` (a list), the
    shader clock sampled while the timed steps run is appended to it."""
    import torch

    for i in range(max(warmup, len(run.sets))):
        run.step(i)
    torch.cuda.synchronize()
    during = None if clocks is None else (lambda: clocks.append(sclk_now()))
    step_groups, wall = time_groups(run.step, steps, run.stream, during=during)
    fwd_groups, _ = time_groups(run.fwd, steps, run.stream)
    return step_groups, fwd_groups, wall


def summarize(w, step_groups, fwd_groups, peak):
    ms_step = median(step_groups)
    fwd_ms = median(fwd_groups)
    fwd_flop = w.fwd_flop()
    out = {
        "ms_per_step": round(ms_step, 4),
        "step_group_ms": [round(x, 4) for x in step_groups],
        "fwd_ms": round(fwd_ms, 4),
        "fwd_group_ms": [round(x, 4) for x in fwd_groups],
        "fwd_tflops": round(fwd_flop / (fwd_ms * 1e-3) / 1e12, 2),
    }
    out["fwd_pct_of_peak"] = round(100 * out["fwd_tflops"] / peak, 2)
    if w.backward:
        bwd_ms = ms_step - fwd_ms
        out["bwd_ms"] = round(bwd_ms, 4)
        out["bwd_tflops"] = round(w.bwd_flop() / (bwd_ms * 1e-3) / 1e12, 2)
        out["bwd_pct_of_peak"] = round(100 * out["bwd_tflops"] / peak, 2)
        out["step_tflops"] = round((fwd_flop + w.bwd_flop()) / (ms_step * 1e-3) / 1e12, 2)
    return out


def roofline_fracs(w, res, peak):
    """Fraction of each direction's roofline: the larger of the time at the
    MFMA peak for its credited FLOP and the time at the HBM peak for its
    algorithmic bytes, over the measured time."""
    fb, bb = algo_bytes(w)
    out = {}
    t_f = max(w.fwd_flop() / (peak * 1e12), fb / (HBM_PEAK_GBS * 1e9))
    out["fwd_roofline_frac"] = round(t_f / (res["fwd_ms"] * 1e-3), 4)
    out["fwd_bound"] = "hbm" if fb / (HBM_PEAK_GBS * 1e9) > w.fwd_flop() / (peak * 1e12) else "mfma"
    if w.backward:
        t_b = max(w.bwd_flop() / (peak * 1e12), bb / (HBM_PEAK_GBS * 1e9))
        out["bwd_roofline_frac"] = round(t_b / (res["bwd_ms"] * 1e-3), 4)
        out["bwd_bound"] = "hbm" if bb / (HBM_PEAK_GBS * 1e9) > w.bwd_flop() / (peak * 1e12) else "mfma"
    out["fwd_algo_bytes"], out["bwd_algo_bytes"] = fb, (bb if w.backward else None)
    return out


# Workloads measured beside the default one in the same run: the DiT
# self-attention forward (its own >= 50% gate), the two DiT cross-attention
# shapes and the decoder shape against their rooflines, warm and with inputs
# rotated through more memory than the 256 MB last-level cache, and the
# float32 path (against the fp32 matrix peak).
EXTRA = [("dit_self", False), ("dit_cross_512", True), ("dit_cross_257", True),
         ("decoder_mha_causal", True), ("vae_attn_f32", False)]
ROTATE_BYTES = 1 << 30


def extra_workloads(dev, stream, steps: int, warmup: int):
    import torch

    from flash_attention_transformers_amd import workloads as W

    out = {}
    for name, rotate in EXTRA:
        w = W.WORKLOADS[name]
        peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
        run = DenseRun(w, dev, stream)
        sg, fg, _ = measure(run, steps, warmup)
        res = {"warm": summarize(w, sg, fg, peak)}
        res["warm"].update(roofline_fracs(w, res["warm"], peak))
        if rotate:
            copies = -(-ROTATE_BYTES // run.footprint())
            del run
            torch.cuda.empty_cache()
            run = DenseRun(w, dev, stream, copies=copies)
            sg, fg, _ = measure(run, steps, warmup)
            res["rotated"] = summarize(w, sg, fg, peak)
            res["rotated"].update(roofline_fracs(w, res["rotated"], peak))
            res["rotated"]["input_sets"] = copies
            res["rotated"]["rotated_bytes"] = copies * run.footprint()
        res["config"] = (f"B={w.B} Hq={w.Hq} Hkv={w.Hkv} Sq={w.Sq} Skv={w.Skv} D={w.D} "
                         f"causal={int(w.causal)} {w.dtype} "
                         + ("forward + backward" if w.backward else "forward only"))
        out[name] = res
        del run
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa_causal")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other workloads measured beside the default one")
    ap.add_argument("--copy-probe", action="store_true", help="run the HBM calibration copy")
    ap.add_argument("--gemm-probe", action="store_true", help="time the library bf16 GEMM")
    args = ap.parse_args()
    if args.copy_probe:
        copy_probe(max(args.steps, 1))
        return
    if args.gemm_probe:
        gemm_probe(max(args.steps, 1))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(attention heads shard across GPUs with no change to the kernel).", file=sys.stderr)
        sys.exit(2)

    import torch

    import flash_attention_transformers_amd as fa
    from flash_attention_transformers_amd import workloads as W

    if args.workload in W.PAGED_WORKLOADS:
        main_paged(args, W.PAGED_WORKLOADS[args.workload])
        return
    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    fa.load_library()
    stream = torch.cuda.current_stream(dev)
    clocks_before = read_clocks()
    run = DenseRun(w, dev, stream)
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS

    # Timed region: exactly `steps` steps in 3 consecutive groups, nothing
    # else on the stream; the figure is the median of the group means.
    during = []
    step_groups, fwd_groups, wall = measure(run, args.steps, args.warmup, clocks=during)
    res = summarize(w, step_groups, fwd_groups, peak)
    ms_step = res["ms_per_step"]
    # Per-kernel breakdown: the same number of steps again, with an event
    # between consecutive kernels.  Each event costs ~12 us of stream time at
    # a kernel boundary, so these steps run a little longer than the timed
    # ones; kernel_ms[k] is the span between the events around kernel k.
    kern_ms = run.kernel_ms(args.steps)
    clocks_after = read_clocks()

    fwd_flop = w.fwd_flop()
    step_flop = fwd_flop + (w.bwd_flop() if w.backward else 0.0)
    value = step_flop / (ms_step * 1e-3) / 1e12

    # Roofline of the kernel with the largest share of the step.
    F = fwd_flop
    per_launch = {"fwd": F, "dkdv": 2.0 * F, "dq": 1.5 * F}
    dom = max((n for n in run.names if n in per_launch), key=lambda n: kern_ms[n])
    kname = roofline_kernel(dom, w.dtype)
    achieved = per_launch[dom] / (kern_ms[dom] * 1e-3) / 1e12
    roofline = {
        "kernel": kname,
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": _traffic_from_profile(kname, w.name),
        "flop_per_launch": per_launch[dom],
    }
    line = {
        "metric": "attention TFLOPS fwd and fwd+bwd at 1 MI355X; % of bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1), resident in HBM)",
        "config": {
            "workload": f"{w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Sq={w.Sq} Skv={w.Skv} "
                        f"D={w.D} causal={int(w.causal)}; step = "
                        + ("forward + backward" if w.backward else "forward only"),
            "global_batch": w.B, "seq_len": w.Sq, "parallelism": "single GPU",
        },
        "timing": "the timed steps run as 3 consecutive groups with HIP events between them; "
                  "ms_per_step and fwd_ms are the medians of the group means (the forward "
                  "alone is timed the same way after the steps)",
        "pct_of_peak": round(100 * value / peak, 2),
        "fwd_tflops": res["fwd_tflops"],
        "fwd_pct_of_peak": res["fwd_pct_of_peak"],
        "bwd_tflops": res.get("bwd_tflops"),
        "bwd_pct_of_peak": res.get("bwd_pct_of_peak"),
        "fwd_ms": res["fwd_ms"],
        "bwd_ms": res.get("bwd_ms"),
        "step_group_ms": res["step_group_ms"],
        "fwd_group_ms": res["fwd_group_ms"],
        "kernel_ms_note": "per-kernel spans from a second pass of the same steps with an event "
                          "between kernels (about 12 us of event cost per kernel boundary)",
        "wall_s_timed_region": round(wall, 4),
        "kernel_ms": {n: round(t, 4) for n, t in kern_ms.items()},
        "clocks": {"before": clocks_before, "sclk_mhz_during_timed_steps": during[0],
                   "after": clocks_after,
                   "note": "amdsmi samples; before/after are read with the GPU idle, the "
                           "sample during the timed steps once they are all enqueued; the "
                           "effective clock per kernel (GRBM_GUI_ACTIVE over kernel time) is "
                           "in the counter summaries"},
        "roofline": roofline,
    }
    if not args.no_extra and args.workload == "gqa_causal":
        del run
        torch.cuda.empty_cache()
        line["workloads"] = extra_workloads(dev, stream, max(args.steps // 2, 6), args.warmup)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
