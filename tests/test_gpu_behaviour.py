"""GPU behaviour beyond parity: determinism, NaN-poisoned tails and guard
words, GQA versus repeated-KV MHA, invariants, rejection and empty problems.
All calls go through the C ABI."""
import math

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


def fwd_bwd(t, causal, scale=None):
    o, lse = fa.fwd(t["q"], t["k"], t["v"], causal=causal, scale=scale)
    dq, dk, dv = fa.bwd(t["q"], t["k"], t["v"], o, lse, t["do"], causal=causal, scale=scale)
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)


@pytest.mark.parametrize("shape", [(2, 8, 2, 700, 700, 128, True), (1, 4, 4, 2000, 200, 128, False),
                                   (2, 4, 4, 300, 300, 64, True)])
def test_bitwise_determinism(shape, dev):
    import torch

    B, Hq, Hkv, Sq, Skv, D, causal = shape
    H.say(f"[determinism] {shape}")
    w = W.Workload("det", B, Hq, Hkv, Sq, Skv, D, causal, "bf16", 9, True)
    t = W.to_torch(W.make_inputs(w), dev)
    a = fwd_bwd(t, causal)
    b = fwd_bwd(t, causal)
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n].view(torch.int16) if a[n].dtype == torch.bfloat16 else a[n],
                           b[n].view(torch.int16) if b[n].dtype == torch.bfloat16 else b[n]), n


def _poisoned(t, pad):
    """Copy t into the middle of a NaN-filled buffer; return (view, buffer)."""
    import torch

    n = t.numel()
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=t.dtype, device=t.device)
    buf[pad:pad + n] = t.reshape(-1)
    return buf[pad:pad + n].view(t.shape), buf


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_nan_poisoned_tails_and_guards(dtype, D, dev):
    import torch

    H.say(f"[nan guards] {dtype} D={D}")
    w = W.Workload("guard", 1, 2, 1, 131, 257, D, False, dtype, 11, True)
    t = W.to_torch(W.make_inputs(w), dev)
    clean = fwd_bwd(t, False)
    pad = 4096  # elements of NaN before and after every input
    tp, bufs = {}, []
    for n in ("q", "k", "v", "do"):
        tp[n], buf = _poisoned(t[n], pad)
        bufs.append(buf)
    # outputs: NaN-prefilled with NaN guard regions on both sides
    outs = {}
    for n, like in (("o", t["q"]), ("dq", t["q"]), ("dk", t["k"]), ("dv", t["v"])):
        outs[n] = _poisoned(torch.full_like(like, float("nan")), pad)
    lse_v, lse_buf = _poisoned(torch.full((1, 2, 131), float("nan"), device=dev), pad)
    fa.mattn_fwd(tp["q"], tp["k"], tp["v"], outs["o"][0], lse_v, False, None)
    ws = fa.bwd_workspace(tp["q"], tp["k"])
    ws.fill_(255)  # contents on entry must not matter
    fa.mattn_bwd(tp["q"], tp["k"], tp["v"], outs["o"][0], lse_v, tp["do"], outs["dq"][0],
                 outs["dk"][0], outs["dv"][0], ws, False, None)
    torch.cuda.synchronize()
    for n in ("o", "dq", "dk", "dv"):
        view, buf = outs[n]
        assert torch.isfinite(view).all(), n
        a, b = view, clean[n]
        if a.dtype == torch.bfloat16:
            a, b = a.view(torch.int16), b.view(torch.int16)
        assert torch.equal(a, b), n
        assert torch.isnan(buf[:pad]).all() and torch.isnan(buf[-pad:]).all(), f"guard {n}"
    assert torch.equal(lse_v, clean["lse"])
    assert torch.isnan(lse_buf[:pad]).all() and torch.isnan(lse_buf[-pad:]).all()


def test_gqa_matches_repeated_kv(dev):
    import torch

    H.say("[gqa vs repeated kv]")
    G = 4
    w = W.Workload("gqa", 2, 8, 2, 260, 260, 128, True, "bf16", 13, True)
    t = W.to_torch(W.make_inputs(w), dev)
    a = fwd_bwd(t, True)
    tr = dict(t)
    tr["k"] = t["k"].repeat_interleave(G, dim=1).contiguous()
    tr["v"] = t["v"].repeat_interleave(G, dim=1).contiguous()
    b = fwd_bwd(tr, True)
    torch.cuda.synchronize()
    # the forward of a query head does identical arithmetic either way
    assert torch.equal(a["o"].view(torch.int16), b["o"].view(torch.int16))
    assert torch.equal(a["lse"], b["lse"])
    assert torch.equal(a["dq"].view(torch.int16), b["dq"].view(torch.int16))
    for n in ("dk", "dv"):
        summed = b[n].float().view(2, 2, G, 260, 128).sum(2)
        assert H.rel_l2(a[n].float().cpu().numpy(), summed.cpu().numpy().astype(np.float64)) < 1e-2, n


def test_gradient_sum_invariants(dev):
    # sum_j dK_j = 0 and sum_j dV_j = sum over the group's query rows of dO
    H.say("[invariants]")
    w = W.Workload("inv", 1, 4, 2, 256, 256, 64, True, "bf16", 17, True)
    inp = W.make_inputs(w)
    t = W.to_torch(inp, dev)
    g = fwd_bwd(t, True)
    dk = g["dk"].float().cpu().numpy().astype(np.float64)
    dv = g["dv"].float().cpu().numpy().astype(np.float64)
    s_dk = dk.sum(2)
    assert np.abs(s_dk).max() <= 2e-2 * np.abs(dk).sum(2).max()
    want = inp.vals["do"].astype(np.float64).reshape(1, 2, 2, 256, 64).sum((2, 3))
    assert np.abs(dv.sum(2) - want).max() <= 2e-2 * np.abs(want).max()


def test_rejection_leaves_outputs_untouched(dev):
    import torch

    H.say("[rejection]")
    q = torch.randn(1, 3, 64, 64, device=dev, dtype=torch.bfloat16)
    k = torch.randn(1, 2, 64, 64, device=dev, dtype=torch.bfloat16)  # 3 % 2 != 0
    o = torch.full_like(q, float("nan"))
    lse = torch.full((1, 3, 64), float("nan"), device=dev)
    with pytest.raises(fa.MattnError) as e:
        fa.mattn_fwd(q, k, k, o, lse)
    assert e.value.status == fa.MATTN_ERR_INVALID_ARG
    q96 = torch.randn(1, 2, 64, 96, device=dev, dtype=torch.bfloat16)
    with pytest.raises(fa.MattnError) as e:
        fa.fwd(q96, q96, q96)
    assert e.value.status == fa.MATTN_ERR_UNSUPPORTED
    qc = torch.randn(1, 2, 65, 64, device=dev, dtype=torch.bfloat16)
    kc = torch.randn(1, 2, 64, 64, device=dev, dtype=torch.bfloat16)
    oc = torch.full_like(qc, float("nan"))
    lc = torch.full((1, 2, 65), float("nan"), device=dev)
    with pytest.raises(fa.MattnError) as e:
        fa.mattn_fwd(qc, kc, kc, oc, lc, causal=True)
    assert e.value.status == fa.MATTN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all() and torch.isnan(lse).all()
    assert torch.isnan(oc.float()).all() and torch.isnan(lc).all()


def test_empty_problems(dev):
    import torch

    H.say("[empty]")
    q = torch.empty(0, 2, 16, 64, device=dev, dtype=torch.bfloat16)
    o, lse = fa.fwd(q, q, q)
    assert o.numel() == 0
    # no query rows: every key's gradient is zero
    q0 = torch.empty(1, 2, 0, 64, device=dev, dtype=torch.bfloat16)
    k = torch.randn(1, 2, 40, 64, device=dev, dtype=torch.bfloat16)
    o0 = torch.empty_like(q0)
    l0 = torch.empty(1, 2, 0, device=dev)
    dq = torch.empty_like(q0)
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(k, float("nan"))
    ws = torch.empty(256, dtype=torch.uint8, device=dev)
    fa.mattn_bwd(q0, k, k, o0, l0, q0, dq, dk, dv, ws)
    torch.cuda.synchronize()
    assert (dk.float() == 0).all() and (dv.float() == 0).all()


@pytest.mark.parametrize("shape", [(1, 2, 2, 150, 90, 64), (1, 16, 4, 4100, 257, 128)])
def test_negative_and_zero_scale(shape, dev):
    """A negative scale negates Q and a zero scale zeroes it inside the
    kernels, on a D=64 shape and a ragged D=128 one.  At D=128 the negative
    scale is -1/sqrt(D), the magnitude the bf16 O gate is set for: -0.3 there
    sharpens the softmax so far that |O| nears 4, where one bf16 step of the
    stored O is 1/64, and the forward lands at 0.0225."""
    B, Hq, Hkv, Sq, Skv, D = shape
    H.say(f"[scale sign] {shape}")
    for scale in (-0.3 if D == 64 else -D ** -0.5, 0.0):
        for dtype in ("bf16", "f32"):
            if dtype == "f32" and D == 128:
                continue
            w = W.Workload("scale", B, Hq, Hkv, Sq, Skv, D, False, dtype, 19, True)
            inp = W.make_inputs(w)
            t = W.to_torch(inp, dev)
            g = fwd_bwd(t, False, scale=scale)
            import oracle

            v = inp.vals
            ro, _ = oracle.attention_forward(v["q"], v["k"], v["v"], False, scale)
            rdq, rdk, rdv, _ = oracle.attention_backward(v["q"], v["k"], v["v"], v["do"], False, scale)
            tol = H.TOL[dtype]
            assert H.max_abs(H.to_np(g["o"]), ro) <= tol["o_max_abs"]
            assert H.rel_l2(H.to_np(g["dv"]), rdv) <= tol["grad_rel_l2"]
            if scale != 0.0:
                assert H.rel_l2(H.to_np(g["dq"]), rdq) <= tol["grad_rel_l2"]
                assert H.rel_l2(H.to_np(g["dk"]), rdk) <= tol["grad_rel_l2"]
            else:
                assert np.abs(H.to_np(g["dq"])).max() == 0 and np.abs(H.to_np(g["dk"])).max() == 0


def _bwd_noalloc(lib, t, o, lse, dq, dk, dv, w, stream):
    import ctypes

    vp = ctypes.c_void_p
    return lib.mattn_bwd_noalloc(
        vp(t["q"].data_ptr()), vp(t["k"].data_ptr()), vp(t["v"].data_ptr()), vp(o.data_ptr()),
        vp(lse.data_ptr()), vp(t["do"].data_ptr()), vp(dq.data_ptr()), vp(dk.data_ptr()),
        vp(dv.data_ptr()), w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, int(w.causal),
        ctypes.c_float(w.scale), 0, vp(stream))


@pytest.mark.parametrize("shape", [(1, 8, 2, 700, 700, 128, True), (1, 4, 4, 1500, 257, 128, False)])
def test_graph_capture_replays(shape, dev):
    """mattn_fwd and mattn_bwd_noalloc captured into one HIP graph (torch's
    graph API; every tensor allocated beforehand; the calls enqueue kernels
    only), then replayed on three input sets that eager copies place in the
    captured buffers, with synchronisations between the replays: every
    replay gives the bits of eager mattn_fwd / mattn_bwd on the same inputs.
    The second shape takes the split short-KV backward (fp32 partials in the
    static scratch and their fixed-order reduction)."""
    import torch

    B, Hq, Hkv, Sq, Skv, D, causal = shape
    H.say(f"[graph] {shape}")
    wls = [W.Workload("graph", B, Hq, Hkv, Sq, Skv, D, causal, "bf16", s, True) for s in (31, 32, 33)]
    ins = [W.to_torch(W.make_inputs(w), dev) for w in wls]
    w = wls[0]
    static = {n: ins[0][n].clone() for n in ("q", "k", "v", "do")}
    o = torch.empty_like(static["q"])
    lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(static[n]) for n in ("q", "k", "v"))
    lib = fa.load_library()

    def run(stream):
        fa.mattn_fwd(static["q"], static["k"], static["v"], o, lse, causal=causal, scale=w.scale,
                     stream=stream)
        assert _bwd_noalloc(lib, static, o, lse, dq, dk, dv, w, stream.cuda_stream) == 0

    # Eager warm-up on a side stream; it also looks up the scratch array's
    # device address, so the capture itself makes no runtime queries of that.
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        run(side)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    for rep, t in enumerate(ins):
        for n in static:
            static[n].copy_(t[n])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = fwd_bwd(t, causal, scale=w.scale)
        torch.cuda.synchronize()
        got = dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv)
        for n in ref:
            a, b = got[n], ref[n]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"replay {rep}: {n}"


def test_concurrent_streams(dev):
    """Forward and backward of two problems enqueued on two streams at once,
    each with its own workspace, give the same bits as the same calls made
    one after the other: the library keeps no state shared between calls
    (the allocation-free backward's static scratch aside)."""
    import torch

    H.say("[two streams]")
    shapes = [(1, 8, 2, 900, 900, 128, True), (1, 4, 4, 1500, 257, 128, False)]
    wls = [W.Workload("streams", *s, "bf16", 61 + i, True) for i, s in enumerate(shapes)]
    ins = [W.to_torch(W.make_inputs(w), dev) for w in wls]
    ref = [fwd_bwd(t, w.causal, scale=w.scale) for t, w in zip(ins, wls)]
    torch.cuda.synchronize()
    outs = []
    for t in ins:
        o = torch.empty_like(t["q"])
        lse = torch.empty(t["q"].shape[:3], dtype=torch.float32, device=dev)
        outs.append(dict(o=o, lse=lse, dq=torch.empty_like(t["q"]), dk=torch.empty_like(t["k"]),
                         dv=torch.empty_like(t["v"]), ws=fa.bwd_workspace(t["q"], t["k"])))
    streams = [torch.cuda.Stream(device=dev) for _ in ins]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream(dev))
    for t, w, g, s in zip(ins, wls, outs, streams):
        fa.mattn_fwd(t["q"], t["k"], t["v"], g["o"], g["lse"], causal=w.causal, scale=w.scale,
                     stream=s)
    for t, w, g, s in zip(ins, wls, outs, streams):
        fa.mattn_bwd(t["q"], t["k"], t["v"], g["o"], g["lse"], t["do"], g["dq"], g["dk"], g["dv"],
                     g["ws"], causal=w.causal, scale=w.scale, stream=s)
    torch.cuda.synchronize()
    for i, (g, r) in enumerate(zip(outs, ref)):
        for n in r:
            a, b = g[n], r[n]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"problem {i}: {n}"


@pytest.mark.parametrize("shape", [(1, 8, 2, 300, 300, 128, True), (1, 2, 2, 1000, 257, 128, False),
                                   (1, 2, 2, 100, 70, 64, False)])
def test_stage_sequence_equals_bwd(shape, dev):
    """Preprocess, dK/dV and dQ enqueued separately give mattn_bwd's bits."""
    import torch

    B, Hq, Hkv, Sq, Skv, D, causal = shape
    H.say(f"[stages] {shape}")
    w = W.Workload("stages", B, Hq, Hkv, Sq, Skv, D, causal, "bf16", 23, True)
    t = W.to_torch(W.make_inputs(w), dev)
    ref = fwd_bwd(t, causal)
    dq, dk, dv = (torch.full_like(ref[n], float("nan")) for n in ("dq", "dk", "dv"))
    ws = fa.bwd_workspace(t["q"], t["k"])
    args = (t["q"], t["k"], t["v"], ref["o"], ref["lse"], t["do"], dq, dk, dv, ws)
    fa.mattn_bwd_stages(*args, fa.MATTN_BWD_PREPROCESS, causal)
    fa.mattn_bwd_stages(*args, fa.MATTN_BWD_DQ, causal)
    torch.cuda.synchronize()
    assert torch.isnan(dk.float()).all() and torch.isnan(dv.float()).all()  # not selected yet
    fa.mattn_bwd_stages(*args, fa.MATTN_BWD_DKDV, causal)
    torch.cuda.synchronize()
    for n, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.equal(x.view(torch.int16), ref[n].view(torch.int16)), n


@pytest.mark.parametrize("shape", [(2, 4, 2, 200, 260, 128, True, "bf16"),
                                   (1, 8, 2, 300, 257, 128, False, "bf16"),
                                   (1, 2, 2, 150, 90, 64, False, "f32"),
                                   (1, 4, 2, 130, 130, 128, True, "f32")])
def test_key_translation_invariance(shape, dev):
    """Adding one vector c to every key of a KV head leaves O, dQ, dK and dV
    unchanged (the softmax is shift-invariant per query row) and moves LSE_i
    by scale * <q_i, c>.  Keys and c are multiples of 1/8 with small
    magnitude, so k + c is exact in bf16 and both runs see exactly the
    translated problem.  Each output is compared between the two runs within
    its parity tolerance relative to the tensor's norm; LSE within twice its
    tolerance (each run carries its own error)."""
    import torch

    B, Hq, Hkv, Sq, Skv, D, causal, dtype = shape
    H.say(f"[key translation] {shape}")
    rng = np.random.default_rng(29)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def dev_t(a):
        return torch.from_numpy(np.asarray(a, np.float32)).to(dev).to(tdt).contiguous()

    q = dev_t(rng.standard_normal((B, Hq, Sq, D), dtype=np.float32))
    v = dev_t(rng.standard_normal((B, Hkv, Skv, D), dtype=np.float32))
    do = dev_t(rng.standard_normal((B, Hq, Sq, D), dtype=np.float32))
    k_np = rng.integers(-16, 17, size=(B, Hkv, Skv, D)).astype(np.float32) / 8
    c_np = rng.integers(-8, 9, size=(B, Hkv, 1, D)).astype(np.float32) / 8
    k, k2 = dev_t(k_np), dev_t(k_np + c_np)
    scale = D ** -0.5
    a = fwd_bwd(dict(q=q, k=k, v=v, do=do), causal, scale)
    b = fwd_bwd(dict(q=q, k=k2, v=v, do=do), causal, scale)
    torch.cuda.synchronize()
    tol = H.TOL[dtype]
    qh = q.float().cpu().numpy().astype(np.float64)
    shift = scale * np.einsum("bhsd,bhd->bhs", qh,
                              np.repeat(c_np[:, :, 0, :].astype(np.float64), Hq // Hkv, axis=1))
    lse_err = np.abs(H.to_np(b["lse"]) - H.to_np(a["lse"]) - shift).max()
    res = {"o_max_abs": H.max_abs(H.to_np(b["o"]), H.to_np(a["o"])),
           "o_rel_l2": H.rel_l2(H.to_np(b["o"]), H.to_np(a["o"])),
           "lse_shift_max_abs": float(lse_err)}
    for n in ("dq", "dk", "dv"):
        res[n] = H.rel_l2(H.to_np(b[n]), H.to_np(a[n]))
    H.say(f"    {res}")
    H.RESULTS.append((f"key_translation_{'x'.join(map(str, shape))}", "invariance", res))
    assert res["o_max_abs"] <= tol["o_max_abs"], res
    assert res["o_rel_l2"] <= tol["o_rel_l2"], res
    assert res["lse_shift_max_abs"] <= 2 * tol["lse_max_abs"], res
    for n in ("dq", "dk", "dv"):
        assert res[n] <= tol["grad_rel_l2"], (n, res)
