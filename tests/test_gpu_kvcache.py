"""GPU parity of the paged-KV-cache forward against the float64 oracle, plus
its behaviour: poisoned unused pages and tails, determinism, and agreement
with the dense forward.  All calls go through the C ABI."""
import numpy as np
import pytest

import flash_attention_transformers_amd as fa
import oracle
from flash_attention_transformers_amd import workloads as W

import harness as H

pytestmark = pytest.mark.gpu

TOL = H.TOL["bf16"]


@pytest.fixture(scope="module")
def dev():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    fa.load_library()
    return torch.device("cuda:0")


def run(t, causal, scale=None):
    import torch

    o, lse = fa.fwd_kvcache(t["q"], t["k_cache"], t["v_cache"], t["block_table"], t["seqlens"],
                            causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def compare(w, inp, o, lse, seqs=None):
    v = inp.vals
    seqs = range(w.B) if seqs is None else seqs
    for b in seqs:
        ro, rl = oracle.kvcache_forward(v["q"][b:b + 1], v["k_cache"], v["v_cache"],
                                        inp.block_table[b:b + 1], inp.seqlens[b:b + 1],
                                        w.causal, w.scale)
        go = H.to_np(o[b:b + 1])
        gl = lse[b:b + 1].cpu().numpy().astype(np.float64)
        # rows that see no key: O exactly 0 and LSE exactly -inf
        none = np.isneginf(rl)
        assert np.array_equal(np.isneginf(gl), none), b
        assert np.all(go[none] == 0), b
        fin = ~none
        res = dict(b=b, o_max_abs=H.max_abs(go, ro), o_rel_l2=H.rel_l2(go, ro),
                   lse_max_abs=H.max_abs(gl[fin], rl[fin]) if fin.any() else 0.0)
        H.say(f"    {res}")
        assert res["o_max_abs"] <= TOL["o_max_abs"], res
        assert res["o_rel_l2"] <= TOL["o_rel_l2"], res
        assert res["lse_max_abs"] <= TOL["lse_max_abs"], res


# (name, B, Hq, Hkv, Sq, D, page_size, seqlens, causal)
CASES = [
    ("decode_gqa_split", 4, 8, 2, 1, 128, 64, (1, 64, 200, 384), True),
    ("decode_mha_d64", 3, 4, 4, 1, 64, 128, (0, 77, 512), False),
    ("prefill_chunk", 2, 4, 2, 16, 128, 64, (16, 500), True),
    ("rows_without_keys", 1, 2, 1, 8, 128, 64, (5,), True),
    ("many_splits", 1, 8, 8, 1, 128, 64, (6300,), True),
    ("page128_offsets", 2, 4, 1, 4, 128, 128, (300, 640), True),
    ("two_query_chunks", 1, 32, 2, 16, 64, 64, (250,), True),
    ("noncausal_prefill_d64", 2, 6, 3, 5, 64, 64, (3, 129), False),
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[c[0] for c in CASES])
def test_kvcache_parity(idx, dev):
    name, B, Hq, Hkv, Sq, D, ps, lens, causal = CASES[idx]
    w = W.PagedWorkload(name, B, Hq, Hkv, Sq, D, ps, lens, causal, seed=100 + idx)
    H.say(f"[kvcache parity] {w}")
    inp = W.make_paged_inputs(w)
    t = W.paged_to_torch(inp, dev)
    o, lse = run(t, causal)
    compare(w, inp, o, lse)


def test_unused_pages_and_tails_are_never_read(dev):
    import torch

    w = W.PagedWorkload("poison", 3, 8, 2, 2, 128, 64, (100, 7, 257), True, seed=31, extra_pages=5)
    H.say(f"[kvcache poison] {w}")
    inp = W.make_paged_inputs(w)
    t = W.paged_to_torch(inp, dev)
    o_clean, l_clean = run(t, True)
    kc, vc = t["k_cache"].clone(), t["v_cache"].clone()
    used = set()
    for b, L in enumerate(w.seqlens):
        for tok in range(L, w.pages_per_seq * w.page_size):
            p = int(inp.block_table[b, tok // w.page_size])
            kc[p, :, tok % w.page_size] = float("nan")
            vc[p, :, tok % w.page_size] = float("nan")
        used.update(int(p) for p in inp.block_table[b, : -(-L // w.page_size)])
    for p in range(w.num_pages):
        if p not in used:
            kc[p] = float("nan")
            vc[p] = float("inf")
    t2 = dict(t, k_cache=kc, v_cache=vc)
    o, lse = run(t2, True)
    assert torch.equal(o.view(torch.int16), o_clean.view(torch.int16))
    assert torch.equal(lse, l_clean)


def test_kvcache_deterministic(dev):
    import torch

    w = W.PagedWorkload("det", 2, 8, 8, 1, 128, 64, (3000, 4100), True, seed=33)
    inp = W.make_paged_inputs(w)
    t = W.paged_to_torch(inp, dev)
    a = run(t, True)
    b = run(t, True)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


def test_kvcache_matches_dense_forward(dev):
    # Identity block table and full lengths: the cache is just a reshaped
    # dense K/V, so the paged result must agree with mattn_fwd.
    import torch

    B, Hq, Hkv, S, D, ps = 2, 8, 2, 256, 128, 64
    w = W.Workload("dense_ref", B, Hq, Hkv, S, S, D, True, "bf16", 35, False)
    t = W.to_torch(W.make_inputs(w), dev)
    o_d, l_d = fa.fwd(t["q"], t["k"], t["v"], causal=True)
    pps = S // ps
    kc = t["k"].view(B, Hkv, pps, ps, D).permute(0, 2, 1, 3, 4).reshape(B * pps, Hkv, ps, D).contiguous()
    vc = t["v"].view(B, Hkv, pps, ps, D).permute(0, 2, 1, 3, 4).reshape(B * pps, Hkv, ps, D).contiguous()
    bt = torch.arange(B * pps, dtype=torch.int32, device=dev).view(B, pps).contiguous()
    sl = torch.full((B,), S, dtype=torch.int32, device=dev)
    o, lse = fa.fwd_kvcache(t["q"], kc, vc, bt, sl, causal=True)
    torch.cuda.synchronize()
    assert H.max_abs(H.to_np(o), H.to_np(o_d)) <= 2e-2
    assert H.max_abs(lse.cpu().numpy(), l_d.cpu().numpy()) <= 1e-3


def test_decode_paged_workload_sampled(dev):
    # The benchmark's decode workload at full size, checked on two sequences.
    w = W.PAGED_WORKLOADS["decode_paged"]
    H.say(f"[kvcache sampled] {w}")
    inp = W.make_paged_inputs(w)
    t = W.paged_to_torch(inp, dev)
    o, lse = run(t, w.causal)
    compare(w, inp, o, lse, seqs=(0, w.B - 1))


def test_bad_page_ids_and_lengths_do_not_fault(dev):
    # Page ids outside [0, num_pages) read as zeros through an empty
    # descriptor, lengths are clamped to the table's capacity (negative ones
    # to 0); the other sequences are unaffected.
    import torch

    w = W.PagedWorkload("badmeta", 3, 4, 2, 1, 128, 64, (200, 150, 120), True, seed=41)
    inp = W.make_paged_inputs(w)
    t = W.paged_to_torch(inp, dev)
    o_ref, l_ref = run(t, True)
    bt = t["block_table"].clone()
    bt[1, 0] = -1
    bt[1, 1] = w.num_pages + 5
    sl = t["seqlens"].clone()
    sl[2] = -7
    t2 = dict(t, block_table=bt, seqlens=sl)
    o, lse = run(t2, True)
    assert torch.equal(o[0].view(torch.int16), o_ref[0].view(torch.int16))
    assert torch.equal(lse[0], l_ref[0])
    assert torch.isfinite(o[1].float()).all()
    assert (o[2].float() == 0).all() and torch.isneginf(lse[2]).all()
    # a length beyond the table's capacity is clamped to it
    sl3 = t["seqlens"].clone()
    sl3[0] = 10 ** 6
    o3, l3 = run(dict(t, seqlens=sl3), True)
    v = inp.vals
    ro, rl = oracle.kvcache_forward(v["q"][:1], v["k_cache"], v["v_cache"], inp.block_table[:1],
                                    [w.pages_per_seq * 64], True, w.scale)
    assert H.max_abs(H.to_np(o3[:1]), ro) <= TOL["o_max_abs"]


def test_kvcache_graph_replay_follows_device_lengths(dev):
    """mattn_fwd_kvcache captured into a HIP graph (every buffer allocated
    beforehand, the split workspace sized from the shapes alone), then
    replayed with new queries and new per-sequence lengths written into the
    captured buffers between replays, as a decode loop does: each replay
    gives the bits of an eager call on the same inputs, including a length
    of 0 (a row with no key)."""
    import torch

    w = W.PagedWorkload("graph", 3, 8, 2, 1, 128, 64, (700, 64, 1500), True, seed=37)
    H.say(f"[kvcache graph] {w}")
    t = W.paged_to_torch(W.make_paged_inputs(w), dev)
    q = t["q"].clone()
    sl = t["seqlens"].clone()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    need = fa.mattn_fwd_kvcache_workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.D, w.page_size,
                                               w.pages_per_seq)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def call(stream):
        fa.mattn_fwd_kvcache(q, t["k_cache"], t["v_cache"], t["block_table"], sl, o, lse, ws,
                             causal=True, scale=w.scale, stream=stream)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        call(side)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    gen = torch.Generator(device=dev).manual_seed(5)
    for rep, lens in enumerate([(700, 64, 1500), (701, 0, 1499), (1, 640, 1536)]):
        q.copy_(torch.randn(q.shape, generator=gen, device=dev).to(q.dtype))
        sl.copy_(torch.tensor(lens, dtype=torch.int32, device=dev))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ro, rl = fa.fwd_kvcache(q, t["k_cache"], t["v_cache"], t["block_table"], sl, causal=True,
                                scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ro.view(torch.int16)), f"replay {rep}: o"
        assert torch.equal(lse, rl), f"replay {rep}: lse"
