"""GPU parity of libmattn against the float64 oracle, called through the C ABI
(via the ctypes binding) on seeded inputs.

Every case compares every output element (O, LSE and, with a backward, dQ,
dK, dV) with the oracle, the five workloads included at their full sizes.
The one exception is the largest accepted query length, where rows at both
ends are compared and dK/dV are checked through sums that hold at any size.
"""
import numpy as np
import pytest

from flash_attention_transformers_amd import workloads as W

import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch

    import flash_attention_transformers_amd as fa

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    fa.load_library()
    return torch.device("cuda:0")


def wl(name, B, Hq, Hkv, Sq, Skv, D, causal, dtype="bf16", seed=5, backward=True):
    return W.Workload(name, B, Hq, Hkv, Sq, Skv, D, causal, dtype, seed, backward)


SMALL = [
    wl("nc_d128_ragged", 1, 2, 2, 300, 257, 128, False),
    wl("nc_d64_ragged", 2, 2, 1, 130, 70, 64, False),
    wl("causal_d64_misaligned", 1, 3, 3, 200, 200, 64, True),
    wl("causal_d128_gqa4", 1, 8, 2, 320, 320, 128, True),
    wl("causal_bottom_right", 1, 2, 2, 100, 300, 128, True),
    wl("causal_bottom_right_d64", 2, 2, 2, 33, 190, 64, True),
    wl("one_key", 1, 2, 2, 70, 1, 128, False),
    wl("seventeen_keys", 1, 2, 1, 129, 17, 64, False),
    wl("one_query", 1, 2, 2, 1, 200, 128, False),
    wl("decode_row_causal", 1, 4, 2, 1, 300, 128, True),
    wl("split_q_chunks", 1, 2, 2, 1000, 257, 128, False),
    wl("split_q_chunks_gqa", 1, 4, 2, 1100, 130, 64, False),
    wl("f32_d64", 1, 2, 2, 128, 128, 64, False, dtype="f32"),
    wl("f32_d128_causal_gqa", 1, 4, 2, 150, 150, 128, True, dtype="f32"),
    wl("f32_ragged_cross", 2, 2, 1, 70, 33, 64, False, dtype="f32"),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_parity_small(w, dev):
    H.check_full(w, dev)


def test_parity_tiny_f32_workload(dev):
    H.check_full(W.WORKLOADS["tiny_mha_f32"], dev)


# The float32 path on the fp32 matrix cores, at shapes that take each of its
# workgroup sizes (4, 2 and 1 waves of 32 rows or keys; f32_waves in
# attn_f32.hip picks them from the row or key count), with ragged tails,
# grouped heads, bottom-right causal masking and a short, tile-misaligned key
# range.  Forward and dQ / dK-dV waves per workgroup: 4/4, 4/2, 2/1, 1/1, 1/1.
F32 = [
    wl("f32_w4_noncausal_d64", 2, 8, 8, 4100, 4200, 64, False, dtype="f32"),
    wl("f32_w4_w2_causal_gqa_d128", 1, 4, 2, 8200, 8200, 128, True, dtype="f32"),
    wl("f32_w2_w1_causal_gqa_d128", 1, 4, 2, 6000, 6000, 128, True, dtype="f32"),
    wl("f32_bottom_right_d128", 1, 3, 1, 77, 301, 128, True, dtype="f32"),
    wl("f32_cross_257_d128", 1, 4, 4, 2000, 257, 128, False, dtype="f32"),
]


@pytest.mark.parametrize("w", F32, ids=[w.name for w in F32])
def test_parity_f32_matrix_path(w, dev):
    H.check_full(w, dev)


# The five workloads (and the float32 VAE-frame one) at full size, every element.
@pytest.mark.parametrize("name", ["decoder_mha_causal", "gqa_causal", "dit_self", "dit_cross_512",
                                  "dit_cross_257", "vae_attn_f32"])
def test_parity_workload_full(name, dev):
    w = W.WORKLOADS[name]
    H.check_full(w, dev, backward=w.backward)


# Shapes large enough to take the eight-wave forward workgroups: two query
# heads of one KV head per workgroup (even group sizes, causal with the
# diagonal off the tile grid, and non-causal), four heads of 64 rows (causal,
# group size 4, 520 workgroups), and 256 rows of one head (non-causal, one
# query head per KV head).  Query and key lengths are ragged.
W8 = [
    wl("w8_head_pairs_causal", 1, 16, 4, 8100, 8292, 128, True, backward=False),
    wl("w8_head_quads_causal", 1, 32, 8, 4100, 4200, 128, True, backward=False),
    wl("w8_head_pairs_noncausal_g2", 1, 16, 8, 8100, 2100, 128, False, backward=False),
    wl("w8_rows256_noncausal", 1, 16, 16, 8000, 2100, 128, False, backward=False),
]


@pytest.mark.parametrize("w", W8, ids=[w.name for w in W8])
def test_parity_eight_wave_forward(w, dev):
    H.check_full(w, dev, backward=False)


# Short key sequences at D = 128 under many query rows, forward only: grouped
# KV heads with a ragged last query tile, one key tile (64 keys), a single
# key (a walk of one tile whose softmax is exactly 1) and eight full tiles.
SHORT_KV = [
    wl("short_kv_gqa4_ragged_300", 1, 32, 8, 2100, 300, 128, False, backward=False),
    wl("short_kv_one_tile_64", 2, 16, 16, 2000, 64, 128, False, backward=False),
    wl("short_kv_single_key", 1, 64, 64, 1030, 1, 128, False, backward=False),
    wl("short_kv_eight_tiles_512", 4, 8, 2, 2048, 512, 128, False, backward=False),
]


@pytest.mark.parametrize("w", SHORT_KV, ids=[w.name for w in SHORT_KV])
def test_parity_short_kv_forward(w, dev):
    H.check_full(w, dev, backward=False)


# Large query groups: multi-query attention (group of 16 on one KV head,
# causal), a group of 8 at D = 64 with ragged lengths, a group of 8 large
# enough for the eight-wave four-head forward (two workgroups per KV head)
# with its backward, and a group of 16 on the split short-KV backward.  The
# dK/dV kernel sums each KV head's whole group in registers.
GROUPS = [
    wl("mqa_g16_causal", 1, 16, 1, 300, 300, 128, True),
    wl("g8_d64_ragged", 2, 16, 2, 200, 457, 64, False),
    wl("g8_w8_head_quads_causal", 1, 32, 4, 4100, 4100, 128, True),
    wl("g16_split_short_kv", 1, 16, 1, 1500, 200, 128, False),
]


@pytest.mark.parametrize("w", GROUPS, ids=[w.name for w in GROUPS])
def test_parity_large_groups(w, dev):
    H.check_full(w, dev, backward=w.backward)


# Backward on a long GQA shape (group size 2) with ragged lengths and the
# causal diagonal off the tile grid.
def test_parity_long_gqa_backward(dev):
    H.check_full(wl("gqa2_causal_ragged_long", 1, 32, 16, 4000, 4100, 128, True), dev)


def _random_shapes(n, seed):
    """Seeded small shapes spanning the parameter space: batch, group size,
    head dim, ragged and one-row/one-key lengths, causal (Skv >= Sq) or not,
    bf16 mostly and some fp32."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.choice([1, 2, 4]))
        Hkv = int(rng.integers(1, 4))
        D = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        Sq = int(rng.choice([1, int(rng.integers(2, 70)), int(rng.integers(70, 400))]))
        Skv = int(rng.choice([1, int(rng.integers(2, 70)), int(rng.integers(70, 400))]))
        if causal and Skv < Sq:
            Sq, Skv = Skv, Sq
        dtype = "f32" if i % 6 == 5 else "bf16"
        out.append(wl(f"rand{i}_G{G}_D{D}_{'c' if causal else 'n'}_{Sq}x{Skv}_{dtype}",
                      int(rng.integers(1, 3)), Hkv * G, Hkv, Sq, Skv, D, causal,
                      dtype=dtype, seed=100 + i))
    return out


RANDOM = _random_shapes(24, 20261202)


@pytest.mark.parametrize("w", RANDOM, ids=[w.name for w in RANDOM])
def test_parity_random_shapes(w, dev):
    H.check_full(w, dev)


def test_parity_max_query_rows(dev):
    """The longest query range the boundary accepts for one head at D = 128
    (a tensor of 2^31 - 128 elements, so byte offsets inside the head reach
    2^32 - 256), forward and backward.  Inputs are drawn on the GPU from a
    seeded torch generator (N(0,1), rounded to bf16); rows at the start and
    at the very end are compared with the oracle: O, LSE and dQ (each row's
    dQ depends only on its own row and on K/V when attention is
    non-causal).  dK and dV sum over all 2^24 rows, so they are checked
    through two identities that hold at any size (attention is non-causal,
    so every row sees every key): each row of P sums to one, hence
    sum_j dV_j = sum_i dO_i, and each row of dS sums to zero, hence
    sum_j dK_j = 0, each within the gradient tolerance relative to the norm
    of the tensor it checks."""
    import torch

    import flash_attention_transformers_amd as fa

    D, Skv = 128, 100
    Sq = (1 << 31) // D - 1
    gen = torch.Generator(device=dev).manual_seed(31)

    def draw(n):
        return torch.randn(1, 1, n, D, generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)

    q, k, v, do = draw(Sq), draw(Skv), draw(Skv), draw(Sq)
    scale = D ** -0.5
    o, lse = fa.fwd(q, k, v, causal=False, scale=scale)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=False, scale=scale)
    torch.cuda.synchronize()
    rows = torch.tensor(list(range(0, 64)) + list(range(Sq - 200, Sq)), device=dev)

    def pick(t):
        return t[0, 0].index_select(0, rows).float().cpu().numpy().astype(np.float64)

    qs, dos, go, gdq = pick(q), pick(do), pick(o), pick(dq)
    glse = lse[0, 0].index_select(0, rows).cpu().numpy().astype(np.float64)
    kk = k[0, 0].float().cpu().numpy().astype(np.float64)
    vv = v[0, 0].float().cpu().numpy().astype(np.float64)
    gdk = dk[0, 0].float().cpu().numpy().astype(np.float64)
    gdv = dv[0, 0].float().cpu().numpy().astype(np.float64)
    do_sum = np.zeros(D)
    for c0 in range(0, Sq, 1 << 20):
        do_sum += do[0, 0, c0:c0 + (1 << 20)].float().sum(0).double().cpu().numpy()
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    ro, rlse = H.oracle.forward_head(qs, kk, vv, False, scale)
    rdq, _, _, _ = H.oracle.backward_head(qs, kk, vv, dos, False, scale)
    tol = H.TOL["bf16"]
    res = dict(o_max_abs=H.max_abs(go, ro), o_rel_l2=H.rel_l2(go, ro),
               lse_max_abs=H.max_abs(glse, rlse), dq=H.rel_l2(gdq, rdq),
               dv_sum=float(np.linalg.norm(gdv.sum(0) - do_sum) / np.linalg.norm(do_sum)),
               dk_sum=float(np.linalg.norm(gdk.sum(0)) / np.linalg.norm(gdk)))
    H.say(f"[parity max rows] Sq={Sq} {res}")
    H.RESULTS.append(("max_query_rows", "rows at both ends; dK/dV sums", res))
    assert res["o_max_abs"] <= tol["o_max_abs"], res
    assert res["o_rel_l2"] <= tol["o_rel_l2"], res
    assert res["lse_max_abs"] <= tol["lse_max_abs"], res
    assert res["dq"] <= tol["grad_rel_l2"], res
    assert res["dv_sum"] <= tol["grad_rel_l2"], res
    assert res["dk_sum"] <= tol["grad_rel_l2"], res
