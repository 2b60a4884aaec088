"""Pins for the paged-KV-cache oracle (no GPU needed).

The paged forward is the dense oracle (pinned in test_oracle.py) applied to
each sequence's gathered, length-cut K/V.  These checks tie the gather and
the length handling to cases whose answer is fixed independently: a cache
that is just a reshaped dense K/V, page permutations, poisoned tokens past
the effective length, the decode row equal to the last causal row, empty
sequences, and a brute-force per-row softmax.  A planted mistake (using the
allocated length instead of the effective one) must fail a pin.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import kvcache as OK


def paged_case(B, Hq, Hkv, Sq, D, page_size, pages_per_seq, seqlens, seed, extra_pages=3):
    """Random q and a cache whose pages are handed out in a shuffled order."""
    r = np.random.default_rng(seed)
    num_pages = B * pages_per_seq + extra_pages
    q = r.standard_normal((B, Hq, Sq, D))
    kc = r.standard_normal((num_pages, Hkv, page_size, D))
    vc = r.standard_normal((num_pages, Hkv, page_size, D))
    perm = r.permutation(num_pages)
    bt = perm[:B * pages_per_seq].reshape(B, pages_per_seq)
    return q, kc, vc, bt, np.asarray(seqlens)


def dense_from_pages(cache, bt_row, L):
    return np.concatenate([cache[p] for p in bt_row], axis=1)[:, :L]


def test_identity_table_full_length_is_dense_attention():
    B, Hq, Hkv, Sq, D, ps, pps = 2, 4, 2, 6, 8, 4, 3
    r = np.random.default_rng(1)
    q = r.standard_normal((B, Hq, Sq, D))
    k = r.standard_normal((B, Hkv, ps * pps, D))
    v = r.standard_normal((B, Hkv, ps * pps, D))
    # cache page b*pps + p holds tokens [p*ps, (p+1)*ps) of sequence b
    kc = k.reshape(B, Hkv, pps, ps, D).transpose(0, 2, 1, 3, 4).reshape(B * pps, Hkv, ps, D)
    vc = v.reshape(B, Hkv, pps, ps, D).transpose(0, 2, 1, 3, 4).reshape(B * pps, Hkv, ps, D)
    bt = np.arange(B * pps).reshape(B, pps)
    for causal in (False, True):
        o, lse = OK.kvcache_forward(q, kc, vc, bt, [ps * pps] * B, causal, 0.3)
        ro, rl = oracle.attention_forward(q, k, v, causal, 0.3)
        np.testing.assert_array_equal(o, ro)
        np.testing.assert_array_equal(lse, rl)


def test_page_permutation_and_poisoned_tail():
    B, Hq, Hkv, Sq, D, ps, pps = 3, 4, 2, 5, 8, 4, 4
    lens = [13, 16, 1]
    q, kc, vc, bt, sl = paged_case(B, Hq, Hkv, Sq, D, ps, pps, lens, 2)
    ref_o, ref_l = OK.kvcache_forward(q, kc, vc, bt, sl, True, 0.25)
    # tokens past each sequence's length, and pages nobody lists, are never read
    kc2, vc2 = kc.copy(), vc.copy()
    used = set()
    for b, L in enumerate(lens):
        for t in range(L, ps * pps):
            kc2[bt[b, t // ps], :, t % ps] = np.nan
            vc2[bt[b, t // ps], :, t % ps] = np.nan
        used.update(int(p) for p in bt[b, : -(-L // ps)])
    for p in range(kc.shape[0]):
        if p not in used:
            kc2[p], vc2[p] = np.inf, np.nan
    o, lse = OK.kvcache_forward(q, kc2, vc2, bt, sl, True, 0.25)
    np.testing.assert_array_equal(o, ref_o)
    np.testing.assert_array_equal(lse, ref_l)
    # against the dense oracle on each sequence's truncated K/V
    for b, L in enumerate(lens):
        ro, rl = oracle.attention_forward(q[b:b + 1], dense_from_pages(kc, bt[b], L)[None],
                                          dense_from_pages(vc, bt[b], L)[None], True, 0.25)
        np.testing.assert_allclose(o[b], ro[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], rl[0], rtol=0, atol=1e-14)


def test_decode_row_is_last_causal_row():
    # Sq = 1 against L cached tokens equals the last row of causal attention
    # of L queries over the same keys (query L-1 sees every key).
    Hq, Hkv, D, ps, L = 4, 2, 8, 4, 11
    r = np.random.default_rng(3)
    qfull = r.standard_normal((1, Hq, L, D))
    k = r.standard_normal((1, Hkv, L, D))
    v = r.standard_normal((1, Hkv, L, D))
    pps = -(-L // ps)
    pad = pps * ps - L
    kp = np.concatenate([k, np.zeros((1, Hkv, pad, D))], axis=2)
    vp = np.concatenate([v, np.zeros((1, Hkv, pad, D))], axis=2)
    kc = kp.reshape(Hkv, pps, ps, D).transpose(1, 0, 2, 3)
    vc = vp.reshape(Hkv, pps, ps, D).transpose(1, 0, 2, 3)
    bt = np.arange(pps)[None]
    full_o, full_l = oracle.attention_forward(qfull, k, v, True, 0.2)
    for causal in (True, False):
        o, lse = OK.kvcache_forward(qfull[:, :, -1:], kc, vc, bt, [L], causal, 0.2)
        np.testing.assert_allclose(o[0, :, 0], full_o[0, :, -1], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[0, :, 0], full_l[0, :, -1], rtol=0, atol=1e-14)


def test_empty_and_short_sequences():
    B, Hq, Hkv, Sq, D, ps, pps = 2, 2, 1, 4, 8, 4, 2
    q, kc, vc, bt, _ = paged_case(B, Hq, Hkv, Sq, D, ps, pps, [0, 2], 4)
    o, lse = OK.kvcache_forward(q, kc, vc, bt, [0, 2], True, 0.5)
    # no keys at all: O = 0, LSE = -inf
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    # causal with L = 2 < Sq = 4: rows 0, 1 see nothing; row 2 sees key 0,
    # row 3 sees keys 0 and 1
    assert np.all(o[1, :, :2] == 0) and np.all(np.isneginf(lse[1, :, :2]))
    k0 = kc[bt[1, 0], 0, 0]
    np.testing.assert_allclose(o[1, :, 2], np.broadcast_to(vc[bt[1, 0], 0, 0], (Hq, D)), atol=1e-15)
    np.testing.assert_allclose(lse[1, :, 2], 0.5 * q[1, :, 2] @ k0, atol=1e-14)


def test_brute_force_rows():
    # Per-row softmax written out with math.exp over the gathered keys.
    B, Hq, Hkv, Sq, D, ps, pps = 2, 4, 2, 3, 5, 4, 3
    lens = [9, 5]
    q, kc, vc, bt, sl = paged_case(B, Hq, Hkv, Sq, D, ps, pps, lens, 5)
    o, lse = OK.kvcache_forward(q, kc, vc, bt, sl, True, 0.37)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        for h in range(Hq):
            for i in range(Sq):
                keys = [t for t in range(L) if t <= i + L - Sq]
                s = []
                for t in keys:
                    kt = kc[bt[b, t // ps], h // G, t % ps]
                    s.append(0.37 * sum(q[b, h, i, d] * kt[d] for d in range(D)))
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = sum(w)
                want = [sum(w[n] * vc[bt[b, keys[n] // ps], h // G, keys[n] % ps][d]
                            for n in range(len(keys))) / tot for d in range(D)]
                np.testing.assert_allclose(o[b, h, i], want, rtol=1e-12, atol=1e-13)
                assert abs(lse[b, h, i] - (m + math.log(tot))) < 1e-12


def test_planted_allocated_length_mistake_fails():
    B, Hq, Hkv, Sq, D, ps, pps = 1, 2, 1, 2, 8, 4, 3
    q, kc, vc, bt, sl = paged_case(B, Hq, Hkv, Sq, D, ps, pps, [6], 6)

    def wrong(q, kc, vc, bt, sl, causal, scale):
        return OK.kvcache_forward(q, kc, vc, bt, [ps * pps] * len(sl), causal, scale)

    ref = oracle.attention_forward(q, dense_from_pages(kc, bt[0], 6)[None],
                                   dense_from_pages(vc, bt[0], 6)[None], True, 0.3)
    good = OK.kvcache_forward(q, kc, vc, bt, sl, True, 0.3)
    bad = wrong(q, kc, vc, bt, sl, True, 0.3)
    np.testing.assert_allclose(good[0], ref[0], atol=1e-14)
    with pytest.raises(AssertionError):
        np.testing.assert_allclose(bad[0], ref[0], atol=1e-6)
