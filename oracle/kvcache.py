"""CPU float64 oracle for attention over a paged KV cache (decode and chunked
prefill).

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests and ``bench.py``'s ``cpu_baseline`` leg may call it.  It shares no
code with the HIP path.

The cache holds fixed-size pages; a sequence's keys and values are the first
``seqlens_k[b]`` tokens of the pages its block-table row lists, in that
order.  Two readings come from the pages:

* the keys attended to are exactly the sequence's *effective* length, not
  the allocated buffer behind it: the LingBot report's FA2/FA3 comparison
  (section on same-card hardware counters) had to redo its float64
  reference after counting the padding region, and its per-call length
  supplement shows the allocated length overstating the work by about 41%;
* decoding one token against cached K/V is the last row of full causal
  attention (xtrain evolution page, milestone M2a of the decode engine).

So the oracle gathers each sequence's pages into a dense [Hkv, L, D] block,
cuts it at L = seqlens_k[b], and hands it to the dense oracle, with the
causal mask aligned bottom-right against L (query i of Sq sees key j iff
j <= i + L - Sq).  Rows that see no key get O = 0 and LSE = -inf.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_forward


def gather_kv(cache, pages, seqlen: int) -> np.ndarray:
    """Dense [Hkv, seqlen, D] float64 block of one sequence.

    cache: [num_pages, Hkv, page_size, D]; pages: that sequence's block-table
    row (page ids in token order)."""
    cache = np.asarray(cache)
    page_size = cache.shape[2]
    n = -(-seqlen // page_size)  # pages that hold the sequence's tokens
    if n == 0:
        return np.zeros((cache.shape[1], 0, cache.shape[3]))
    blocks = [np.asarray(cache[int(p)], dtype=np.float64) for p in pages[:n]]
    return np.concatenate(blocks, axis=1)[:, :seqlen]


def kvcache_forward(q, k_cache, v_cache, block_table, seqlens_k, causal: bool, scale: float):
    """q: [B,Hq,Sq,D]; k_cache/v_cache: [num_pages,Hkv,page_size,D];
    block_table: [B, pages_per_seq] int; seqlens_k: [B] int.
    -> O [B,Hq,Sq,D], LSE [B,Hq,Sq] (float64)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Sq, D = q.shape
    o = np.zeros((B, Hq, Sq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        L = int(seqlens_k[b])
        kb = gather_kv(k_cache, block_table[b], L)
        vb = gather_kv(v_cache, block_table[b], L)
        o[b:b + 1], lse[b:b + 1] = attention_forward(q[b:b + 1], kb[None], vb[None], causal, scale)
    return o, lse
