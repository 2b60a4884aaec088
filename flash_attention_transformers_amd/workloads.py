"""Seeded synthetic attention inputs and the five workload shapes.

This module holds no attention arithmetic: it only draws the inputs that both
the HIP path and the CPU checker consume, so that the two always see the same
values.

Recipe (the same for every workload):

* ``numpy.random.default_rng(seed)`` (PCG64), then ``standard_normal`` in
  float32, drawn in the order q, k, v, dO, each with its full BHSD shape.
* Optional per-tensor multipliers (the DiT self-attention workload scales q
  and k by float32(1/sqrt(2)) *before* rounding).
* For bf16 workloads every tensor is rounded to bfloat16 with
  round-to-nearest-even; the oracle receives exactly those rounded values
  upcast to float64, so input rounding is never counted as kernel error.

The shapes follow the decoder-training and DiT/world-model workloads of the
source pages: the LingBot pipeline report ("Attention: real inputs, backends,
error and timing" and the FA2/FA3 hardware-comparison sections: head dim 128,
a per-GPU share of 10 heads, 30x52 latent tokens per frame, text KV of 512)
and the xtrain evolution page (table row T14: head dim 64 decoder; row T15:
grouped KV heads).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    causal: bool
    dtype: str  # "bf16" or "f32"
    seed: int
    backward: bool
    qk_mult: float = 1.0  # multiplier applied to q and k before rounding

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def fwd_flop(self) -> float:
        """Credited forward work: 4*B*Hq*Sq*Skv*D, halved when causal."""
        f = 4.0 * self.B * self.Hq * self.Sq * self.Skv * self.D
        return f / 2 if self.causal else f

    def bwd_flop(self) -> float:
        """Credited backward work: 2.5x the credited forward work."""
        return 2.5 * self.fwd_flop()

    def with_shape(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny_mha_f32", 1, 2, 2, 128, 128, 64, False, "f32", 1, True),
        Workload("decoder_mha_causal", 8, 12, 12, 1024, 1024, 64, True, "bf16", 2, True),
        Workload("gqa_causal", 4, 32, 8, 4096, 4096, 128, True, "bf16", 3, True),
        Workload("dit_self", 1, 10, 10, 32760, 32760, 128, False, "bf16", 4, False,
                 qk_mult=1.0 / math.sqrt(2.0)),
        Workload("dit_cross_512", 1, 10, 10, 32760, 512, 128, False, "bf16", 51, True),
        Workload("dit_cross_257", 1, 10, 10, 32760, 257, 128, False, "bf16", 52, True),
        # float32 attention over the latent frames of one generated chunk of a
        # 480x832 video, the VAE's fp32 attention that the LingBot report's
        # kernel ledger names without printing its shape: each frame attends
        # over its own 60x104 tokens (before the 2x2 patches that give the
        # report's 30x52 DiT tokens per frame), a chunk is 3 latent frames
        # (the report's per-chunk 4680 = 3 x 1560 tokens) taken as the batch,
        # and the channel width is taken as 3 heads of 128.
        Workload("vae_attn_f32", 3, 3, 3, 6240, 6240, 128, False, "f32", 71, True),
    ]
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    Inputs here are finite normal draws; NaN/Inf are not produced by the
    generator and are not handled specially.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    # For finite x the sum stays below 2^32 (the largest finite pattern,
    # 0xFF7FFFFF, plus 0x8000), so 32-bit arithmetic is exact.
    rounded = bits + np.uint32(0x7FFF)
    rounded += (bits >> np.uint32(16)) & np.uint32(1)
    rounded >>= np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass
class Inputs:
    """Host copies of one seeded input set.

    ``vals`` holds float32 arrays with exactly the values the GPU sees (for
    bf16 workloads these are the rounded values); ``bits`` holds the raw
    bf16 bit patterns (uint16) for bf16 workloads, else None.
    """
    workload: Workload
    vals: Dict[str, np.ndarray]
    bits: Optional[Dict[str, np.ndarray]]


def make_inputs(w: Workload, seed: Optional[int] = None) -> Inputs:
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shapes = {
        "q": (w.B, w.Hq, w.Sq, w.D),
        "k": (w.B, w.Hkv, w.Skv, w.D),
        "v": (w.B, w.Hkv, w.Skv, w.D),
        "do": (w.B, w.Hq, w.Sq, w.D),
    }
    raw = {}
    for name in ("q", "k", "v", "do"):
        a = rng.standard_normal(shapes[name], dtype=np.float32)
        if name in ("q", "k") and w.qk_mult != 1.0:
            a = a * np.float32(w.qk_mult)
        raw[name] = a
    if w.dtype == "bf16":
        bits = {n: round_to_bf16_bits(a) for n, a in raw.items()}
        vals = {n: bf16_bits_to_f32(b) for n, b in bits.items()}
        return Inputs(w, vals, bits)
    return Inputs(w, raw, None)


def to_torch(inp: Inputs, device) -> Dict[str, "object"]:
    """Device tensors (torch) holding exactly ``inp``'s values."""
    import torch

    out = {}
    for n, a in inp.vals.items():
        if inp.bits is not None:
            t = torch.from_numpy(inp.bits[n].view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(a)
        out[n] = t.to(device).contiguous()
    return out


@dataclasses.dataclass(frozen=True)
class PagedWorkload:
    """Queries against a paged KV cache: B sequences of effective key counts
    ``seqlens``, each holding ceil(max(seqlens) / page_size) pages listed in a
    shuffled block table (so neighbouring tokens of a sequence live in
    scattered pages), plus ``extra_pages`` pages no sequence lists."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    D: int
    page_size: int
    seqlens: Tuple[int, ...]
    causal: bool
    seed: int
    extra_pages: int = 2

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def pages_per_seq(self) -> int:
        return max(1, -(-max(self.seqlens) // self.page_size))

    @property
    def num_pages(self) -> int:
        return self.B * self.pages_per_seq + self.extra_pages

    def fwd_flop(self) -> float:
        """Credited forward FLOP: 4*D per (query head, query, visible key),
        counting the key rectangle Sq x L per sequence, halved when causal
        and Sq > 1 (a decoded row sees every cached key)."""
        pairs = sum(self.Sq * L for L in self.seqlens)
        f = 4.0 * self.Hq * self.D * pairs
        return f / 2 if (self.causal and self.Sq > 1) else f

    def kv_bytes(self) -> float:
        """K and V bytes of the effective lengths (bf16): what a single pass
        has to read from HBM."""
        return 2.0 * 2 * self.Hkv * self.D * sum(self.seqlens)


def _seqlens(n: int, lo: int, hi: int, seed: int) -> Tuple[int, ...]:
    r = np.random.default_rng(seed)
    return tuple(int(x) for x in r.integers(lo, hi + 1, size=n))


# Decode against KV caches whose effective lengths span the pages' KV growth
# (4680 to 28080 keys per sequence, LingBot report, per-chunk work table),
# grouped KV heads as in the xtrain decoder (row T15).
PAGED_WORKLOADS: Dict[str, PagedWorkload] = {
    w.name: w
    for w in [
        PagedWorkload("decode_paged", 8, 32, 8, 1, 128, 64, _seqlens(8, 4680, 28080, 61), True, 62),
    ]
}


@dataclasses.dataclass
class PagedInputs:
    workload: PagedWorkload
    vals: Dict[str, np.ndarray]       # q, k_cache, v_cache: float32 with the bf16 values
    bits: Dict[str, np.ndarray]       # the same as bf16 bit patterns (uint16)
    block_table: np.ndarray           # [B, pages_per_seq] int32
    seqlens: np.ndarray               # [B] int32


def make_paged_inputs(w: PagedWorkload) -> PagedInputs:
    """PCG64(seed): standard_normal float32 drawn in the order q, k_cache,
    v_cache, rounded to bf16 (RNE); then a permutation of the page ids, whose
    first B * pages_per_seq entries form the block table row by row."""
    rng = np.random.default_rng(w.seed)
    shapes = {"q": (w.B, w.Hq, w.Sq, w.D),
              "k_cache": (w.num_pages, w.Hkv, w.page_size, w.D),
              "v_cache": (w.num_pages, w.Hkv, w.page_size, w.D)}
    bits = {}
    for n in ("q", "k_cache", "v_cache"):
        bits[n] = round_to_bf16_bits(rng.standard_normal(shapes[n], dtype=np.float32))
    vals = {n: bf16_bits_to_f32(b) for n, b in bits.items()}
    perm = rng.permutation(w.num_pages).astype(np.int32)
    bt = np.ascontiguousarray(perm[:w.B * w.pages_per_seq].reshape(w.B, w.pages_per_seq))
    return PagedInputs(w, vals, bits, bt, np.asarray(w.seqlens, dtype=np.int32))


def paged_to_torch(inp: PagedInputs, device) -> Dict[str, "object"]:
    import torch

    out = {n: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(device).contiguous()
           for n, b in inp.bits.items()}
    out["block_table"] = torch.from_numpy(inp.block_table).to(device).contiguous()
    out["seqlens"] = torch.from_numpy(inp.seqlens).to(device).contiguous()
    return out


def head_sample(w: Workload, n: int, seed: int = 0) -> Tuple[Tuple[int, int], ...]:
    """A fixed, seeded choice of (b, h) pairs, always including the first and
    the last head."""
    pairs = [(0, 0), (w.B - 1, w.Hq - 1)]
    rng = np.random.default_rng(1000 + seed)
    while len(pairs) < min(n, w.B * w.Hq):
        p = (int(rng.integers(w.B)), int(rng.integers(w.Hq)))
        if p not in pairs:
            pairs.append(p)
    return tuple(pairs)
