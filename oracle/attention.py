"""CPU float64 oracle for scaled-dot-product attention, forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only
the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may call it.  It shares no code with the HIP path.

What it computes is the *composed* (materialised-scores) attention that the
xtrain evolution page (infrastructure-phase table, row T4) builds from
matmul + softmax, and against which its fused flash kernel (row T14) is
checked.  The fused kernel reaches that same result up to rounding: the
online-softmax rescaling is an exact identity, which is why the page reports
flash == composed.  So this oracle is simply the definition written out in
float64, with the whole score row of every query materialised:

    S_ij  = scale * <q_i, k_j>                      (masked entries -> -inf)
    P_ij  = exp(S_ij - max_j S_ij) / sum_j exp(S_ij - max_j S_ij)
    O_i   = sum_j P_ij v_j          LSE_i = max_j S_ij + ln sum_j exp(...)

and its gradient for a given dO (row T14: the flash-style backward recomputes
the scores and uses the per-row scalar D = sum(dO * O) to simplify the softmax
Jacobian):

    Dlt_i = <dO_i, O_i>             dP_ij = <dO_i, v_j>
    dS_ij = P_ij (dP_ij - Dlt_i)
    dQ_i  = scale * sum_j dS_ij k_j
    dK_j  = scale * sum_i dS_ij q_i     dV_j = sum_i P_ij dO_i

Grouped KV heads follow row T15 of the same table: query head h reads KV head
floor(h / G) with G = Hq / Hkv (the repeat-kv convention dst = kvh*G + r), and
the KV-head gradients are the deterministic sum over the group's G query
heads, taken in ascending r.

Readings where the pages are silent (each is listed in the design notes):

* causal masking is aligned bottom-right: key j is visible to query i iff
  j <= i + (Skv - Sq); with Sq == Skv this is the usual j <= i.
* a query row with no visible key has O = 0, LSE = -inf and zero gradients.
* LSE uses the natural logarithm of the scaled scores.

Every query row is defined independently of every other, so the functions
below visit rows in groups only to bound memory; within a row nothing is
blocked or reordered: the full score row is formed, then the softmax, then
the products.  Matrix products use numpy (BLAS) in float64.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

_ROW_CHUNK = 1024


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def visible(rows: np.ndarray, Sq: int, Skv: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), Skv]: which keys each query row may attend to."""
    rows = np.asarray(rows)
    if not causal:
        return np.ones((rows.shape[0], Skv), dtype=bool)
    return np.arange(Skv)[None, :] <= (rows[:, None] + (Skv - Sq))


def probs_head(q, k, causal: bool, scale: float, rows: Optional[Sequence[int]] = None):
    """Softmax probabilities P [n, Skv] and LSE [n] of one head, for the given
    query rows (all rows if None).  q: [Sq, D], k: [Skv, D]."""
    q, k = _f64(q), _f64(k)
    Sq, Skv = q.shape[0], k.shape[0]
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    s = scale * (q[rows] @ k.T)
    vis = visible(rows, Sq, Skv, causal)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1) if Skv > 0 else np.full(len(rows), -np.inf)
    has = np.isfinite(m)
    e = np.exp(s - np.where(has, m, 0.0)[:, None])  # exp(-inf) = 0 for masked keys
    l = e.sum(axis=1)
    p = e / np.where(l > 0, l, 1.0)[:, None]
    with np.errstate(divide="ignore"):
        lse = np.where(has, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return p, lse


def forward_head(q, k, v, causal: bool, scale: float,
                 rows: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """O [n, D] and LSE [n] of one head for the given query rows."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(rows), v.shape[1]))
    lse = np.empty(len(rows))
    for s0 in range(0, len(rows), _ROW_CHUNK):
        r = rows[s0:s0 + _ROW_CHUNK]
        p, l = probs_head(q, k, causal, scale, r)
        o[s0:s0 + len(r)] = p @ v
        lse[s0:s0 + len(r)] = l
    return o, lse


def backward_head(q, k, v, do, causal: bool, scale: float):
    """Gradients of L = sum(dO * O) for one query head and the KV head it
    reads: (dq [Sq, D], dk [Skv, D], dv [Skv, D], Dlt [Sq])."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    p, _ = probs_head(q, k, causal, scale)
    o = p @ v
    dlt = np.sum(do * o, axis=1)
    dp = do @ v.T
    ds = p * (dp - dlt[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    dv = p.T @ do
    return dq, dk, dv, dlt


def _group(q, k) -> int:
    Hq, Hkv = q.shape[1], k.shape[1]
    if Hkv == 0 or Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return Hq // Hkv


def attention_forward(q, k, v, causal: bool, scale: float):
    """q: [B,Hq,Sq,D], k/v: [B,Hkv,Skv,D] -> O [B,Hq,Sq,D], LSE [B,Hq,Sq]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Sq, D = q.shape
    G = _group(q, k)
    o = np.zeros((B, Hq, Sq, v.shape[3]))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h // G], v[b, h // G], causal, scale)
    return o, lse


def attention_backward(q, k, v, do, causal: bool, scale: float):
    """-> dq [B,Hq,Sq,D], dk/dv [B,Hkv,Skv,D], Dlt [B,Hq,Sq]."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    G = _group(q, k)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dlt = np.zeros((B, Hq, Sq))
    for b in range(B):
        for kv in range(Hkv):
            for r in range(G):  # ascending group member: h = kv*G + r
                h = kv * G + r
                dq[b, h], dkh, dvh, dlt[b, h] = backward_head(
                    q[b, h], k[b, kv], v[b, kv], do[b, h], causal, scale)
                dk[b, kv] += dkh
                dv[b, kv] += dvh
    return dq, dk, dv, dlt


def dq_rows(q, k, v, do, causal: bool, scale: float, rows: Sequence[int]) -> np.ndarray:
    """dQ of one head for selected query rows only (each dQ row depends on
    its own query row alone)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    rows = np.asarray(rows, dtype=np.int64)
    p, _ = probs_head(q, k, causal, scale, rows)
    o = p @ v
    dlt = np.sum(do[rows] * o, axis=1)
    ds = p * (do[rows] @ v.T - dlt[:, None])
    return scale * (ds @ k)
