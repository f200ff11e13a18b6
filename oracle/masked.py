"""Exact attention with grouped key/value heads, sliding windows and packed variable-length
sequences, in float64 (three passes, scores and probabilities materialised).

Test infrastructure only: imported by tests/ and bench.py's CPU-baseline leg, never by the
product path.

Sources ("Learn: The Memory Wall & FlashAttention", the flash_attn interface example and
Exercise 5 of "FlashAttention 2 & 3: Work Partitioning, Warp Specialization & FP8"):
- grouped-query attention: the number of key/value heads divides the number of query heads;
  query head h reads key/value head h // (Hq / Hkv), with no copies of K and V;
- sliding window (left, right): the window counts keys strictly to each side of the query,
  so query i sees key j iff i - left <= j <= i + right, and with the causal mask also j <= i
  ((4095, 0) with the causal mask is a window of 4096 keys including the query itself). A
  negative bound means no limit on that side (flash_attn's -1);
- packed variable-length batches: the sequences of a batch are concatenated along the token
  axis and cu_seqlens (B + 1 non-decreasing offsets, cu_seqlens[0] = 0) marks where each one
  starts; a query sees only keys of its own sequence, and positions (for the causal mask and
  the window) count from the start of that sequence.
- a row with no visible key gets O = 0 and LSE = -inf (the dead-row guard of Exercise 5: it
  contributes nothing); it cannot occur with the causal mask or a window that contains the
  query, since the query then sees itself.

Layout: without cu_seqlens Q is [B, Hq, N, d] and K, V are [B, Hkv, N, d]; with cu_seqlens the
batch dimension is 1 and N is the total number of tokens: Q [1, Hq, N, d], K, V [1, Hkv, N, d].
O has Q's shape and LSE is [B, Hq, N] (or [1, Hq, N]).
"""

from __future__ import annotations

import numpy as np

from oracle.attention import _as_f64


def visible_mask(n: int, causal: bool, left: int, right: int) -> np.ndarray:
    """[n, n] boolean: query i (row) sees key j (column) of one sequence."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    ok = np.ones((n, n), dtype=bool)
    if causal:
        ok &= j <= i
    if left >= 0:
        ok &= j >= i - left
    if right >= 0:
        ok &= j <= i + right
    return ok


def _sequence_fp64(q, k, v, scale: float, ok: np.ndarray):
    """Three-pass attention of one head of one sequence under the visibility mask ok."""
    s = np.where(ok, scale * (q @ k.T), -np.inf)
    alive = ok.any(axis=1)
    m = np.where(alive, s.max(axis=1, initial=-np.inf), 0.0)       # pass 1: row max
    e = np.where(ok, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)                                               # pass 2: row sum
    p = e / np.where(alive, l, 1.0)[:, None]                        # pass 3: probabilities
    lse = np.where(alive, m + np.log(np.where(alive, l, 1.0)), -np.inf)
    return p @ v, lse


def attention_ext_fp64(q, k, v, scale: float, causal: bool, window=(-1, -1), cu_seqlens=None):
    """(O, LSE) with grouped heads, an optional sliding window and optional packed sequences."""
    q, k, v = (_as_f64(x) for x in (q, k, v))
    b_, hq, n, d = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("the number of key/value heads must divide the number of query heads")
    g = hq // hkv
    left, right = int(window[0]), int(window[1])
    out = np.zeros((b_, hq, n, v.shape[3]))
    lse = np.full((b_, hq, n), -np.inf)
    if cu_seqlens is None:
        segs = [(bi, 0, n) for bi in range(b_)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        if b_ != 1 or cu[0] != 0 or cu[-1] != n or np.any(np.diff(cu) < 0):
            raise ValueError("packed sequences: batch 1, cu_seqlens from 0 to N, non-decreasing")
        segs = [(0, int(a), int(c)) for a, c in zip(cu[:-1], cu[1:])]
    for bi, a, c in segs:
        if c == a:
            continue
        ok = visible_mask(c - a, causal, left, right)
        for h in range(hq):
            out[bi, h, a:c], lse[bi, h, a:c] = _sequence_fp64(q[bi, h, a:c], k[bi, h // g, a:c], v[bi, h // g, a:c],
                                                              scale, ok)
    return out, lse


def attention_ext_rows_fp64(q, k, v, scale: float, causal: bool, window, b: int, h: int, rows):
    """(O[rows], LSE[rows]) of batch b, query head h, without packing: the same three passes
    restricted to the chosen query rows (a rows x N block of scores), for long sequences."""
    g = q.shape[1] // k.shape[1]
    qh, kh, vh = (_as_f64(x) for x in (q[b, h], k[b, h // g], v[b, h // g]))
    n = qh.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    ok = visible_mask(n, causal, int(window[0]), int(window[1]))[rows]
    s = np.where(ok, scale * (qh[rows] @ kh.T), -np.inf)
    m = s.max(axis=1)                           # every row sees itself: finite
    e = np.where(ok, np.exp(s - m[:, None]), 0.0)
    l = e.sum(axis=1)
    return (e / l[:, None]) @ vh, m + np.log(l)


def visible_pairs(n: int, causal: bool, left: int, right: int) -> int:
    """Number of (query, key) pairs one head of one sequence of length n computes with."""
    i = np.arange(n)
    hi = np.full(n, n - 1)
    if causal:
        hi = np.minimum(hi, i)
    if right >= 0:
        hi = np.minimum(hi, i + right)
    lo = np.zeros(n, dtype=np.int64)
    if left >= 0:
        lo = np.maximum(lo, i - left)
    return int(np.maximum(hi - lo + 1, 0).sum())
