"""Attention of a few query positions against a long key/value sequence (decoding), in
float64, and the split-key form that combines partial softmax states.

Test infrastructure only: imported by tests/ and bench.py's CPU-baseline leg, never by the
product path.

Sources:
- "FlashAttention 2 & 3: Work Partitioning, Warp Specialization & FP8", the paragraph on
  the decode regime (after the xFormers comparison): at decode time the query is one token,
  so Q K^T is a matrix-vector product and the query-parallel grid has nothing to split;
  FlashDecoding splits the key/value sequence instead, each part computes a partial softmax
  and the parts are combined with the online-softmax merge.
- "FlashAttention-3 & GPU Kernel Optimization", section "Online softmax tiling
  mathematics": the merge of two partial states (``oracle.attention.merge_states``).
- "Learn: The Memory Wall & FlashAttention", the flash_attn interface example: grouped-query
  attention, where the number of key/value heads divides the number of query heads.

Readings (the pages fix none of these for decoding):
- the Nq queries are the last Nq positions of a sequence of Nk keys; under the causal mask
  query i (0-based) sees keys j <= Nk - Nq + i. For Nq = Nk this is the forward's mask;
  for Nq = 1 every key is visible;
- query head h reads key/value head h // (Hq / Hkv), the usual grouping;
- a partial state over keys that a query cannot see is (m, l, O~) = (-inf, 0, 0) and drops
  out of the merge.

Layout: Q [B, Hq, Nq, d]; K, V [B, Hkv, Nk, d]; O [B, Hq, Nq, d]; LSE [B, Hq, Nq].
"""

from __future__ import annotations

import numpy as np

from oracle.attention import _as_f64, merge_states


def _hidden(nq: int, nk: int, k0: int, k1: int, causal: bool) -> np.ndarray:
    """[nq, k1 - k0] mask of the keys k0 .. k1-1 that query i may not see."""
    keys = np.arange(k0, k1)[None, :]
    if not causal:
        return np.zeros((nq, k1 - k0), dtype=bool)
    return keys > (nk - nq + np.arange(nq))[:, None]


def decode_head_fp64(q, k, v, scale: float, causal: bool):
    """(O [Nq, d], LSE [Nq]) of one query head against its key/value head, three passes with
    the scores and probabilities materialised (requires Nq <= Nk)."""
    q, k, v = (_as_f64(x) for x in (q, k, v))
    nq, nk = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    s = np.where(_hidden(nq, nk, 0, nk, causal), -np.inf, s)
    m = s.max(axis=1)                      # pass 1: row max (key 0 is visible to every query)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)                      # pass 2: row sum
    p = e / l[:, None]                     # pass 3: probabilities, then P V
    return p @ v, m + np.log(l)


def attention_decode_fp64(q, k, v, scale: float, causal: bool):
    """(O, LSE) over [B, Hq, Nq, d] queries and [B, Hkv, Nk, d] keys/values, float64."""
    q, k, v = (_as_f64(x) for x in (q, k, v))
    b_, hq, nq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv != 0:
        raise ValueError("the number of key/value heads must divide the number of query heads")
    g = hq // hkv
    out = np.zeros((b_, hq, nq, v.shape[3]))
    lse = np.zeros((b_, hq, nq))
    for bi in range(b_):
        for h in range(hq):
            out[bi, h], lse[bi, h] = decode_head_fp64(q[bi, h], k[bi, h // g], v[bi, h // g], scale, causal)
    return out, lse


def partial_state_fp64(q, k, v, scale: float, causal: bool, k0: int, k1: int):
    """Softmax state (m, l, O~) of the queries of one head over keys k0 .. k1-1: m the largest
    visible score, l = sum exp(s - m), O~ = sum exp(s - m) v (not divided by l); a query with
    no visible key there gets (-inf, 0, 0)."""
    q, k, v = (_as_f64(x) for x in (q, k, v))
    nq, nk = q.shape[0], k.shape[0]
    s = scale * (q @ k[k0:k1].T)
    hide = _hidden(nq, nk, k0, k1, causal)
    s = np.where(hide, -np.inf, s)
    any_visible = ~hide.all(axis=1) if k1 > k0 else np.zeros(nq, dtype=bool)
    m = np.where(any_visible, s.max(axis=1, initial=-np.inf), -np.inf)
    e = np.where(hide, 0.0, np.exp(s - np.where(any_visible, m, 0.0)[:, None]))
    return m, e.sum(axis=1), e @ v[k0:k1]


def merge_all_fp64(states):
    """Fold partial states with the page-5 merge; states with l = 0 (no visible key) drop out."""
    m = l = o = None
    for sm, sl, so in states:
        if m is None:
            m, l, o = sm.copy(), sl.copy(), so.copy()
            continue
        empty_new, empty_old = sl == 0, l == 0
        # rows where one side is empty take the other side unchanged
        both = ~empty_new & ~empty_old
        mb, lb, ob = merge_states(np.where(both, m, 0.0), np.where(both, l, 0.0), np.where(both[:, None], o, 0.0),
                                  np.where(both, sm, 0.0), np.where(both, sl, 0.0), np.where(both[:, None], so, 0.0))
        m = np.where(both, mb, np.where(empty_old, sm, m))
        l = np.where(both, lb, np.where(empty_old, sl, l))
        o = np.where(both[:, None], ob, np.where(empty_old[:, None], so, o))
    return m, l, o


def decode_head_split_fp64(q, k, v, scale: float, causal: bool, edges):
    """(O, LSE) of one head computed over the key ranges [edges[i], edges[i+1]) separately and
    merged: the split-key form."""
    states = [partial_state_fp64(q, k, v, scale, causal, a, b) for a, b in zip(edges[:-1], edges[1:])]
    m, l, o = merge_all_fp64(states)
    return o / l[:, None], m + np.log(l)
