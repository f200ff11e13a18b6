"""Three-pass exact attention in float64, plus the streaming recurrence it is pinned by.

Test infrastructure only: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py, never by the product path.

Sources (the five pages on exact attention):
- "Learn: The Memory Wall & FlashAttention", section 4 "The attention memory
  problem": S = Q K^T / sqrt(d), P = softmax(S), O = P V, computed as three
  separate steps with S and P materialised. This module does exactly that,
  with a general ``scale`` in place of 1/sqrt(d).
- same page, section 5.1 "Deriving the online softmax": safe softmax (subtract
  the row max m), and the streaming recurrence over key blocks with running
  (m, l, o), rescale factor alpha = exp(m_old - m_new), and one division at
  the end. ``online_softmax_attention`` follows it step by step; it exists to
  pin the three-pass form, not to be fast.
- "FlashAttention 2 & 3: Work Partitioning, Warp Specialization & FP8",
  section "The backward pass: recompute, and the one identity that makes it
  tile-able": the forward also returns the per-row logsumexp L = m + log l of
  the scaled scores (natural log), one number per query row.
- same page, "Edit 1 - defer the rescaling" (its reference loop): the causal
  mask hides key positions greater than the query position (top-left aligned,
  the diagonal is visible).
- same page, Exercise 5 (sliding window): a row whose keys are all masked
  contributes nothing (P -> 0, alpha -> 1). In this module such a row gets
  O = 0 and LSE = -inf; with a causal mask and equal query and key lengths it
  cannot occur, since key 0 is visible to every query.
- "FlashAttention-3 & GPU Kernel Optimization" (page 5), section "Online
  softmax tiling mathematics": the merge of two partial states (m1, l1, O1) and
  (m2, l2, O2). ``merge_states`` is that formula.

Layout: Q, K, V are [B, H, N, d] (batch, head, sequence, head dim), O is the
same shape and LSE is [B, H, N].
"""

from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _as_f64(x) -> np.ndarray:
    """Upcast a NumPy array or a CPU torch tensor (any float dtype) to float64."""
    if hasattr(x, "detach"):  # torch tensor: go through float32/float64 on the CPU
        import torch  # local import: the oracle does not otherwise need torch

        x = x.detach().to("cpu")
        if x.dtype not in (torch.float64,):
            x = x.to(torch.float64)
        return x.numpy()
    return np.asarray(x, dtype=np.float64)


def _causal_mask(rows: np.ndarray, n_keys: int) -> np.ndarray:
    """True where key position > query position (hidden by the causal mask)."""
    keys = np.arange(n_keys)[None, :]
    return keys > rows[:, None]


def attention_probs_fp64(q, k, scale: float, causal: bool):
    """Return (S, m, l, P) for one head; q, k are [N, d].

    Pass 1 m = row max of S, pass 2 l = row sum of exp(S - m), pass 3
    P = exp(S - m) / l (safe softmax, section 5.1 of the memory-wall page).
    Fully masked rows (m = -inf) get P = 0 and l = 0.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    n = q.shape[0]
    s = scale * (q @ k.T)
    if causal:
        s = np.where(_causal_mask(np.arange(n), k.shape[0]), NEG_INF, s)
    m = s.max(axis=1)
    dead = ~np.isfinite(m)
    m_safe = np.where(dead, 0.0, m)
    e = np.exp(s - m_safe[:, None])
    e[dead] = 0.0
    l = e.sum(axis=1)
    p = np.zeros_like(e)
    live = ~dead
    p[live] = e[live] / l[live, None]
    return s, m, l, p


def attention_head_fp64(q, k, v, scale: float, causal: bool, rows=None, chunk: int = 2048):
    """Three-pass attention for one head; q, k, v are [N, d].

    ``rows`` (optional 1-D integer array) selects the query rows to compute;
    each selected row still sees every key (subject to the causal mask), so a
    sampled row is exactly the row of the full result. Rows are processed in
    chunks of ``chunk`` so that S stays a few hundred MiB; rows are
    independent, so chunking changes nothing in the arithmetic.

    Returns (O [R, d], LSE [R]) in float64.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    n_keys = k.shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], v.shape[1]), dtype=np.float64)
    lse = np.full((rows.shape[0],), NEG_INF, dtype=np.float64)
    for r0 in range(0, rows.shape[0], chunk):
        r = rows[r0:r0 + chunk]
        s = scale * (q[r] @ k.T)                       # S: scaled scores [c, N]
        if causal:
            s = np.where(_causal_mask(r, n_keys), NEG_INF, s)
        m = s.max(axis=1)                              # pass 1: row max
        live = np.isfinite(m)
        e = np.exp(s[live] - m[live, None])            # pass 2: exp(S - m), row sums
        l = e.sum(axis=1)
        p = e / l[:, None]                             # pass 3: P = exp(S - m) / l
        out[r0:r0 + r.shape[0]][live] = p @ v          # O = P V
        lse_c = lse[r0:r0 + r.shape[0]]
        lse_c[live] = m[live] + np.log(l)              # L = m + log l
    return out, lse


def attention_fp64(q, k, v, scale: float, causal: bool):
    """Three-pass attention over [B, H, N, d] inputs; returns (O, LSE) in float64."""
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    b, h, n, d = q.shape
    out = np.zeros((b, h, n, v.shape[3]), dtype=np.float64)
    lse = np.zeros((b, h, n), dtype=np.float64)
    for bi in range(b):
        for hi in range(h):
            out[bi, hi], lse[bi, hi] = attention_head_fp64(q[bi, hi], k[bi, hi], v[bi, hi], scale, causal)
    return out, lse


def online_softmax_attention(q, k, v, scale: float, causal: bool, block_edges, _rescale: bool = True):
    """Streaming attention for one head by the section-5.1 recurrence.

    ``block_edges`` are the key-block boundaries, e.g. [0, 64, 128, ..., N]
    (blocks may have any sizes). Per query row it keeps the running max m,
    the running denominator l and the unnormalised accumulator o, all
    referred to the current max; each block updates

        m_new = max(m, max_j s_j)
        alpha = exp(m - m_new)
        l     = alpha * l + sum_j exp(s_j - m_new)
        o     = alpha * o + sum_j exp(s_j - m_new) v_j

    and the output is o / l after the last block (one division at the end,
    "Edit 1 - defer the rescaling"). Rows that have seen only masked keys keep
    alpha = 1 and add nothing (the Exercise 5 guard).

    ``_rescale=False`` drops alpha from the accumulator update only
    (o = o + sum_j exp(s_j - m_new) v_j, while l keeps its correction): the
    broken variant asked about in Exercise 2 of the FlashAttention 2 & 3 page,
    used by a test to show that exactness then fails.

    Returns (O [N, d], LSE [N], states) where states lists (m, l, o) after
    each block.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    n, d_v = q.shape[0], v.shape[1]
    m = np.full((n,), NEG_INF)
    l = np.zeros((n,))
    o = np.zeros((n, d_v))
    rows = np.arange(n)
    states = []
    for j0, j1 in zip(block_edges[:-1], block_edges[1:]):
        s = scale * (q @ k[j0:j1].T)
        if causal:
            keys = np.arange(j0, j1)[None, :]
            s = np.where(keys > rows[:, None], NEG_INF, s)
        m_blk = s.max(axis=1) if s.shape[1] else np.full((n,), NEG_INF)
        m_new = np.maximum(m, m_blk)
        dead = ~np.isfinite(m_new)
        m_ref = np.where(dead, 0.0, m_new)
        p = np.exp(s - m_ref[:, None])
        p[dead] = 0.0
        alpha = np.where(dead, 1.0, np.exp(m - m_ref))
        l = alpha * l + p.sum(axis=1)
        alpha_o = alpha if _rescale else np.ones((n,))
        o = alpha_o[:, None] * o + p @ v[j0:j1]
        m = m_new
        states.append((m.copy(), l.copy(), o.copy()))
    live = l > 0
    out = np.zeros_like(o)
    out[live] = o[live] / l[live, None]
    lse = np.full((n,), NEG_INF)
    lse[live] = m[live] + np.log(l[live])
    return out, lse, states


def merge_states(m1, l1, o1, m2, l2, o2):
    """Combine two partial softmax states over disjoint key sets (page 5 formula).

    m = max(m1, m2); l = exp(m1 - m) l1 + exp(m2 - m) l2;
    O = exp(m1 - m) O1 + exp(m2 - m) O2, with O1, O2 unnormalised
    accumulators referred to m1 and m2. Returns (m, l, O).
    """
    m = np.maximum(m1, m2)
    a1 = np.exp(m1 - m)
    a2 = np.exp(m2 - m)
    return m, a1 * l1 + a2 * l2, a1[:, None] * o1 + a2[:, None] * o2
