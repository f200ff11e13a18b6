"""Gradients of exact attention in float64 (the backward pass), for one head.

Test infrastructure only: imported by tests/ (and bench.py's CPU-baseline leg),
never by the product path.

Source: "FlashAttention 2 & 3: Work Partitioning, Warp Specialization & FP8",
section "The backward pass: recompute, and the one identity that makes it
tile-able". With O = softmax(scale * Q K^T [+ causal mask]) V, its row
logsumexp L, and the incoming gradient dO, the page gives the gradients in
closed form:

- P_ij = exp(S_ij - L_i), S = scale * Q K^T (masked entries: P_ij = 0);
- dV = P^T dO;
- dP = dO V^T;
- D_i = sum_j P_ij dP_ij, which equals the row dot product sum_c dO_ic O_ic
  (the identity that lets a key tile compute its share locally);
- dS = P o (dP - D) (row-broadcast D; "o" is the elementwise product), the
  softmax Jacobian applied row by row;
- dQ = scale * dS K and dK = scale * dS^T Q.

``attention_bwd_head_fp64`` materialises S, P, dP and dS (small N).
``attention_bwd_sampled_fp64`` computes the same quantities for chosen query
rows (dQ) and chosen key rows (dK, dV) of a long sequence: it needs O and L for
every row (from the forward oracle), then only the matching rows or columns of
S, P, dP and dS. Both follow the formulas above step by step.
"""

from __future__ import annotations

import numpy as np

from oracle.attention import _as_f64, _causal_mask, attention_head_fp64, attention_probs_fp64


def attention_bwd_head_fp64(q, k, v, do, scale: float, causal: bool):
    """(dQ, dK, dV, D) for one head; q, k, v, do are [N, d] (any float dtype)."""
    q, k, v, do = (_as_f64(x) for x in (q, k, v, do))
    _, _, _, p = attention_probs_fp64(q, k, scale, causal)   # P, masked entries 0
    o = p @ v
    dv = p.T @ do
    dp = do @ v.T
    delta = np.sum(do * o, axis=1)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv, delta


def attention_bwd_sampled_fp64(q, k, v, do, scale: float, causal: bool, qrows, kcols, chunk: int = 2048):
    """Rows of the gradients of one head without an N x N matrix.

    Returns (dQ[qrows], dK[kcols], dV[kcols], D) with D over all rows.
    L and O come from the three-pass forward oracle; P entries are rebuilt as
    exp(S - L) exactly as the page does in the backward.
    """
    q, k, v, do = (_as_f64(x) for x in (q, k, v, do))
    n = q.shape[0]
    o, lse = attention_head_fp64(q, k, v, scale, causal, chunk=chunk)
    delta = np.sum(do * o, axis=1)
    qrows = np.asarray(qrows, dtype=np.int64)
    kcols = np.asarray(kcols, dtype=np.int64)

    # dQ rows: full rows of P, dP, dS for the chosen queries
    s = scale * (q[qrows] @ k.T)
    hide = _causal_mask(qrows, k.shape[0]) if causal else np.zeros(s.shape, dtype=bool)
    p = np.where(hide, 0.0, np.exp(np.where(hide, 0.0, s - lse[qrows, None])))
    dp = do[qrows] @ v.T
    ds = p * (dp - delta[qrows, None])
    dq = scale * (ds @ k)

    # dK, dV rows: full columns of P, dP, dS for the chosen keys
    dk = np.zeros((kcols.shape[0], k.shape[1]))
    dv = np.zeros((kcols.shape[0], v.shape[1]))
    for r0 in range(0, n, chunk):
        r = np.arange(r0, min(n, r0 + chunk))
        s = scale * (q[r] @ k[kcols].T)                          # [rows, keys]
        hide = (kcols[None, :] > r[:, None]) if causal else np.zeros(s.shape, dtype=bool)
        p = np.where(hide, 0.0, np.exp(np.where(hide, 0.0, s - lse[r, None])))
        dp = do[r] @ v[kcols].T
        ds = p * (dp - delta[r, None])
        dv += p.T @ do[r]
        dk += scale * (ds.T @ q[r])
    return dq, dk, dv, delta


def attention_bwd_fp64(q, k, v, do, scale: float, causal: bool):
    """(dQ, dK, dV) over [B, H, N, d] inputs, float64."""
    q, k, v, do = (_as_f64(x) for x in (q, k, v, do))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for bi in range(q.shape[0]):
        for hi in range(q.shape[1]):
            dq[bi, hi], dk[bi, hi], dv[bi, hi], _ = attention_bwd_head_fp64(
                q[bi, hi], k[bi, hi], v[bi, hi], do[bi, hi], scale, causal)
    return dq, dk, dv
