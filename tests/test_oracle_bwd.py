"""Pins of the backward oracle (CPU, float64).

The oracle's closed-form gradients ("FlashAttention 2 & 3" page, section "The
backward pass") are checked against things it does not compute itself:
- central finite differences of the scalar f(Q, K, V) = sum(O o G), whose
  gradient with respect to Q, K, V is exactly (dQ, dK, dV) for dO = G; every
  entry of every input is perturbed, so a dropped term, a wrong sign, a missing
  scale or a transposed product fails;
- the page's identity sum_j P_ij dP_ij = sum_c dO_ic O_ic, evaluated both ways;
- rows of dS sum to zero (the softmax Jacobian annihilates constants);
- uniform scores (Q = 0): dV_j = mean over the queries that see key j of dO,
  written out directly;
- permuting the rows of K and V together permutes dK and dV the same way and
  leaves dQ unchanged;
- the sampled form equals the materialising form row for row.
"""

import numpy as np
import pytest

from oracle.attention import attention_head_fp64, attention_probs_fp64
from oracle.attention_bwd import attention_bwd_fp64, attention_bwd_head_fp64, attention_bwd_sampled_fp64


def _inputs(n, d, seed):
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((n, d)) for _ in range(4)]


def _loss(q, k, v, g, scale, causal):
    o, _ = attention_head_fp64(q, k, v, scale, causal)
    return float(np.sum(o * g))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(5, 3), (7, 4)])
def test_gradients_match_central_differences(n, d, causal):
    q, k, v, g = _inputs(n, d, seed=10 * n + d + causal)
    scale = 0.7
    dq, dk, dv, _ = attention_bwd_head_fp64(q, k, v, g, scale, causal)
    eps = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], g, scale, causal)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], g, scale, causal)) / (2 * eps)
        assert np.abs(num - grad).max() <= 1e-7 * max(1.0, np.abs(grad).max()), name


def test_causal_last_key_gradient_comes_from_last_query_only():
    # key N-1 is visible only to query N-1: dV_{N-1} = P_{N-1,N-1} dO_{N-1}
    q, k, v, g = _inputs(6, 4, seed=3)
    _, _, _, p = attention_probs_fp64(q, k, 0.5, True)
    _, _, dv, _ = attention_bwd_head_fp64(q, k, v, g, 0.5, True)
    assert np.allclose(dv[-1], p[-1, -1] * g[-1], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_delta_identity_and_zero_row_sums(causal):
    q, k, v, g = _inputs(40, 16, seed=5)
    scale = 0.25
    _, _, _, delta = attention_bwd_head_fp64(q, k, v, g, scale, causal)
    _, _, _, p = attention_probs_fp64(q, k, scale, causal)
    dp = g @ v.T
    assert np.allclose(delta, np.sum(p * dp, axis=1), rtol=1e-12, atol=1e-12)
    ds = p * (dp - delta[:, None])
    assert np.abs(ds.sum(axis=1)).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores(causal):
    n, d = 9, 5
    _, k, v, g = _inputs(n, d, seed=8)
    q = np.zeros((n, d))
    _, _, dv, _ = attention_bwd_head_fp64(q, k, v, g, 1.0, causal)
    for j in range(n):
        if causal:   # query i >= j sees i + 1 keys, each with probability 1 / (i + 1)
            expect = sum(g[i] / (i + 1) for i in range(j, n))
        else:
            expect = g.mean(axis=0)
        assert np.allclose(dv[j], expect, rtol=0, atol=1e-13)


def test_permuting_keys_and_values_together():
    q, k, v, g = _inputs(30, 8, seed=9)
    perm = np.random.default_rng(1).permutation(30)
    dq, dk, dv, _ = attention_bwd_head_fp64(q, k, v, g, 0.3, False)
    dq2, dk2, dv2, _ = attention_bwd_head_fp64(q, k[perm], v[perm], g, 0.3, False)
    assert np.allclose(dq, dq2, rtol=0, atol=1e-12)
    assert np.allclose(dk[perm], dk2, rtol=0, atol=1e-12)
    assert np.allclose(dv[perm], dv2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_equals_full(causal):
    q, k, v, g = _inputs(300, 16, seed=11)
    scale = 0.25
    dq, dk, dv, delta = attention_bwd_head_fp64(q, k, v, g, scale, causal)
    rows = np.array([0, 1, 77, 150, 299])
    cols = np.array([0, 5, 128, 298, 299])
    sq, sk, sv, sd = attention_bwd_sampled_fp64(q, k, v, g, scale, causal, rows, cols, chunk=64)
    assert np.allclose(sq, dq[rows], rtol=0, atol=1e-12)
    assert np.allclose(sk, dk[cols], rtol=0, atol=1e-12)
    assert np.allclose(sv, dv[cols], rtol=0, atol=1e-12)
    assert np.allclose(sd, delta, rtol=0, atol=1e-12)


def test_batched_layout_is_per_head():
    rng = np.random.default_rng(12)
    q, k, v, g = (rng.standard_normal((2, 3, 20, 8)) for _ in range(4))
    dq, dk, dv = attention_bwd_fp64(q, k, v, g, 0.35, True)
    h = attention_bwd_head_fp64(q[1, 2], k[1, 2], v[1, 2], g[1, 2], 0.35, True)
    assert np.array_equal(dq[1, 2], h[0]) and np.array_equal(dk[1, 2], h[1]) and np.array_equal(dv[1, 2], h[2])
