"""Pins for the CPU oracle: checks against what the pages and the mathematics fix.

None of these tests touches the GPU or the HIP library. Each pin is chosen so
that a plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a wrong scale or mask) fails at least one of them:

- page values: the worked online-softmax example ("Learn: The Memory Wall &
  FlashAttention", Practice problem 2), stored in tests/golden/;
- closed forms: uniform scores give mean(V) and LSE = ln(count); causal row 0
  gives V_0; one dominant score selects its value row;
- invariants: P rows sum to 1, P >= 0, m <= LSE <= m + ln N, permuting K and V
  rows together changes nothing (non-causal);
- independent routes: torch / scipy softmax and logsumexp in float64, and a
  pure-Python brute force on tiny inputs;
- the streaming recurrence of section 5.1 and the page-5 merge formula must
  equal the three-pass result for any block split, and dropping alpha
  (Exercise 2 of the FlashAttention 2 & 3 page) must break it.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_qkv(seed, b, h, n, d, dv=None):
    rng = np.random.default_rng(seed)
    dv = d if dv is None else dv
    return (rng.standard_normal((b, h, n, d)), rng.standard_normal((b, h, n, d)),
            rng.standard_normal((b, h, n, dv)))


# ---------------------------------------------------------------- page values

def _worked_inputs():
    g = json.load(open(os.path.join(GOLDEN, "online_softmax_worked_example.json")))
    scores = g["scores_block1"] + g["scores_block2"]
    q = np.array([[1.0]])
    k = np.array([[s] for s in scores])          # scale 1, d = 1: S_j = k_j
    v = np.array([[x] for x in g["values"]])
    return g, q, k, v


def test_worked_example_three_pass():
    g, q, k, v = _worked_inputs()
    o, lse = A.attention_head_fp64(q, k, v, 1.0, False)
    assert abs(o[0, 0] - g["output"]) <= g["tol"]
    # closed form of the same case: l = e^-3 + e^-1 + 1 + e^-2 referred to max 4
    l = math.exp(-3) + math.exp(-1) + 1.0 + math.exp(-2)
    num = 1 * math.exp(-3) + 2 * math.exp(-1) + 3 + 4 * math.exp(-2)
    assert abs(o[0, 0] - num / l) < 1e-14
    assert abs(lse[0] - (4.0 + math.log(l))) < 1e-14
    assert abs(l - g["after_block2"]["l"]) <= g["tol"]
    _, m, lsum, p = A.attention_probs_fp64(q, k, 1.0, False)
    assert m[0] == 4.0
    assert abs(lsum[0] - g["after_block2"]["l"]) <= g["tol"]
    np.testing.assert_allclose(p[0] * lsum[0], g["weights_global_max"], atol=g["tol"])


def test_worked_example_streaming_states():
    g, q, k, v = _worked_inputs()
    o, lse, states = A.online_softmax_attention(q, k, v, 1.0, False, [0, 2, 4])
    (m1, l1, o1), (m2, l2, o2) = states
    assert m1[0] == g["after_block1"]["m"]
    assert abs(l1[0] - g["after_block1"]["l"]) <= g["tol"]
    assert abs(o1[0, 0] - g["after_block1"]["o"]) <= g["tol"]
    assert abs(math.exp(m1[0] - m2[0]) - g["alpha_block2"]) <= g["tol"]
    assert m2[0] == g["after_block2"]["m"]
    assert abs(l2[0] - g["after_block2"]["l"]) <= g["tol"]
    assert abs(o2[0, 0] - g["after_block2"]["o"]) <= g["tol"]
    assert abs(o[0, 0] - g["output"]) <= g["tol"]


# ---------------------------------------------------------------- independent routes

@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_float64(causal):
    q, k, v = rand_qkv(1, 2, 3, 37, 16)
    scale = 0.37
    o, lse = A.attention_fp64(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * scale
    if causal:
        n = s.shape[-1]
        hide = torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1)
        s = s.masked_fill(hide, float("-inf"))
    ref_o = torch.matmul(torch.softmax(s, dim=-1), tv)
    ref_lse = torch.logsumexp(s, dim=-1)
    assert np.abs(o - ref_o.numpy()).max() < 1e-12
    assert np.abs(lse - ref_lse.numpy()).max() < 1e-12


def test_matches_scipy():
    from scipy.special import logsumexp, softmax

    q, k, v = rand_qkv(2, 1, 1, 50, 8, dv=5)
    s = 0.5 * q[0, 0] @ k[0, 0].T
    o, lse = A.attention_head_fp64(q[0, 0], k[0, 0], v[0, 0], 0.5, False)
    np.testing.assert_allclose(o, softmax(s, axis=1) @ v[0, 0], atol=1e-12)
    np.testing.assert_allclose(lse, logsumexp(s, axis=1), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bruteforce_python(causal):
    rng = np.random.default_rng(3)
    n, d, dv, scale = 5, 3, 2, 0.8
    q = rng.standard_normal((n, d)).tolist()
    k = rng.standard_normal((n, d)).tolist()
    v = rng.standard_normal((n, dv)).tolist()
    o, lse = A.attention_head_fp64(np.array(q), np.array(k), np.array(v), scale, causal)
    for i in range(n):
        keys = range(i + 1) if causal else range(n)
        sc = {j: scale * sum(q[i][t] * k[j][t] for t in range(d)) for j in keys}
        mx = max(sc.values())
        w = {j: math.exp(s - mx) for j, s in sc.items()}
        tot = sum(w.values())
        for c in range(dv):
            want = sum(w[j] * v[j][c] for j in keys) / tot
            assert abs(o[i, c] - want) < 1e-13
        assert abs(lse[i] - (mx + math.log(tot))) < 1e-13


def test_layout_bhnd_heads_independent():
    q, k, v = rand_qkv(4, 2, 3, 11, 4)
    o, lse = A.attention_fp64(q, k, v, 0.5, True)
    for b in range(2):
        for h in range(3):
            oh, lh = A.attention_head_fp64(q[b, h], k[b, h], v[b, h], 0.5, True)
            assert np.array_equal(oh, o[b, h]) and np.array_equal(lh, lse[b, h])
    # swapping two heads of the input swaps the outputs (no cross-head mixing)
    q2, k2, v2 = (x[:, ::-1].copy() for x in (q, k, v))
    o2, _ = A.attention_fp64(q2, k2, v2, 0.5, True)
    assert np.array_equal(o2[:, ::-1], o)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_mean_of_values(causal):
    n, d = 40, 8
    rng = np.random.default_rng(5)
    q = np.zeros((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    o, lse = A.attention_head_fp64(q, k, v, 0.125, causal)
    if causal:
        for i in range(n):
            np.testing.assert_allclose(o[i], v[: i + 1].mean(axis=0), atol=1e-13)
            assert abs(lse[i] - math.log(i + 1)) < 1e-13
    else:
        np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=0), o.shape), atol=1e-13)
        np.testing.assert_allclose(lse, math.log(n), atol=1e-13)


def test_causal_first_row_is_first_value():
    q, k, v = rand_qkv(6, 1, 1, 30, 16)
    o, lse = A.attention_head_fp64(q[0, 0], k[0, 0], v[0, 0], 0.25, True)
    np.testing.assert_allclose(o[0], v[0, 0, 0], atol=1e-15)
    assert abs(lse[0] - 0.25 * q[0, 0, 0] @ k[0, 0, 0]) < 1e-14


def test_dominant_score_selects_value():
    # orthogonal keys; query 1 points along key 17 with a score 150 above all others
    n = d = 64
    rng = np.random.default_rng(7)
    k = 3.0 * np.eye(n)
    v = rng.standard_normal((n, d))
    q = 0.01 * rng.standard_normal((3, d))
    q[1] = 0.0
    q[1, 17] = 400.0
    o, lse = A.attention_head_fp64(q, k, v, 1 / np.sqrt(d), False)
    np.testing.assert_allclose(o[1], v[17], atol=1e-15)
    assert abs(lse[1] - 150.0) < 1e-12


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("causal", [False, True])
def test_probability_invariants(causal):
    q, k, _ = rand_qkv(8, 1, 1, 33, 8)
    s, m, l, p = A.attention_probs_fp64(q[0, 0], k[0, 0], 0.7, causal)
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(axis=1), 1.0, atol=1e-13)
    if causal:
        assert (np.triu(p, 1) == 0).all()
    _, _, v = rand_qkv(9, 1, 1, 33, 8)
    _, lse = A.attention_head_fp64(q[0, 0], k[0, 0], v[0, 0], 0.7, causal)
    counts = np.arange(1, 34) if causal else np.full(33, 33)
    assert (m <= lse + 1e-15).all() and (lse <= m + np.log(counts) + 1e-15).all()


def test_permutation_invariance_non_causal():
    q, k, v = rand_qkv(10, 1, 2, 45, 8)
    perm = np.random.default_rng(11).permutation(45)
    o1, l1 = A.attention_fp64(q, k, v, 0.3, False)
    o2, l2 = A.attention_fp64(q, k[:, :, perm], v[:, :, perm], 0.3, False)
    assert np.abs(o1 - o2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-13
    # permuting K alone does change the result (the pairing of K and V matters)
    o3, _ = A.attention_fp64(q, k[:, :, perm], v, 0.3, False)
    assert np.abs(o1 - o3).max() > 1e-3


def test_row_chunking_and_row_sampling():
    q, k, v = rand_qkv(12, 1, 1, 50, 8)
    full_o, full_l = A.attention_head_fp64(q[0, 0], k[0, 0], v[0, 0], 0.3, True)
    ch_o, ch_l = A.attention_head_fp64(q[0, 0], k[0, 0], v[0, 0], 0.3, True, chunk=7)
    # BLAS may block a different number of rows differently: equal up to rounding
    assert np.abs(full_o - ch_o).max() < 1e-14 and np.abs(full_l - ch_l).max() < 1e-14
    rows = np.array([0, 3, 49, 17])
    so, sl = A.attention_head_fp64(q[0, 0], k[0, 0], v[0, 0], 0.3, True, rows=rows)
    assert np.abs(so - full_o[rows]).max() < 1e-14 and np.abs(sl - full_l[rows]).max() < 1e-14


# ---------------------------------------------------------------- streaming, merge, mutation

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("edges", [[0, 64, 128, 150], [0, 1, 2, 3, 150], [0, 100, 150], [0, 150],
                                   [0, 17, 17, 60, 61, 150]])
def test_streaming_equals_three_pass(causal, edges):
    q, k, v = rand_qkv(13, 1, 1, 150, 16)
    q = 3.0 * q   # larger scores: the running max moves often
    ref_o, ref_l = A.attention_head_fp64(q[0, 0], k[0, 0], v[0, 0], 0.25, causal)
    o, lse, _ = A.online_softmax_attention(q[0, 0], k[0, 0], v[0, 0], 0.25, causal, edges)
    assert np.abs(o - ref_o).max() < 1e-13
    assert np.abs(lse - ref_l).max() < 1e-13


def test_merge_of_two_halves_equals_three_pass():
    q, k, v = rand_qkv(14, 1, 1, 90, 8)
    q, k, v = q[0, 0] * 2.0, k[0, 0], v[0, 0]
    ref_o, ref_l = A.attention_head_fp64(q, k, v, 0.4, False)
    idx1 = np.arange(0, 90, 2)
    idx2 = np.arange(1, 90, 2)
    _, _, st1 = A.online_softmax_attention(q, k[idx1], v[idx1], 0.4, False, [0, len(idx1)])
    _, _, st2 = A.online_softmax_attention(q, k[idx2], v[idx2], 0.4, False, [0, len(idx2)])
    m, l, o = A.merge_states(*st1[-1], *st2[-1])
    assert np.abs(o / l[:, None] - ref_o).max() < 1e-13
    assert np.abs(m + np.log(l) - ref_l).max() < 1e-13


def test_dropping_alpha_breaks_exactness():
    q, k, v = rand_qkv(15, 1, 1, 256, 16)
    q = 3.0 * q
    edges = list(range(0, 257, 32))
    ref_o, _ = A.attention_head_fp64(q[0, 0], k[0, 0], v[0, 0], 0.25, False)
    good, _, _ = A.online_softmax_attention(q[0, 0], k[0, 0], v[0, 0], 0.25, False, edges)
    bad, _, _ = A.online_softmax_attention(q[0, 0], k[0, 0], v[0, 0], 0.25, False, edges, _rescale=False)
    assert np.abs(good - ref_o).max() < 1e-13
    assert np.abs(bad - ref_o).max() > 0.1


def test_scale_is_applied_to_scores():
    q, k, v = rand_qkv(16, 1, 1, 20, 8)
    o1, l1 = A.attention_fp64(q, k, v, 0.5, True)
    o2, l2 = A.attention_fp64(2.0 * q, k, v, 0.25, True)
    assert np.abs(o1 - o2).max() < 1e-13 and np.abs(l1 - l2).max() < 1e-13
    o3, _ = A.attention_fp64(q, k, v, 0.25, True)
    assert np.abs(o1 - o3).max() > 1e-3
