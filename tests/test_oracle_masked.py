"""Pins of the grouped-head / sliding-window / packed-sequence oracle (CPU, float64).

- with no window, no packing and one key/value head per query head it is the pinned forward
  oracle, causal and not;
- the causal window of Exercise 5 (FA2/3 page), w keys ending at the query, computed row by
  row from each row's own key range, equals the window (w - 1, 0);
- closed forms: the window (0, 0) lets every query see only itself, so O = V and
  LSE_i = scale q_i . k_i; windows wider than the sequence change nothing;
- a pure-Python brute force of a two-sided non-causal window on a tiny case;
- packed sequences: each sequence equals the forward oracle run on it alone, and changing the
  keys and values of one sequence leaves the others unchanged (no attention across the
  boundaries); empty sequences are allowed;
- grouped heads equal the key/value heads repeated Hq / Hkv times;
- the visible-pair count equals the number of True entries of the mask;
- the sampled-rows form equals the full form on those rows.
"""

import math

import numpy as np
import pytest

from oracle.attention import attention_fp64
from oracle.masked import attention_ext_fp64, attention_ext_rows_fp64, visible_mask, visible_pairs


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_plain_case_is_the_forward_oracle(causal):
    q, k, v = _rand(1, 2, 3, 45, 16), _rand(2, 2, 3, 45, 16), _rand(3, 2, 3, 45, 16)
    o, lse = attention_ext_fp64(q, k, v, 0.3, causal)
    o2, lse2 = attention_fp64(q, k, v, 0.3, causal)
    assert np.allclose(o, o2, rtol=0, atol=1e-13) and np.allclose(lse, lse2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("w", [1, 7, 48, 200])
def test_causal_window_of_w_keys_row_by_row(w):
    """The sliding window of Exercise 5 on "FlashAttention 2 & 3: Work Partitioning, Warp
    Specialization & FP8": query i sees the w keys max(0, i - w + 1) .. i. Each row is
    computed on its own from that range alone (a softmax over just those scores, in float64,
    with the logsumexp from math.fsum), which must equal the oracle's window (w - 1, 0)."""
    n, d = 96, 16
    q, k, v = _rand(4, n, d), _rand(5, n, d), _rand(6, n, d)
    scale = 1 / math.sqrt(d)
    o, lse = attention_ext_fp64(q[None, None], k[None, None], v[None, None], scale, True, (w - 1, 0))
    for i in range(n):
        keys = range(max(0, i - w + 1), i + 1)
        scores = [scale * float(np.dot(q[i], k[j])) for j in keys]
        top = max(scores)
        weights = [math.exp(x - top) for x in scores]
        total = math.fsum(weights)
        row = sum(wt * v[j] for wt, j in zip(weights, keys)) / total
        assert np.allclose(o[0, 0, i], row, rtol=0, atol=1e-13)
        assert abs(lse[0, 0, i] - (top + math.log(total))) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_window_zero_sees_only_itself(causal):
    q, k, v = _rand(7, 1, 2, 30, 8), _rand(8, 1, 2, 30, 8), _rand(9, 1, 2, 30, 8)
    o, lse = attention_ext_fp64(q, k, v, 0.5, causal, (0, 0))
    assert np.allclose(o, v, rtol=0, atol=1e-14)
    assert np.allclose(lse, 0.5 * np.einsum("bhnd,bhnd->bhn", q, k), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_wide_window_changes_nothing(causal):
    q, k, v = _rand(10, 1, 2, 40, 8), _rand(11, 1, 2, 40, 8), _rand(12, 1, 2, 40, 8)
    a = attention_ext_fp64(q, k, v, 0.4, causal, (39, 39))
    b = attention_ext_fp64(q, k, v, 0.4, causal, (-1, -1))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_two_sided_window_brute_force():
    n, d, left, right, scale = 11, 4, 3, 2, 0.7
    q, k, v = _rand(13, n, d), _rand(14, n, d), _rand(15, n, d)
    o, lse = attention_ext_fp64(q[None, None], k[None, None], v[None, None], scale, False, (left, right))
    for i in range(n):
        keys = [j for j in range(n) if i - left <= j <= i + right]
        sc = [scale * sum(q[i, c] * k[j, c] for c in range(d)) for j in keys]
        mx = max(sc)
        ws = [math.exp(x - mx) for x in sc]
        tot = sum(ws)
        for c in range(d):
            assert abs(o[0, 0, i, c] - sum(wj * v[j, c] for wj, j in zip(ws, keys)) / tot) <= 1e-13
        assert abs(lse[0, 0, i] - (mx + math.log(tot))) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_packed_sequences_are_independent(causal):
    cu = [0, 13, 13, 50, 64]          # an empty sequence in the middle
    q, k, v = _rand(16, 1, 4, 64, 8), _rand(17, 1, 2, 64, 8), _rand(18, 1, 2, 64, 8)
    o, lse = attention_ext_fp64(q, k, v, 0.3, causal, (-1, -1), cu)
    for a, c in zip(cu[:-1], cu[1:]):
        if c == a:
            continue
        o2, lse2 = attention_ext_fp64(q[:, :, a:c], k[:, :, a:c], v[:, :, a:c], 0.3, causal)
        assert np.allclose(o[:, :, a:c], o2, rtol=0, atol=1e-13)
        assert np.allclose(lse[:, :, a:c], lse2, rtol=0, atol=1e-13)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 13:50] += 1.0
    v2[:, :, 13:50] -= 2.0
    o3, _ = attention_ext_fp64(q, k2, v2, 0.3, causal, (-1, -1), cu)
    assert np.array_equal(o3[:, :, :13], o[:, :, :13]) and np.array_equal(o3[:, :, 50:], o[:, :, 50:])
    assert np.abs(o3[:, :, 13:50] - o[:, :, 13:50]).max() > 0.1


def test_packed_window_counts_from_the_sequence_start():
    cu = [0, 20, 45]
    q, k, v = _rand(19, 1, 1, 45, 8), _rand(20, 1, 1, 45, 8), _rand(21, 1, 1, 45, 8)
    o, _ = attention_ext_fp64(q, k, v, 0.3, True, (5, 0), cu)
    o2, _ = attention_ext_fp64(q[:, :, 20:], k[:, :, 20:], v[:, :, 20:], 0.3, True, (5, 0))
    assert np.allclose(o[:, :, 20:], o2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("window", [(-1, -1), (9, 0), (4, 6)])
def test_grouped_heads_equal_repeated_heads(window):
    q = _rand(22, 2, 6, 33, 8)
    k, v = _rand(23, 2, 2, 33, 8), _rand(24, 2, 2, 33, 8)
    a = attention_ext_fp64(q, k, v, 0.35, window[1] == 0, window)
    b = attention_ext_fp64(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), 0.35, window[1] == 0, window)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("n,causal,left,right", [(50, True, -1, -1), (50, False, -1, -1), (50, True, 9, 0),
                                                 (50, False, 4, 6), (7, False, 0, 0), (64, True, 100, -1)])
def test_visible_pairs(n, causal, left, right):
    assert visible_pairs(n, causal, left, right) == int(visible_mask(n, causal, left, right).sum())


@pytest.mark.parametrize("causal,window", [(True, (-1, -1)), (True, (20, 0)), (False, (7, 12)), (False, (-1, -1))])
def test_sampled_rows_equal_full(causal, window):
    q = _rand(25, 2, 4, 70, 8)
    k, v = _rand(26, 2, 2, 70, 8), _rand(27, 2, 2, 70, 8)
    o, lse = attention_ext_fp64(q, k, v, 0.3, causal, window)
    rows = [0, 5, 31, 32, 69]
    o2, lse2 = attention_ext_rows_fp64(q, k, v, 0.3, causal, window, 1, 3, rows)
    assert np.allclose(o2, o[1, 3, rows], rtol=0, atol=1e-13) and np.allclose(lse2, lse[1, 3, rows], rtol=0, atol=1e-13)
