"""Pins of the decoding oracle (CPU, float64).

- Nq = Nk with one key/value head per query head is ordinary attention: equal to the pinned
  forward oracle, causal and not (the decode mask is the forward's mask when Nq = Nk);
- a library route on tiny inputs: torch float64 softmax with the mask built from its
  definition (key j hidden from query i iff j > Nk - Nq + i);
- grouped heads: the same as repeating every key/value head Hq / Hkv times;
- closed forms: with Q = 0 every visible key gets the same weight, so O_i is the mean of the
  values query i sees and LSE_i = ln(count), count = Nk (non-causal) or Nk - Nq + i + 1;
- the last query under the causal mask sees every key (equal to the non-causal row);
- the split-key form (partial states over arbitrary key ranges, including ranges that some
  queries cannot see at all, merged with the page-5 formula) equals the three-pass result.
"""

import numpy as np
import pytest
import torch

from oracle.attention import attention_fp64
from oracle.decode import (attention_decode_fp64, decode_head_fp64, decode_head_split_fp64,
                           partial_state_fp64)


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_forward_oracle(causal):
    q, k, v = _rand(1, 2, 3, 37, 16), _rand(2, 2, 3, 37, 16), _rand(3, 2, 3, 37, 16)
    o, lse = attention_decode_fp64(q, k, v, 0.3, causal)
    o2, lse2 = attention_fp64(q, k, v, 0.3, causal)
    assert np.allclose(o, o2, rtol=0, atol=1e-12) and np.allclose(lse, lse2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_softmax(causal):
    q, k, v = _rand(4, 5, 8), _rand(5, 23, 8), _rand(6, 23, 8)
    o, lse = decode_head_fp64(q, k, v, 0.4, causal)
    qt, kt, vt = (torch.from_numpy(x) for x in (q, k, v))
    s = 0.4 * qt @ kt.T
    if causal:
        i = torch.arange(5)[:, None]
        j = torch.arange(23)[None, :]
        s = s.masked_fill(j > 23 - 5 + i, float("-inf"))
    assert np.allclose(o, (torch.softmax(s, dim=1) @ vt).numpy(), rtol=0, atol=1e-13)
    assert np.allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_heads_equal_repeated_heads(causal):
    q = _rand(7, 2, 8, 3, 16)        # Hq = 8
    k, v = _rand(8, 2, 2, 50, 16), _rand(9, 2, 2, 50, 16)   # Hkv = 2
    o, lse = attention_decode_fp64(q, k, v, 0.25, causal)
    o2, lse2 = attention_decode_fp64(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.25, causal)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # and a query head of group 1 differs from what key/value head 0 would give
    o3, _ = decode_head_fp64(q[0, 5], k[0, 0], v[0, 0], 0.25, causal)
    assert np.abs(o3 - o[0, 5]).max() > 1e-3


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_closed_form(causal):
    nq, nk = 4, 19
    q = np.zeros((nq, 8))
    k, v = _rand(10, nk, 8), _rand(11, nk, 8)
    o, lse = decode_head_fp64(q, k, v, 1.0, causal)
    for i in range(nq):
        cnt = nk - nq + i + 1 if causal else nk
        assert np.allclose(o[i], v[:cnt].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(lse[i] - np.log(cnt)) <= 1e-13


def test_last_query_sees_every_key():
    q, k, v = _rand(12, 6, 8), _rand(13, 40, 8), _rand(14, 40, 8)
    oc, lc = decode_head_fp64(q, k, v, 0.5, True)
    on, ln_ = decode_head_fp64(q, k, v, 0.5, False)
    assert np.allclose(oc[-1], on[-1], rtol=0, atol=1e-13) and abs(lc[-1] - ln_[-1]) <= 1e-13
    assert np.abs(oc[0] - on[0]).max() > 1e-3     # the first query does not


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("edges", [[0, 100], [0, 1, 2, 100], [0, 33, 64, 65, 97, 100], [0, 50, 96, 100]])
def test_split_merge_equals_three_pass(causal, edges):
    # with causal and Nq = 6, queries 0..2 cannot see keys 95..99: the range [96, 100) is
    # empty for some of them and must drop out of the merge
    q, k, v = _rand(15, 6, 16), _rand(16, 100, 16), _rand(17, 100, 16)
    o, lse = decode_head_fp64(q, k, v, 0.3, causal)
    o2, lse2 = decode_head_split_fp64(q, k, v, 0.3, causal, edges)
    assert np.allclose(o, o2, rtol=0, atol=1e-12) and np.allclose(lse, lse2, rtol=0, atol=1e-12)


def test_partial_state_of_invisible_range_is_empty():
    q, k, v = _rand(18, 4, 8), _rand(19, 30, 8), _rand(20, 30, 8)
    m, l, o = partial_state_fp64(q, k, v, 1.0, True, 28, 30)   # query i sees keys <= 26 + i
    assert np.isneginf(m[0]) and l[0] == 0 and not o[0].any()        # query 0 sees neither
    assert np.isfinite(m[3]) and l[3] > 0                             # query 3 sees both
