"""Host-side helpers of bench.py (CPU).

- the FLOP count of the grouped-head / window / packed workloads counts the (query, key)
  pairs the oracle's visibility mask allows (oracle/masked.py, itself pinned by brute force);
- the source hash that ties stored counter readings to the kernel code ignores comments and
  whitespace but not code.
"""

import pytest

import bench
from exact_attention_06_amd.workloads import EXT_WORKLOADS
from oracle.masked import visible_mask


@pytest.mark.parametrize("n,causal,left,right", [(1, False, -1, -1), (1, True, -1, -1), (37, False, -1, -1),
                                                 (37, True, -1, -1), (64, True, 15, 0), (64, False, 15, 0),
                                                 (50, False, 4, 9), (50, False, -1, 3), (50, False, 6, -1),
                                                 (33, True, 100, 100), (20, False, 0, 0)])
def test_visible_pairs_match_the_oracle_mask(n, causal, left, right):
    assert bench.visible_pairs(n, causal, left, right) == int(visible_mask(n, causal, left, right).sum())


def test_visible_pairs_of_the_benchmarked_windows():
    for name in bench.EXT_BENCH:
        w = EXT_WORKLOADS[name]
        n = 300   # the same window on a short row
        assert bench.visible_pairs(n, w.causal, *w.window) == int(visible_mask(n, w.causal, *w.window).sum()), name


def test_code_only_ignores_comments_and_spacing():
    a = "int f(int x) {  // returns x\n    return x + 1; /* one */\n}\n"
    b = "int f(int x) {\n  return x + 1;\n}"
    c = "int f(int x) { return x + 2; }"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only(c)
