"""fa_decode_noalloc, the decoding entry point that allocates nothing, against fa_decode (the
same kernels with a caller-provided workspace), through the C ABI.

Two calls in a row on one stream: the first uses the whole static scratch (the largest
workspace any shape needs: 255 sequences, one key/value head, 32 query rows, 512 keys, 510
splits in all), the second a smaller problem with fewer splits, so that it runs over the first
call's stale states. Each must equal fa_decode's output bit for bit, and the oracle within the
forward's bounds.
"""

import ctypes

import pytest
import torch

from exact_attention_06_amd import fa_decode, fa_decode_workspace_size, lib
from exact_attention_06_amd.workloads import make_decode_inputs
from oracle.decode import attention_decode_fp64
from tests._parity import Tally, all_finite, nan_out, say

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 8486400


def noalloc(q, k, v, causal):
    """One call of the C entry point on the current stream, into NaN-filled outputs."""
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    o = nan_out(q.shape, torch.bfloat16)
    lse = nan_out((B, Hq, Nq), torch.float32)
    st = lib().fa_decode_noalloc(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                 ctypes.c_void_p(v.data_ptr()), ctypes.c_void_p(o.data_ptr()),
                                 ctypes.c_void_p(lse.data_ptr()), B, Hq, Hkv, Nq, Nk, d, d ** -0.5, int(causal), 1,
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, st
    return o, lse


def test_noalloc_equals_decode_on_two_calls():
    cases = [((255, 1, 1, 32, 512, 128), True, 51), ((2, 8, 2, 3, 3000, 128), False, 52)]
    for (B, Hq, Hkv, Nq, Nk, d), causal, seed in cases:
        need = fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d)
        say(f"noalloc decode {(B, Hq, Hkv, Nq, Nk, d)} causal={causal}: workspace {need} B")
        assert 0 < need <= SCRATCH_BYTES
        q, k, v = (x.cuda() for x in make_decode_inputs(B, Hq, Hkv, Nq, Nk, d, seed))
        o, lse = noalloc(q, k, v, causal)
        o_ws, lse_ws = fa_decode(q, k, v, causal=causal)
        torch.cuda.synchronize()
        all_finite(o, lse)
        assert torch.equal(o, o_ws) and torch.equal(lse, lse_ws)
        o_ref, lse_ref = attention_decode_fp64(q.cpu(), k.cpu(), v.cpu(), d ** -0.5, causal)
        t = Tally(f"noalloc {(B, Hq, Hkv, Nq, Nk, d)}")
        t.add(None, o.float().cpu(), o_ref, lse.cpu(), lse_ref)
        t.check()
    assert SCRATCH_BYTES == fa_decode_workspace_size(255, 1, 1, 32, 512, 128)
