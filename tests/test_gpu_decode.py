"""GPU parity of split-key decoding (fa_decode) against the float64 decoding oracle, through
the C ABI.

Bounds: the forward's bf16 bounds (tests/_parity.py): max |O_gpu - O_ref| <= 1e-2 and mean
<= 1e-3 over every element, LSE relative error <= 1e-4. The arithmetic is
the forward's (bf16 products, fp32 accumulation, P rounded to bf16 for the PV product, l summed
from fp32 P); the merge of the splits' states adds a few fp32 roundings.
Decoding outputs are small, so every case compares every output row with the oracle, the
full-size workloads included; outputs start as NaN.
"""

import numpy as np
import pytest
import torch

from exact_attention_06_amd import fa_decode, fa_decode_workspace_size, fa_fwd
from exact_attention_06_amd.workloads import DECODE_WORKLOADS, make_decode_inputs, make_qkv
from oracle.decode import attention_decode_fp64
from tests._parity import BF16_MAX_ABS, Tally, all_finite, nan_out, to_np

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def check(name, o, lse, o_ref, lse_ref):
    all_finite(o, lse)
    t = Tally(name)
    t.add(None, o.float().cpu(), o_ref, lse.cpu(), lse_ref)
    t.check()


def run(q, k, v, causal, ws=None):
    o = nan_out(q.shape, torch.bfloat16)
    lse = nan_out(q.shape[:3], torch.float32)
    fa_decode(q.cuda(), k.cuda(), v.cuda(), o, lse, workspace=ws, causal=causal)
    torch.cuda.synchronize()
    return o, lse


SHAPES = [  # (B, Hq, Hkv, Nq, Nk, d): one split and several, ragged caches, short caches,
            # more than 32 query rows per key/value head (two column groups), many queries
    (2, 8, 2, 1, 4096, 128), (1, 4, 4, 1, 1000, 128), (3, 6, 3, 1, 37, 64), (1, 2, 1, 1, 1, 128),
    (2, 16, 2, 5, 3000, 128), (1, 64, 1, 1, 2048, 64), (1, 2, 2, 7, 7, 128), (2, 4, 1, 3, 517, 64),
    (1, 8, 8, 32, 5000, 128),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHAPES)
def test_decode_small_full_compare(shape, causal):
    B, Hq, Hkv, Nq, Nk, d = shape
    say(f"decode {shape} causal={causal} workspace={fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d)} B")
    q, k, v = make_decode_inputs(B, Hq, Hkv, Nq, Nk, d, seed=300 + Nk + Nq)
    o, lse = run(q, k, v, causal)
    o_ref, lse_ref = attention_decode_fp64(q, k, v, d ** -0.5, causal)
    check(str(shape), o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("name", list(DECODE_WORKLOADS))
def test_decode_workloads_every_row(name):
    w = DECODE_WORKLOADS[name]
    say(f"decode workload {name}")
    q, k, v = make_decode_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.seed)
    o, lse = run(q, k, v, w.causal)
    o_ref, lse_ref = attention_decode_fp64(q, k, v, w.scale, w.causal)
    check(name, o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("Nq,causal", [(1, False), (3, True)])
def test_decode_very_long_cache(Nq, causal):
    # 262144 keys: 8192 tiles, the split count at its cap of 64
    B, Hq, Hkv, Nk, d = 1, 8, 2, 262144, 128
    say(f"decode long cache Nk={Nk} Nq={Nq} causal={causal}, workspace {fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d)} B")
    q, k, v = make_decode_inputs(B, Hq, Hkv, Nq, Nk, d, seed=33 + Nq)
    o, lse = run(q, k, v, causal)
    o_ref, lse_ref = attention_decode_fp64(q, k, v, d ** -0.5, causal)
    check(f"Nk={Nk}", o, lse, o_ref, lse_ref)


def test_decode_equals_forward_when_lengths_match():
    # Nq = Nk with one key/value head per query head is the forward problem
    B, H, N, d = 1, 3, 300, 128
    q, k, v = make_qkv(B, H, N, d, 41)
    for causal in (False, True):
        o, lse = run(q, k, v, causal)
        of, lf = fa_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal)
        torch.cuda.synchronize()
        assert float((o.float() - of.float()).abs().max()) <= 2 * BF16_MAX_ABS   # each within 1e-2 of the oracle
        assert float((lse - lf).abs().max()) <= 2e-4 * max(1.0, float(lf.abs().max()))


def test_decode_uniform_scores_closed_form():
    B, Hq, Hkv, Nq, Nk, d = 2, 8, 2, 2, 3333, 128
    _, k, v = make_decode_inputs(B, Hq, Hkv, Nq, Nk, d, 5)
    q = torch.zeros(B, Hq, Nq, d, dtype=torch.bfloat16)
    o, lse = run(q, k, v, False)
    mean_v = to_np(v).mean(axis=2)                                   # [B, Hkv, d]
    ref = np.repeat(mean_v, Hq // Hkv, axis=1)[:, :, None, :].repeat(Nq, axis=2)
    check("uniform", o, lse, ref, np.full((B, Hq, Nq), np.log(Nk)))


def test_decode_deterministic_and_reuses_workspace():
    B, Hq, Hkv, Nq, Nk, d = 4, 8, 2, 1, 8192, 128
    q, k, v = make_decode_inputs(B, Hq, Hkv, Nq, Nk, d, 6)
    need = fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d)
    assert need > 0
    ws = torch.full((need + 4096,), 255, dtype=torch.uint8, device="cuda")   # stale contents, larger than needed
    a = run(q, k, v, False, ws)
    b = run(q, k, v, False, ws)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_decode_empty_problem():
    q = torch.empty((1, 4, 0, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((1, 2, 16, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = fa_decode(q, k, k)
    torch.cuda.synchronize()
    assert o.numel() == 0 and lse.numel() == 0
