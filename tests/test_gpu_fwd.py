"""GPU parity of fa_fwd (fp32 and bf16) against the float64 oracle, through the C ABI.

Every workload (the tiny fp32 case, B=4 H=16 N=2k non-causal and causal, the 16k causal long
context, the d = 64 and d = 256 head-dim sweep, the 8k headline non-causal and causal and the
short-sequence sweep) is compared element by element over its whole output: every row of
every head, against the three-pass oracle run head by head. The smaller shapes span several
tiles, ragged tails and edge lengths. Outputs start as NaN, so an unwritten tile fails.
Bounds (tests/_parity.py): bf16 max |dO| <= 1e-2, mean <= 1e-3, LSE relative <= 1e-4; the
stress inputs (Q scaled by 8) add one bf16 ulp of the reference.
"""

import numpy as np
import pytest
import torch

from exact_attention_06_amd import fa_fwd
from exact_attention_06_amd.workloads import WORKLOADS, Workload, make_qkv
from oracle.attention import attention_fp64, attention_head_fp64
from tests._parity import (BF16_MAX_ABS, BF16_MEAN_ABS, F32_LSE_REL, F32_MAX_ABS, LSE_REL, Tally, all_finite,
                           compare_heads, lse_rel_err, nan_out, o_err, o_excess, sample_rows, say, to_np)

pytestmark = pytest.mark.gpu


def run_gpu(q, k, v, causal, scale=None, stream=None):
    """fa_fwd on NaN-filled outputs; returns (o, lse) on the GPU."""
    B, H, N, d = q.shape
    o = nan_out(q.shape, q.dtype)
    lse = nan_out((B, H, N), torch.float32)
    fa_fwd(q.cuda(), k.cuda(), v.cuda(), o, lse, causal=causal, scale=scale, stream=stream)
    torch.cuda.synchronize()
    return o, lse


def check_full(q, k, v, causal, dtype, scale=None, stress=False):
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    o, lse = run_gpu(q, k, v, causal, scale)
    all_finite(o, lse)
    o_ref, lse_ref = attention_fp64(q, k, v, scale, causal)
    t = Tally(f"{dtype} {tuple(q.shape)} causal={causal}")
    t.add(None, o.float().cpu(), o_ref, lse.cpu(), lse_ref)
    if dtype == "f32":
        t.check(F32_MAX_ABS, F32_MAX_ABS, F32_LSE_REL)
    elif stress:
        # Q scaled by 8: |O| near 1, where the bf16 output alone costs up to half an ulp
        t.report()
        ex = o_excess(o.float().cpu(), o_ref, BF16_MAX_ABS)
        mean_tol = BF16_MEAN_ABS + float(np.mean(np.abs(o_ref))) * 2.0 ** -9
        say(f"  stress bound: excess over 1e-2 + 2^-8|O_ref| {ex:.3g}, mean bound {mean_tol:.3g}")
        assert ex <= 0 and t.mean <= mean_tol and t.lse_floor <= LSE_REL
    else:
        t.check()
    return o, lse


SMALL = [  # (B, H, N, d): several 128-query / 64-key tiles, ragged tails, edge lengths
    (2, 3, 300, 64), (2, 3, 300, 128), (1, 2, 200, 256), (1, 1, 1, 128), (1, 1, 63, 64),
    (1, 2, 129, 128), (1, 1, 64, 256), (1, 1, 65, 256), (3, 1, 257, 128), (1, 2, 1000, 64),
    # d = 128 at N >= 2048 takes the 256-query (8-wave) workgroups when non-causal
    (1, 1, 2048, 128), (1, 2, 2100, 128),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SMALL)
def test_bf16_small_full_compare(shape, causal):
    B, H, N, d = shape
    say(f"bf16 {shape} causal={causal}")
    q, k, v = make_qkv(B, H, N, d, seed=100 + N + d, dtype="bf16")
    check_full(q, k, v, causal, "bf16")


# grids of many more workgroups than the GPU holds at once, with ragged lengths: 8-wave
# (N >= 2048) and 4-wave (d = 64, d = 128 below 2048) workgroups, workgroup counts that are
# multiples of 8 (contiguous per-XCD ranges in the remap) and ones that are not
LARGE_GRIDS = [(3, 100, 700, 128), (2, 100, 2100, 128), (2, 150, 1000, 64), (1, 257, 700, 128), (1, 37, 2085, 128)]


@pytest.mark.parametrize("shape", LARGE_GRIDS)
def test_bf16_large_grid_full_compare(shape):
    B, H, N, d = shape
    say(f"bf16 large grid {shape}")
    q, k, v = make_qkv(B, H, N, d, seed=600 + N + H, dtype="bf16")
    o, lse = run_gpu(q, k, v, False)
    t = compare_heads(o, lse, lambda b, h: attention_head_fp64(q[b, h], k[b, h], v[b, h], d ** -0.5, False),
                      [(b, h) for b in range(B) for h in range(H)], f"large grid {shape}")
    t.check()


# causal grids with 16 or more heads per XCD walk the heads in groups, each group query block
# first (launch_fwd_kernel picks the group size): 8-wave d = 128 with a ragged last block (4 of
# the XCD's 16 heads per group), 4-wave d = 128 below 2048 (16 of 32) and d = 64 (4 of 16);
# and a causal d = 256 grid, whose order is head by head
HEAD_GROUP_GRIDS = [(8, 16, 2100, 128), (16, 16, 1024, 128), (8, 16, 4096, 64),
                    # d = 256 walks each XCD's heads one after another (costliest block first)
                    (2, 16, 1100, 256)]


@pytest.mark.parametrize("shape", HEAD_GROUP_GRIDS)
def test_causal_head_groups_whole_output(shape):
    B, H, N, d = shape
    say(f"bf16 causal head groups {shape}")
    q, k, v = make_qkv(B, H, N, d, seed=650 + N + d, dtype="bf16")
    o, lse = run_gpu(q, k, v, True)
    t = compare_heads(o, lse, lambda b, h: attention_head_fp64(q[b, h], k[b, h], v[b, h], d ** -0.5, True),
                      [(b, h) for b in range(B) for h in range(H)], f"causal head groups {shape}")
    t.check()


# N <= 128 at d = 64 and 128 runs the short-sequence kernel (a whole head in one workgroup's
# LDS, exact two-pass softmax): lengths from one key to the full 128, with ragged last blocks
SHORT = [(2, 3, 1, 64), (1, 2, 17, 128), (2, 2, 32, 64), (1, 3, 33, 128), (1, 2, 64, 128), (2, 1, 100, 64),
         (1, 2, 127, 128), (3, 2, 128, 64), (2, 2, 128, 128)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", SHORT)
def test_bf16_short_full_compare(shape, causal):
    B, H, N, d = shape
    say(f"bf16 short {shape} causal={causal}")
    q, k, v = make_qkv(B, H, N, d, seed=400 + N + d, dtype="bf16")
    check_full(q, k, v, causal, "bf16")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_short_peaked_softmax(d, causal):
    """The short kernel's scores up to about +-40 (Q scaled by 8): rows dominated by a few
    keys, where a row max taken over too few keys would overflow or lose the row."""
    say(f"bf16 short peaked d={d} causal={causal}")
    q, k, v = make_qkv(2, 2, 120, d, seed=500 + d, dtype="bf16")
    check_full((q.float() * 8).to(torch.bfloat16), k, v, causal, "bf16", stress=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_bf16_peaked_softmax(d, causal):
    """Q scaled by 8 (exact in bf16): scores up to about +-40, each row dominated by a few
    keys, and the running max moves by more than the rescale threshold (2^8 in exp2 units)
    from block to block, so the accumulator-rescale branch runs often. |O| is near 1 here
    (mean 0.6), so rounding O to bf16 alone costs a mean of 8e-4: a stress case."""
    say(f"bf16 peaked d={d} causal={causal}")
    q, k, v = make_qkv(1, 2, 700, d, seed=300 + d, dtype="bf16")
    check_full((q.float() * 8).to(torch.bfloat16), k, v, causal, "bf16", stress=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 256, 64), (2, 1, 300, 128), (1, 1, 130, 256), (1, 1, 5, 64)])
def test_f32_small_full_compare(shape, causal):
    B, H, N, d = shape
    say(f"f32 {shape} causal={causal}")
    q, k, v = make_qkv(B, H, N, d, seed=200 + N + d, dtype="f32")
    check_full(q, k, v, causal, "f32")


def test_tiny_f32_workload():
    w = WORKLOADS["tiny_f32"]
    say(f"workload {w.name}")
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.seed, "f32")
    o, lse = check_full(q, k, v, False, "f32")
    assert o.shape == (1, 2, 256, 64) and lse.shape == (1, 2, 256) and o.dtype == torch.float32


def check_workload_whole(w, causal):
    """Every element of the workload's output against the oracle, head by head."""
    say(f"workload {w.name} causal={causal} (whole output)")
    q, k, v = make_qkv(w.B, w.H, w.N, w.d, w.seed, w.dtype)
    o, lse = run_gpu(q, k, v, causal)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    t = compare_heads(o, lse, lambda b, h: attention_head_fp64(q[b, h], k[b, h], v[b, h], w.scale, causal), heads,
                      f"{w.name} causal={causal}")
    t.check()


@pytest.mark.parametrize("name,causal", [
    ("b4h16n2k_d128", False), ("b4h16n2k_d128", True), ("long_n16k_d128", True),
    ("b8h16n4k_d64", False), ("b8h16n4k_d256", False),
    ("b4h16n8k_d128", False), ("b4h16n8k_d128", True),
    ("short_b64h16n128_d128", False), ("short_b64h16n128_d128", True), ("short_b64h16n256_d128", False),
    ("short_b64h16n512_d128", False),
])
def test_workload_whole_output(name, causal):
    check_workload_whole(WORKLOADS[name], causal)


@pytest.mark.parametrize("B,H,N,d,causal", [(1, 2, 65536, 128, False), (1, 2, 65536, 128, True),
                                            (1, 1, 131072, 64, True)])
def test_very_long_sequences_sampled(B, H, N, d, causal):
    """Row offsets and per-head byte counts far beyond the workloads: every element written
    and finite, and sampled rows (each the oracle's exact row) within the bounds."""
    w = Workload(f"long_b{B}h{H}n{N}_d{d}", B, H, N, d, "bf16", (causal,), 21)
    say(f"{w.name} causal={causal} (sampled rows)")
    q, k, v = make_qkv(B, H, N, d, w.seed, "bf16")
    o, lse = run_gpu(q, k, v, causal)
    all_finite(o, lse)
    t = Tally(f"{w.name} sampled")
    for b in range(B):
        for h in range(H):
            rows = sample_rows(N, 96, seed=b * 1000 + h)
            o_ref, lse_ref = attention_head_fp64(q[b, h], k[b, h], v[b, h], w.scale, causal, rows=rows)
            idx = torch.from_numpy(rows).cuda()
            t.add((b, h), o[b, h][idx].float().cpu(), o_ref, lse[b, h][idx].cpu(), lse_ref)
    t.check()


# ---------------------------------------------------------------- closed forms on the GPU

@pytest.mark.parametrize("d", [64, 128, 256])
def test_uniform_scores_give_mean_of_values(d):
    say(f"uniform scores d={d}")
    _, k, v = make_qkv(1, 2, 333, d, seed=7, dtype="bf16")
    q = torch.zeros_like(k)
    o, lse = run_gpu(q, k, v, False)
    vm = to_np(v).mean(axis=2, keepdims=True)
    assert o_err(o, np.broadcast_to(vm, o.shape))[0] <= BF16_MAX_ABS
    assert np.abs(to_np(lse) - np.log(333)).max() <= LSE_REL * np.log(333)
    oc, lc = run_gpu(q, k, v, True)
    cm = np.cumsum(to_np(v), axis=2) / np.arange(1, 334)[None, None, :, None]
    assert o_err(oc, cm)[0] <= BF16_MAX_ABS
    # row 0 has LSE = ln 1 = 0 exactly; the others ln(i + 1)
    lref = np.log(np.arange(1, 334))[None, None]
    assert np.abs(to_np(lc) - lref).max() <= LSE_REL * np.log(2)
    assert lse_rel_err(lc[:, :, 1:], np.broadcast_to(lref[:, :, 1:], lc[:, :, 1:].shape)) <= LSE_REL


def test_causal_first_row_equals_first_value():
    q, k, v = make_qkv(2, 2, 190, 128, seed=8, dtype="bf16")
    o, _ = run_gpu(q, k, v, True)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


# ---------------------------------------------------------------- launch properties

def test_deterministic_and_stream():
    q, k, v = make_qkv(2, 4, 777, 128, seed=9, dtype="bf16")
    o1, l1 = run_gpu(q, k, v, True)
    o2, l2 = run_gpu(q, k, v, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o3, l3 = run_gpu(q, k, v, True, stream=s)
    s.synchronize()
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_empty_and_no_lse():
    q = torch.empty(2, 3, 0, 128, dtype=torch.bfloat16, device="cuda")
    o, lse = fa_fwd(q, q, q)
    torch.cuda.synchronize()
    assert o.shape == q.shape and lse.shape == (2, 3, 0)
    # without LSE the outputs are the same (N = 100: short-sequence kernel; 300: streaming)
    for n, d in ((100, 64), (300, 128)):
        q, k, v = make_qkv(1, 1, n, d, seed=10, dtype="bf16")
        o1 = nan_out(q.shape, q.dtype)
        fa_fwd(q.cuda(), k.cuda(), v.cuda(), o1, want_lse=False)
        o2, _ = fa_fwd(q.cuda(), k.cuda(), v.cuda())
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)


def test_scale_argument():
    q, k, v = make_qkv(1, 2, 150, 64, seed=11, dtype="bf16")
    check_full(q, k, v, True, "bf16", scale=0.3)
    check_full(q, k, v, False, "bf16", scale=0.01)
