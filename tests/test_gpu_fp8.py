"""GPU parity of the FP8 path (fa_prep_fp8, fa_fwd_fp8) against the oracle, through the C ABI.

- fa_prep_fp8 without rotation reproduces the oracle's codes and scales bit for bit (both
  sides compute amax, amax/448 and x/s in float32 and round to nearest even).
- With rotation, on inputs whose fast Walsh-Hadamard transform is exact in float32 (small
  integers times a power of two, with outliers) at d = 64 and d = 256, where 1/sqrt(d) is a
  power of two: the rotated values are then exact on both sides, and the GPU's codes and
  scales equal the oracle's bit for bit. On general inputs both sides rotate in float64 (the
  GPU by a fast transform, the oracle by a dense product) and round once to float32; they
  agree to ~1e-16 relative, so the float32 values, and hence the scales and codes, are the
  same unless a value lies within ~1e-15 of a rounding midpoint: bit for bit on the small
  shapes, and at most a few codes (neighbouring E4M3 values) in the 201M of the workload.
- fa_fwd_fp8 is compared with attention on the dequantised inputs (O_deq, LSE_deq) over the
  whole output: max |dO| <= 6e-2, mean <= 1e-3, LSE relative <= 1e-4. The FP8 workload is
  checked twice at full size: on the oracle's codes, and through the GPU's own rotation and
  quantisation (codes that may differ from the oracle's by one step on a few near-midpoint
  values, so the bound covers that too). The error against the original float32 inputs
  (O_true) is reported: it is dominated by the input quantisation itself.
"""

import numpy as np
import pytest
import torch

from exact_attention_06_amd import fa_fwd_fp8, fa_prep_fp8
from exact_attention_06_amd.workloads import WORKLOADS, make_fp8_exact_inputs, make_fp8_inputs
from oracle.attention import attention_head_fp64
from oracle.e4m3 import e4m3_decode
from oracle.fp8 import block_dequantize, block_quantize, fp8_inputs, fp8_reference, rotate_to_f32
from tests._parity import (BF16_MEAN_ABS, FP8_MAX_ABS, LSE_REL, Tally, all_finite, nan_out, o_err, say)

pytestmark = pytest.mark.gpu


def prep(x, signs=None):
    B, H, N, d = x.shape
    nsb = (N + 63) // 64
    x8 = torch.full((B, H, N, d), 0x7F, dtype=torch.uint8, device="cuda")   # e4m3 NaN until written
    s = nan_out((B, H, nsb), torch.float32)
    fa_prep_fp8(x.cuda(), None if signs is None else signs.cuda(), x8, s)
    torch.cuda.synchronize()
    return x8, s


def fwd(q8, k8, v8, sq, sk, sv, causal=False):
    B, H, N, d = q8.shape
    o = nan_out((B, H, N, d), torch.float32)
    lse = nan_out((B, H, N), torch.float32)
    fa_fwd_fp8(q8, k8, v8, sq, sk, sv, o, lse, causal=causal)
    torch.cuda.synchronize()
    all_finite(o, lse)
    return o, lse


@pytest.mark.parametrize("shape", [(1, 2, 200, 128), (2, 1, 64, 64), (1, 1, 130, 256)])
def test_prep_without_rotation_is_bit_exact(shape):
    say(f"prep no-rotation {shape}")
    x, _, _, _ = make_fp8_inputs(*shape, seed=21)
    x8, s = prep(x)
    codes, scales = block_quantize(x.numpy())
    assert np.array_equal(s.cpu().numpy(), scales)
    assert np.array_equal(x8.cpu().numpy(), codes)


@pytest.mark.parametrize("shape", [(2, 2, 200, 64), (1, 3, 130, 256), (1, 1, 64, 256), (1, 2, 1, 64)])
def test_prep_with_rotation_is_bit_exact_on_exact_transforms(shape):
    """Integer parity of the rotated quantiser: the rotation is exact on these inputs, so the
    codes and scales depend only on the float32 amax / 448, x / s and the E4M3 rounding."""
    say(f"prep rotation, exact transform {shape}")
    x, signs = make_fp8_exact_inputs(*shape, seed=25)
    x8, s = prep(x, signs)
    codes, scales = block_quantize(rotate_to_f32(x.numpy(), signs.numpy()))
    assert np.array_equal(s.cpu().numpy(), scales)
    g = x8.cpu().numpy()
    say(f"  codes differing: {int((g != codes).sum())} of {g.size}")
    assert np.array_equal(g, codes)


@pytest.mark.parametrize("shape", [(1, 2, 200, 128), (2, 1, 64, 64), (1, 1, 130, 256)])
def test_prep_with_rotation(shape):
    say(f"prep rotation {shape}")
    x, _, _, signs = make_fp8_inputs(*shape, seed=22)
    x8, s = prep(x, signs)
    codes, scales = block_quantize(rotate_to_f32(x.numpy(), signs.numpy()))
    assert np.array_equal(s.cpu().numpy(), scales)
    assert np.array_equal(x8.cpu().numpy(), codes)


def check_vs_deq(o, lse, o_deq, lse_deq, label, o_true=None):
    t = Tally(label)
    t.add(None, o.float().cpu(), o_deq, lse.cpu(), lse_deq)
    if o_true is not None:
        mt, _ = o_err(o.float().cpu(), o_true)
        floor, _ = o_err(o_deq, o_true)
        say(f"  vs O_true max={mt:.3g} (O_deq vs O_true {floor:.3g})")
    t.check(FP8_MAX_ABS, BF16_MEAN_ABS, LSE_REL)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 2, 300, 128), (2, 2, 128, 64), (1, 1, 200, 256), (1, 1, 1, 128),
                                   (1, 2, 2100, 128), (2, 2, 700, 256), (1, 1, 33, 256), (2, 4, 4000, 128)])
def test_fwd_fp8_small(shape, causal):
    say(f"fwd fp8 {shape} causal={causal}")
    B, H, N, d = shape
    q, k, v, signs = make_fp8_inputs(B, H, N, d, seed=23 + N)
    ref = fp8_reference(q.numpy(), k.numpy(), v.numpy(), signs.numpy(), 1.0 / np.sqrt(d), causal)
    t = {n: torch.from_numpy(ref[n]).cuda() for n in ("q8", "k8", "v8", "sq", "sk", "sv")}
    o, lse = fwd(t["q8"], t["k8"], t["v8"], t["sq"], t["sk"], t["sv"], causal)
    check_vs_deq(o, lse, ref["O_deq"], ref["LSE_deq"], f"fp8 {shape} causal={causal}", ref["O_true"])


def test_fp8_end_to_end_small():
    say("fp8 end to end (prep on GPU, then fwd)")
    q, k, v, signs = make_fp8_inputs(2, 2, 512, 128, seed=24)
    q8, sq = prep(q, signs)
    k8, sk = prep(k, signs)
    v8, sv = prep(v)
    o, lse = fwd(q8, k8, v8, sq, sk, sv)
    ref = fp8_reference(q.numpy(), k.numpy(), v.numpy(), signs.numpy(), 1 / np.sqrt(128), False)
    # the GPU quantiser may round a few near-midpoint values the other way than the oracle's
    # (float32 vs float64 rotation), so its codes may differ from the oracle's by one step there
    check_vs_deq(o, lse, ref["O_deq"], ref["LSE_deq"], "fp8 end to end", ref["O_true"])


def test_fp8_workload_whole_output():
    """The FP8 workload at full size, every element: the forward on the oracle's codes, and the
    whole GPU chain (rotation and quantisation of Q, K, V on the GPU, then the forward)."""
    w = WORKLOADS["fp8_b4h16n8k_d128"]
    say(f"workload {w.name} (whole output; oracle codes and the GPU's own)")
    q, k, v, signs = make_fp8_inputs(w.B, w.H, w.N, w.d, w.seed)
    qi = fp8_inputs(q.numpy(), k.numpy(), v.numpy(), signs.numpy())
    t = {n: torch.from_numpy(qi[n]).cuda() for n in ("q8", "k8", "v8", "sq", "sk", "sv")}
    o1, l1 = fwd(t["q8"], t["k8"], t["v8"], t["sq"], t["sk"], t["sv"])
    del t
    q8, sq = prep(q, signs)
    k8, sk = prep(k, signs)
    v8, sv = prep(v)
    o2, l2 = fwd(q8, k8, v8, sq, sk, sv)
    ncode = 0
    for a, n in ((q8, "q8"), (k8, "k8"), (v8, "v8")):
        g = a.cpu().numpy()
        diff = g != qi[n]
        ncode += int(diff.sum())
        # where codes differ (a rotated value within ~1e-15 of a midpoint) they are neighbours
        dg, dr = e4m3_decode(g[diff]), e4m3_decode(qi[n][diff])
        assert (np.abs(dg - dr) <= np.maximum(np.abs(dr), 2.0 ** -6) * 2.0 ** -3 * 1.0001).all()
    say(f"  GPU codes differing from the oracle's: {ncode} of {3 * q.numel()}")
    assert ncode <= 64
    del q8, k8, v8
    o1c, l1c, o2c, l2c = o1.float().cpu(), l1.cpu(), o2.float().cpu(), l2.cpu()
    t1, t2 = Tally(f"{w.name} on the oracle's codes"), Tally(f"{w.name} GPU prep -> GPU forward")
    true_err, floor = 0.0, 0.0
    for b in range(w.B):
        for h in range(w.H):
            qd = block_dequantize(qi["q8"][b, h], qi["sq"][b, h])
            kd = block_dequantize(qi["k8"][b, h], qi["sk"][b, h])
            vd = block_dequantize(qi["v8"][b, h], qi["sv"][b, h])
            o_deq, lse_deq = attention_head_fp64(qd, kd, vd, w.scale, False)
            t1.add((b, h), o1c[b, h], o_deq, l1c[b, h], lse_deq)
            t2.add((b, h), o2c[b, h], o_deq, l2c[b, h], lse_deq)
            if (b, h) in ((0, 0), (3, 15)):   # the original inputs' result, reported
                o_true, _ = attention_head_fp64(q[b, h], k[b, h], v[b, h], w.scale, False)
                true_err = max(true_err, o_err(o1c[b, h], o_true)[0])
                floor = max(floor, o_err(o_deq, o_true)[0])
    say(f"  heads (0,0), (3,15): vs O_true max={true_err:.3g} (O_deq vs O_true {floor:.3g})")
    t1.check(FP8_MAX_ABS, BF16_MEAN_ABS, LSE_REL)
    t2.check(FP8_MAX_ABS, BF16_MEAN_ABS, LSE_REL)
