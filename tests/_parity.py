"""Shared helpers for the GPU parity tests: the tolerances and whole-output comparisons.

Bounds for every parity case whose inputs are iid N(0, 1) (the five workloads, the headline
and the smaller shapes and edge cases built the same way):
- bf16 output O: max |O_gpu - O_ref| <= 1e-2 over every element, and mean <= 1e-3;
- LSE: |LSE_gpu - LSE_ref| <= 1e-4 max(1, |LSE_ref|) for every row: the relative error, with
  an absolute floor of 1e-4 for rows whose LSE is near 0. Such rows exist in the causal and
  packed workloads (|LSE_ref| down to ~1e-3, where m and log l nearly cancel): there the fp32
  rounding of the two terms alone, ~2e-7 absolute, is a relative error of ~2e-4, which no fp32
  computation avoids. The pure relative error is printed beside it;
- fp32 output (fp32 arithmetic throughout): max abs <= 2e-5, LSE relative 1e-5. fp32
  rounding (2^-24 per operation) over sums of a few hundred terms of magnitude <= 1 and the
  ~1-ulp hardware exp2 stay two orders of magnitude below this;
- FP8 output O against attention on the same dequantised E4M3 inputs (O_deq): max abs
  <= 6e-2 over every element; LSE against LSE_deq as above. Against the original fp32 inputs
  (O_true) the error of any FP8 attention on the outlier workload is 0.8 - 3 (max abs: the
  input quantisation alone moves the exact result that far), so that error is reported.

Stress inputs outside the workloads (Q scaled by 8, so that a few keys dominate each row and
|O| is near 1 on average) get one bf16 ulp of the reference added to the bound,
|dO| <= 1e-2 + 2^-8 |O_ref| element-wise and mean <= 1e-3 + mean(2^-9 |O_ref|): rounding O to
bf16 alone costs up to half an ulp, 8e-4 on average there. The plain figures are printed too.

Outputs are pre-filled with NaN before each call, so a tile the kernels never write fails the
comparison.
"""

from __future__ import annotations

import numpy as np
import torch

BF16_MAX_ABS = 1e-2
BF16_MEAN_ABS = 1e-3
LSE_REL = 1e-4
F32_MAX_ABS = 2e-5
F32_LSE_REL = 1e-5
FP8_MAX_ABS = 6e-2
BF16_ULP_REL = 2.0 ** -8


def say(*a):
    print(*a, flush=True)


def to_np(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64, copy=False)
    return t.detach().to("cpu").to(torch.float64).numpy()


def nan_out(shape, dtype, device="cuda") -> torch.Tensor:
    """An output tensor filled with NaN (a result the kernels never write stays NaN)."""
    return torch.full(tuple(shape), float("nan"), dtype=dtype, device=device)


def o_err(o_gpu, o_ref):
    d = np.abs(to_np(o_gpu) - o_ref)
    return (float(d.max()), float(d.mean())) if d.size else (0.0, 0.0)


def o_excess(o_gpu, o_ref, tol_abs) -> float:
    """Stress inputs only: max over elements of |dO| - (tol_abs + 2^-8 |O_ref|) (<= 0: within)."""
    g = to_np(o_gpu)
    if g.size == 0:
        return -tol_abs
    return float((np.abs(g - o_ref) - (tol_abs + BF16_ULP_REL * np.abs(o_ref))).max())


def lse_rel_err(lse_gpu, lse_ref) -> float:
    """max |dLSE| / |LSE_ref| over rows (rows with LSE_ref = -inf, no visible key, must match)."""
    g = to_np(lse_gpu)
    if g.size == 0:
        return 0.0
    dead = ~np.isfinite(lse_ref)
    if dead.any():
        assert np.array_equal(g[dead], lse_ref[dead]), "rows without a visible key need LSE = -inf"
    live = ~dead
    if not live.any():
        return 0.0
    return float((np.abs(g[live] - lse_ref[live]) / np.abs(lse_ref[live])).max())


def lse_floor_err(lse_gpu, lse_ref) -> float:
    """max |dLSE| / max(1, |LSE_ref|) over rows with a visible key."""
    g = to_np(lse_gpu)
    live = np.isfinite(lse_ref)
    if not live.any():
        return 0.0
    return float((np.abs(g[live] - lse_ref[live]) / np.maximum(1.0, np.abs(lse_ref[live]))).max())


class Tally:
    """Running figures of one whole-output comparison (max and mean |dO|, LSE errors)."""

    def __init__(self, label: str):
        self.label = label
        self.max = 0.0
        self.sum = 0.0
        self.count = 0
        self.lse_rel = 0.0
        self.lse_floor = 0.0
        self.where = None
        self.ref_at_max = 0.0

    def add(self, key, o_gpu, o_ref, lse_gpu=None, lse_ref=None):
        g = to_np(o_gpu)
        d = np.abs(g - o_ref)
        if d.size:
            i = int(np.argmax(d))
            if d.flat[i] > self.max or self.where is None:
                self.max = float(d.flat[i])
                self.where = (key, np.unravel_index(i, d.shape))
                self.ref_at_max = float(np.abs(o_ref).flat[i])
            self.sum += float(d.sum())
            self.count += d.size
        if lse_ref is not None:
            self.lse_rel = max(self.lse_rel, lse_rel_err(lse_gpu, lse_ref))
            self.lse_floor = max(self.lse_floor, lse_floor_err(lse_gpu, lse_ref))

    @property
    def mean(self) -> float:
        return self.sum / max(1, self.count)

    def report(self):
        say(f"  {self.label}: {self.count} elements, max|dO|={self.max:.4g} (at {self.where}, |O_ref|="
            f"{self.ref_at_max:.3g}) mean|dO|={self.mean:.3g} LSE rel={self.lse_rel:.3g} "
            f"(max(1,|LSE|) form {self.lse_floor:.3g})")

    def check(self, max_abs=BF16_MAX_ABS, mean_abs=BF16_MEAN_ABS, lse_rel=LSE_REL):
        self.report()
        assert self.count > 0
        assert self.max <= max_abs, f"{self.label}: max|dO| {self.max:.4g} > {max_abs}"
        assert self.mean <= mean_abs, f"{self.label}: mean|dO| {self.mean:.4g} > {mean_abs}"
        assert self.lse_floor <= lse_rel, f"{self.label}: LSE error {self.lse_floor:.3g} > {lse_rel} max(1, |LSE|)"


def all_finite(*ts):
    """Every element written (the outputs started as NaN) and finite."""
    for t in ts:
        if t is not None:
            assert bool(torch.isfinite(t).all()), "an output element is NaN or infinite (not written?)"


def compare_heads(o, lse, ref_head, heads, label: str) -> Tally:
    """Compare o [.., N, d] and lse [.., N] (GPU) with ref_head(b, h) -> (O_ref, LSE_ref) for
    every (b, h) in heads; returns the tally (not yet checked)."""
    all_finite(o, lse)
    oc = o.float().cpu()
    lc = lse.cpu() if lse is not None else None
    t = Tally(label)
    for b, h in heads:
        o_ref, lse_ref = ref_head(b, h)
        t.add((b, h), oc[b, h], o_ref, None if lc is None else lc[b, h], None if lc is None else lse_ref)
    return t


def sample_rows(n: int, count: int, seed: int) -> np.ndarray:
    """Sorted query rows to check: the first and last rows, tile edges, and random rows."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, n // 2, n - 65, n - 64, n - 2, n - 1]
    rows = set(r for r in fixed if 0 <= r < n)
    rows.update(rng.choice(n, size=min(count, n), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)
