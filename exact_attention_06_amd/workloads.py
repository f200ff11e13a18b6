"""Seeded synthetic inputs for the attention forward and backward passes.

This module only draws inputs; it holds none of the attention arithmetic, and
both the GPU path and the CPU oracle read the tensors it returns.

Recipe (the pages draw their examples with ``torch.randn``; the workloads
below have the shapes, sizes and value distributions of the benchmark cases):
- ``g = torch.Generator('cpu').manual_seed(seed)``; Q, then K, then V are drawn
  with ``torch.randn(B, H, N, d, dtype=float32, generator=g)`` (iid N(0, 1)),
  then cast to bfloat16 (round to nearest even) where the workload is bf16.
- FP8 workload: after Q, K, V, for each of Q, K, V in that order exactly
  floor(0.001 * numel) positions are chosen without replacement
  (``torch.randperm(numel, generator=g)``) and multiplied by 20 (outliers);
  then the random +-1 sign vector of the Hadamard rotation is drawn as
  ``where(torch.rand(d, generator=g) > 0.5, 1, -1)``. The signs are the only
  random numbers the method itself uses, so they are an input here.
- Exact-rotation inputs of the FP8 quantiser's bit-level test: integers in [-8, 8] times 2^-2,
  the same fraction of outliers times 20, then the signs (``make_fp8_exact_inputs``).
- Backward workloads: the output gradient dO is the fourth iid N(0, 1) draw of the same
  generator (after Q, K, V), cast to bfloat16.
- Decoding workloads: Q [B, Hq, Nq, d], then K and V [B, Hkv, Nk, d] (the key/value cache),
  iid N(0, 1) from one seeded generator in that order, cast to bfloat16.
- Grouped-head / window / packed workloads: Q [B, Hq, N, d], then K and V [B, Hkv, N, d], iid
  N(0, 1), bfloat16; packed sequence lengths are either given (the pages' example of three
  documents of 300, 1000 and 748 tokens) or cut from the same generator after V: the N
  tokens are split at nseq - 1 distinct positions drawn by torch.randperm(N - 1) + 1.
- The softmax scale is 1/sqrt(d) throughout.

Layout is [B, H, N, d], contiguous.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32", "bf16" or "fp8"
    causal: tuple       # causal settings this workload is run with
    seed: int
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def flops(self, causal: bool) -> float:
        """Counted FLOPs: 4 B H N^2 d, halved for causal."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f / 2 if causal else f


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_f32", 1, 2, 256, 64, "f32", (False,), 1,
                 "tiny reference case, fp32 in and out"),
        Workload("b4h16n2k_d128", 4, 16, 2048, 128, "bf16", (False, True), 2,
                 "bf16, non-causal and causal"),
        Workload("long_n16k_d128", 1, 32, 16384, 128, "bf16", (True,), 3,
                 "long context, causal"),
        Workload("b8h16n4k_d64", 8, 16, 4096, 64, "bf16", (False,), 4, "head-dim sweep, d=64"),
        Workload("b8h16n4k_d256", 8, 16, 4096, 256, "bf16", (False,), 5, "head-dim sweep, d=256"),
        Workload("fp8_b4h16n8k_d128", 4, 16, 8192, 128, "fp8", (False,), 6,
                 "e4m3 with outliers, random-Hadamard rotation, per-64-row scales"),
        Workload("b4h16n8k_d128", 4, 16, 8192, 128, "bf16", (False, True), 7,
                 "headline bf16 N=8k d=128 (same shape as the fp8 case)"),
    ]
    # short sequences: many heads, N/2 FLOPs per byte, below the MFMA/HBM ridge
    + [Workload(f"short_b64h16n{n}_d128", 64, 16, n, 128, "bf16", (False,), 8,
                f"short-sequence sweep, N={n} (bound by HBM)") for n in (128, 256, 512)]
}



@dataclass(frozen=True)
class DecodeWorkload:
    """A few query positions (Nq) against a key/value cache of Nk positions; Hkv key/value
    heads shared by groups of Hq / Hkv query heads."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    seed: int
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def kv_bytes(self) -> int:
        """Algorithmic HBM bytes: K and V read once, Q read, O and LSE written (bf16, fp32 LSE)."""
        return (2 * self.B * self.Hkv * self.Nk * self.d * 2 + 2 * self.B * self.Hq * self.Nq * self.d * 2
                + 4 * self.B * self.Hq * self.Nq)


DECODE_WORKLOADS = {
    w.name: w
    for w in [
        DecodeWorkload("decode_b16_hq32_hkv8_nk8k_d128", 16, 32, 8, 1, 8192, 128, False, 9,
                       "one new token per sequence, grouped heads (4 query heads per key/value head), 8K cache"),
        DecodeWorkload("decode_b2_h32_nk32k_d128", 2, 32, 32, 1, 32768, 128, False, 10,
                       "one new token per sequence, one key/value head per query head, 32K cache"),
        DecodeWorkload("decode_b16_hq32_hkv8_nq4_nk8k_d128", 16, 32, 8, 4, 8192, 128, True, 11,
                       "four new positions per sequence under the causal mask (parity case)"),
    ]
}


def make_decode_inputs(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int):
    """Q [B, Hq, Nq, d], K and V [B, Hkv, Nk, d], iid N(0, 1) drawn in that order, bfloat16."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, Hq, Nq, d, dtype=torch.float32, generator=g)
    k = torch.randn(B, Hkv, Nk, d, dtype=torch.float32, generator=g)
    v = torch.randn(B, Hkv, Nk, d, dtype=torch.float32, generator=g)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


@dataclass(frozen=True)
class ExtWorkload:
    """Forward with grouped key/value heads, an optional window (left, right) and optional packed
    sequences (lengths given, or nseq > 0 seeded cuts of N tokens; the batch is then 1)."""
    name: str
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    window: tuple
    seed: int
    lengths: tuple = ()
    nseq: int = 0
    note: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def packed(self) -> bool:
        return bool(self.lengths) or self.nseq > 0


EXT_WORKLOADS = {
    w.name: w
    for w in [
        ExtWorkload("gqa_b2_hq16_hkv4_n8k_d128_causal", 2, 16, 4, 8192, 128, True, (-1, -1), 12,
                    note="grouped heads (16 query heads share 4 key/value heads), causal: the pages' flash_attn example"),
        ExtWorkload("swa_b2_hq16_hkv4_n8k_d128_w4096", 2, 16, 4, 8192, 128, True, (4095, 0), 13,
                    note="the same with the sliding window (4095, 0): 4096 keys including the query"),
        ExtWorkload("varlen_3docs_hq16_hkv4_d128", 1, 16, 4, 2048, 128, True, (-1, -1), 14, lengths=(300, 1000, 748),
                    note="the pages' packed row: three documents of 300, 1000, 748 tokens, causal"),
        ExtWorkload("varlen_16docs_hq16_hkv4_n16k_d128", 1, 16, 4, 16384, 128, True, (-1, -1), 15, nseq=16,
                    note="16 packed documents of seeded lengths in 16384 tokens, causal"),
    ]
}


def make_ext_inputs(w: ExtWorkload):
    """(q, k, v, cu_seqlens or None) for an ExtWorkload; cu_seqlens is an int32 CPU tensor."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    q = torch.randn(w.B, w.Hq, w.N, w.d, dtype=torch.float32, generator=g).to(torch.bfloat16)
    k = torch.randn(w.B, w.Hkv, w.N, w.d, dtype=torch.float32, generator=g).to(torch.bfloat16)
    v = torch.randn(w.B, w.Hkv, w.N, w.d, dtype=torch.float32, generator=g).to(torch.bfloat16)
    cu = None
    if w.lengths:
        cu = torch.tensor([0] + list(torch.tensor(w.lengths).cumsum(0).tolist()), dtype=torch.int32)
    elif w.nseq > 0:
        cuts = torch.sort(torch.randperm(w.N - 1, generator=g)[: w.nseq - 1] + 1).values
        cu = torch.cat([torch.zeros(1, dtype=torch.int64), cuts, torch.tensor([w.N])]).to(torch.int32)
    return q, k, v, cu


OUTLIER_FRACTION = 0.001
OUTLIER_FACTOR = 20.0


def make_qkv(B: int, H: int, N: int, d: int, seed: int, dtype: str = "bf16"):
    """Draw Q, K, V iid N(0, 1) on the CPU; returns three contiguous tensors of ``dtype``."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, N, d, dtype=torch.float32, generator=g)
    k = torch.randn(B, H, N, d, dtype=torch.float32, generator=g)
    v = torch.randn(B, H, N, d, dtype=torch.float32, generator=g)
    if dtype == "bf16":
        q, k, v = q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)
    elif dtype not in ("f32", "fp8"):
        raise ValueError(f"unknown dtype {dtype}")
    return q, k, v


def make_dout(B: int, H: int, N: int, d: int, seed: int):
    """The output gradient dO of the backward workloads: iid N(0, 1), bfloat16, drawn after
    Q, K, V from the same seeded generator (so Q, K, V equal those of ``make_qkv``)."""
    g = torch.Generator("cpu").manual_seed(seed)
    for _ in range(3):
        torch.randn(B, H, N, d, dtype=torch.float32, generator=g)
    return torch.randn(B, H, N, d, dtype=torch.float32, generator=g).to(torch.bfloat16)


def make_fp8_inputs(B: int, H: int, N: int, d: int, seed: int):
    """FP8 workload inputs: float32 Q, K, V with outliers, and the +-1 rotation signs [d]."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, N, d, dtype=torch.float32, generator=g)
    k = torch.randn(B, H, N, d, dtype=torch.float32, generator=g)
    v = torch.randn(B, H, N, d, dtype=torch.float32, generator=g)
    n_out = int(math.floor(OUTLIER_FRACTION * q.numel()))
    for t in (q, k, v):
        idx = torch.randperm(t.numel(), generator=g)[:n_out]
        flat = t.view(-1)
        flat[idx] = flat[idx] * OUTLIER_FACTOR
    signs = torch.where(torch.rand(d, generator=g) > 0.5, 1.0, -1.0).to(torch.float32)
    return q, k, v, signs


def make_fp8_exact_inputs(B: int, H: int, N: int, d: int, seed: int):
    """Float32 x [B, H, N, d] whose Hadamard rotation is exact in float32 at d = 64 and 256, and
    the +-1 signs [d]: x is an integer in [-8, 8] times 2^-2 (uniform), and floor(0.001 numel)
    positions (randperm) are multiplied by 20 as in the FP8 workload. Every partial sum of the
    transform is then a multiple of 2^-2 below 2^24 (exact), and 1/sqrt(d) is a power of two."""
    g = torch.Generator("cpu").manual_seed(seed)
    x = (torch.randint(-8, 9, (B, H, N, d), generator=g).to(torch.float32) * 0.25).contiguous()
    n_out = int(math.floor(OUTLIER_FRACTION * x.numel()))
    idx = torch.randperm(x.numel(), generator=g)[:n_out]
    flat = x.view(-1)
    flat[idx] = flat[idx] * OUTLIER_FACTOR
    signs = torch.where(torch.rand(d, generator=g) > 0.5, 1.0, -1.0).to(torch.float32)
    return x, signs


def make_inputs(w: Workload):
    """Inputs for a named workload: (q, k, v) or, for fp8, (q32, k32, v32, signs)."""
    if w.dtype == "fp8":
        return make_fp8_inputs(w.B, w.H, w.N, w.d, w.seed)
    return make_qkv(w.B, w.H, w.N, w.d, w.seed, w.dtype)
