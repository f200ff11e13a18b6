"""Per-block FP8 quantisation and the FP8 attention references (test infrastructure only).

Sources:
- "FlashAttention-3: How Warp Specialization ..." page, section 4 "Technique
  3", item "Block-Wise Quantization and Two-Pass Rescaling", and the box
  "Block-Wise Dynamic Scaling & FP32 Accumulation": Q, K and V get one scale
  per block, the score tile is s_Q * s_K * (Q8 K8^T), accumulation stays in
  FP32.
- "FlashAttention 2 & 3" page, the fake quantiser in "Incoherent processing":
  the scale is amax / 448, replaced by 1 when amax is 0, and values are
  divided by it before rounding to FP8.
- same page, "Incoherent processing": Q and K are rotated by the same
  M = (1/sqrt(d)) H D before quantising; the scores, and so the exact result,
  do not change.

Readings where the pages leave a step open:
- a block is 64 consecutive rows (sequence positions) of one (batch, head)
  across all d columns; a last block shorter than 64 rows has its own scale;
- amax, s = amax / 448 and x / s are computed in float32, the precision in
  which the GPU quantiser works, then rounded to E4M3 (nearest, ties to even,
  saturating); the rotation itself is done in float64 and rounded once to
  float32 before quantising;
- V is quantised without rotation (only Q and K are rotated on the first page);
  the reference results do not depend on this choice.

Two references:
- ``O_true, LSE_true``: three-pass attention on the original float32 Q, K, V.
- ``O_deq, LSE_deq``: three-pass attention on the dequantised (rotated) Q, K
  and the dequantised V; this isolates the kernel's arithmetic from the input
  quantisation.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_fp64, attention_head_fp64
from .e4m3 import E4M3_MAX, e4m3_decode, e4m3_encode
from .hadamard import incoherent_rotate

BLOCK_ROWS = 64


def block_quantize(x, block: int = BLOCK_ROWS):
    """Quantise float32 x [..., N, d] to E4M3 codes with one fp32 scale per ``block`` rows.

    Returns (codes uint8 [..., N, d], scales float32 [..., ceil(N / block)]).
    """
    x = np.asarray(x, dtype=np.float32)
    *lead, n, d = x.shape
    nb = -(-n // block)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty((*lead, nb), dtype=np.float32)
    for bi in range(nb):
        r0, r1 = bi * block, min(n, (bi + 1) * block)
        blk = x[..., r0:r1, :]
        amax = np.abs(blk).max(axis=(-1, -2)).astype(np.float32)
        s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
        s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
        scaled = (blk / s[..., None, None]).astype(np.float32)   # float32 division
        codes[..., r0:r1, :] = e4m3_encode(scaled)
        scales[..., bi] = s
    return codes, scales


def block_dequantize(codes, scales, block: int = BLOCK_ROWS) -> np.ndarray:
    """Dequantise codes [..., N, d] with per-block scales back to float64 values."""
    vals = e4m3_decode(codes)
    n = vals.shape[-2]
    row_scale = np.repeat(np.asarray(scales, dtype=np.float64), block, axis=-1)[..., :n]
    return vals * row_scale[..., :, None]


def rotate_to_f32(x, signs) -> np.ndarray:
    """Incoherent rotation in float64, rounded once to float32 (the quantiser's input)."""
    return incoherent_rotate(x, signs).astype(np.float32)


def fp8_inputs(q32, k32, v32, signs):
    """Rotate Q and K (not V) and block-quantise all three; returns a dict of codes and scales."""
    qr = rotate_to_f32(q32, signs) if signs is not None else np.asarray(q32, np.float32)
    kr = rotate_to_f32(k32, signs) if signs is not None else np.asarray(k32, np.float32)
    q8, sq = block_quantize(qr)
    k8, sk = block_quantize(kr)
    v8, sv = block_quantize(np.asarray(v32, np.float32))
    return {"q8": q8, "k8": k8, "v8": v8, "sq": sq, "sk": sk, "sv": sv}


def fp8_reference(q32, k32, v32, signs, scale: float, causal: bool, with_true: bool = True):
    """FP8 references for [B, H, N, d] float32 inputs.

    Returns a dict with the quantised inputs (see ``fp8_inputs``), O_deq and
    LSE_deq, and (if ``with_true``) O_true and LSE_true.
    """
    res = fp8_inputs(q32, k32, v32, signs)
    qd = block_dequantize(res["q8"], res["sq"])
    kd = block_dequantize(res["k8"], res["sk"])
    vd = block_dequantize(res["v8"], res["sv"])
    res["O_deq"], res["LSE_deq"] = attention_fp64(qd, kd, vd, scale, causal)
    if with_true:
        res["O_true"], res["LSE_true"] = attention_fp64(q32, k32, v32, scale, causal)
    return res
