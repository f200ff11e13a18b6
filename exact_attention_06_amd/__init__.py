"""Exact (Flash) attention, forward and backward, for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
``libfa.so`` (include/fa.h); this package is its Python binding:

- ``fa_fwd(q, k, v, causal=..., scale=...)``: fused attention forward for
  float32 or bfloat16 [B, H, N, d] tensors, returning O and the row logsumexp;
- ``fa_prep_fp8(x, signs)``: random-Hadamard rotation and per-64-row E4M3
  block quantisation of a float32 tensor;
- ``fa_fwd_fp8(q8, k8, v8, sq, sk, sv, ...)``: attention forward on E4M3 codes (fp32 O);
- ``fa_bwd(q, k, v, o, dout, lse, ...)``: the gradients dq, dk, dv (bfloat16);
- ``fa_fwd_ext(q, k, v, window=..., cu_seqlens=...)``: the forward with grouped
  key/value heads, a sliding window and packed variable-length sequences;
- ``fa_decode(q, k, v, ...)``: a few query positions against a long key/value
  cache (grouped heads allowed), split over the keys and merged;
  ``fa_decode_noalloc`` does the same with the library's static scratch.

``workloads`` draws the seeded synthetic inputs; ``build`` compiles the library.
"""

from ._lib import (FAError, fa_bwd, fa_decode, fa_decode_noalloc, fa_decode_workspace_size, fa_fwd,  # noqa: F401
                   fa_fwd_ext, fa_fwd_fp8, fa_prep_fp8, lib, status_string)

__all__ = ["FAError", "fa_bwd", "fa_decode", "fa_decode_noalloc", "fa_decode_workspace_size", "fa_fwd", "fa_fwd_ext",
           "fa_fwd_fp8", "fa_prep_fp8", "lib", "status_string"]
