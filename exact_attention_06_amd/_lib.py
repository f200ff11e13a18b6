"""ctypes binding of ``libfa.so`` (the C ABI in include/fa.h).

Argument marshalling only: every step of the attention forward runs in the
HIP kernels behind the C entry points. PyTorch supplies device memory and the
stream; there is no CPU or PyTorch fallback, and a missing library or a
non-GPU tensor is an error.
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libfa.so")

FA_OK = 0
FA_F32 = 0
FA_BF16 = 1
STATUS_NAMES = {
    0: "FA_OK", -1: "FA_ERR_NULLPTR", -2: "FA_ERR_ALIGN", -3: "FA_ERR_SHAPE", -4: "FA_ERR_HEADDIM",
    -5: "FA_ERR_DTYPE", -6: "FA_ERR_SCALE", -7: "FA_ERR_LAUNCH", -8: "FA_ERR_ARG", -9: "FA_ERR_SCRATCH",
}
EXPORTED = ("fa_fwd", "fa_prep_fp8", "fa_fwd_fp8", "fa_bwd", "fa_fwd_ext", "fa_decode_workspace_size", "fa_decode",
            "fa_decode_noalloc", "fa_status_string", "fa_version")

_lib = None


class FAError(RuntimeError):
    """A non-zero status returned by the attention library."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libfa.so (once) and declare the C signatures. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_06_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    L.fa_fwd.restype = i
    L.fa_prep_fp8.argtypes = [vp, vp, vp, vp, i, i, i, i, vp]
    L.fa_prep_fp8.restype = i
    L.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
    L.fa_fwd_fp8.restype = i
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
    L.fa_bwd.restype = i
    L.fa_fwd_ext.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, i, i, vp]
    L.fa_fwd_ext.restype = i
    L.fa_decode_workspace_size.argtypes = [i, i, i, i, i, i]
    L.fa_decode_workspace_size.restype = ctypes.c_size_t
    L.fa_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp, ctypes.c_size_t, vp]
    L.fa_decode.restype = i
    L.fa_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, i, vp]
    L.fa_decode_noalloc.restype = i
    L.fa_status_string.argtypes = [i]
    L.fa_status_string.restype = ctypes.c_char_p
    L.fa_version.argtypes = []
    L.fa_version.restype = i
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().fa_status_string(status).decode()


def _check(status: int) -> None:
    if status != FA_OK:
        raise FAError(status, status_string(status))


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream, device) -> int | None:
    """The HIP stream to launch on: the given one, else the current stream of the tensors'
    device (not of whatever device happens to be current)."""
    if stream is None:
        return torch.cuda.current_stream(device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _require_gpu(*ts):
    """Every tensor given is a contiguous GPU tensor and all of them sit on one device."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("attention tensors must be contiguous GPU tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"attention tensors must share one device ({dev} and {t.device})")


def _expect(t, shape, dtype, name):
    """A caller-provided output or workspace tensor has the shape and dtype the kernels write."""
    if t is not None and (tuple(t.shape) != tuple(shape) or t.dtype != dtype):
        raise ValueError(f"{name} must be {dtype} of shape {list(shape)}, got {t.dtype} {list(t.shape)}")


def _bhnd(q):
    if q.dim() != 4:
        raise ValueError("expected [B, H, N, d] tensors")
    return tuple(int(x) for x in q.shape)


def fa_fwd(q, k, v, o=None, lse=None, *, scale=None, causal=False, want_lse=True, stream=None):
    """O = softmax(scale Q K^T [causal]) V and the row logsumexp, on the GPU.

    q, k, v: contiguous [B, H, N, d] torch tensors on the GPU, all float32 or all
    bfloat16. ``o`` / ``lse`` may be given (preallocated outputs) or are
    allocated here. Returns (o, lse); lse is None if ``want_lse`` is False and
    none was given.
    """
    B, H, N, d = _bhnd(q)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same [B, H, N, d] shape")
    if q.dtype == torch.bfloat16:
        dt = FA_BF16
    elif q.dtype == torch.float32:
        dt = FA_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    if o is None:
        o = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _expect(o, (B, H, N, d), q.dtype, "o")
    _expect(lse, (B, H, N), torch.float32, "lse")
    _require_gpu(q, k, v, o, lse)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    _check(lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, scale, int(bool(causal)), dt,
                        _stream(stream, q.device)))
    return o, lse


def fa_prep_fp8(x, signs=None, x8=None, s=None, *, stream=None):
    """Rotate (if ``signs`` is given) and block-quantise float32 x [B, H, N, d] to e4m3.

    Returns (x8 uint8 [B, H, N, d], s float32 [B, H, ceil(N/64)]).
    """
    B, H, N, d = _bhnd(x)
    if x.dtype != torch.float32:
        raise ValueError("fa_prep_fp8 takes float32 input")
    nsb = (N + 63) // 64
    if x8 is None:
        x8 = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((B, H, nsb), dtype=torch.float32, device=x.device)
    if signs is not None and (signs.dtype != torch.float32 or signs.numel() != d):
        raise ValueError("signs must be float32 with d entries")
    _expect(x8, (B, H, N, d), torch.uint8, "x8")
    _expect(s, (B, H, nsb), torch.float32, "s")
    _require_gpu(x, x8, s, signs)
    _check(lib().fa_prep_fp8(_ptr(x), _ptr(x8), _ptr(s), _ptr(signs), B, H, N, d, _stream(stream, x.device)))
    return x8, s


def fa_fwd_fp8(q8, k8, v8, sq, sk, sv, o=None, lse=None, *, scale=None, causal=False, want_lse=True, stream=None):
    """Attention forward on e4m3 codes with per-64-row scales; returns (o float32, lse)."""
    B, H, N, d = _bhnd(q8)
    for t in (q8, k8, v8):
        if t.dtype != torch.uint8 or t.shape != q8.shape:
            raise ValueError("q8, k8, v8 must be uint8 [B, H, N, d] code tensors")
    nsb = (N + 63) // 64
    for t in (sq, sk, sv):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H, nsb):
            raise ValueError("scales must be float32 [B, H, ceil(N/64)]")
    if o is None:
        o = torch.empty((B, H, N, d), dtype=torch.float32, device=q8.device)
    if lse is None and want_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    _expect(o, (B, H, N, d), torch.float32, "o")
    _expect(lse, (B, H, N), torch.float32, "lse")
    _require_gpu(q8, k8, v8, sq, sk, sv, o, lse)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    _check(lib().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(sq), _ptr(sk), _ptr(sv), _ptr(o), _ptr(lse),
                            B, H, N, d, scale, int(bool(causal)), _stream(stream, q8.device)))
    return o, lse


def fa_bwd(q, k, v, o, dout, lse, dq=None, dk=None, dv=None, delta=None, *, scale=None, causal=False, stream=None):
    """Gradients (dq, dk, dv) of attention from the forward's inputs, output o, logsumexp
    lse and the output gradient dout; bfloat16 [B, H, N, d] tensors, lse float32 [B, H, N].
    Outputs and the fp32 [2, B, H, N] workspace ``delta`` are allocated here unless given."""
    B, H, N, d = _bhnd(q)
    for t in (k, v, o, dout):
        if t.shape != q.shape or t.dtype != torch.bfloat16:
            raise ValueError("q, k, v, o, dout must be bfloat16 [B, H, N, d] tensors of one shape")
    if q.dtype != torch.bfloat16:
        raise ValueError("the backward takes bfloat16 tensors")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be float32 [B, H, N]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    delta = torch.empty((2, B, H, N), dtype=torch.float32, device=q.device) if delta is None else delta
    if delta.dtype != torch.float32 or delta.numel() < 2 * B * H * N:
        raise ValueError("delta must be a float32 workspace of 2*B*H*N elements")
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _expect(t, (B, H, N, d), torch.bfloat16, name)
    _require_gpu(q, k, v, o, dout, lse, dq, dk, dv, delta)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    _check(lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                        _ptr(delta), B, H, N, d, scale, int(bool(causal)), FA_BF16, _stream(stream, q.device)))
    return dq, dk, dv


def fa_decode_workspace_size(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int) -> int:
    """Bytes of fp32 workspace fa_decode needs for this shape (0: none)."""
    return int(lib().fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d))


def fa_decode(q, k, v, o=None, lse=None, workspace=None, *, scale=None, causal=False, want_lse=True, stream=None):
    """Decoding attention: q [B, Hq, Nq, d] against the key/value cache k, v [B, Hkv, Nk, d]
    (bfloat16; Hkv divides Hq), split over the keys. Returns (o, lse); o is bfloat16
    [B, Hq, Nq, d], lse float32 [B, Hq, Nq]. The workspace (uint8 or float32 GPU tensor of at
    least fa_decode_workspace_size(...) bytes) is allocated here unless given."""
    B, Hq, Nq, d = _bhnd(q)
    Bk, Hkv, Nk, dk = _bhnd(k)
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("k and v must be [B, Hkv, Nk, d] with the batch and head dim of q")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("fa_decode takes bfloat16 tensors")
    o = torch.empty_like(q) if o is None else o
    if lse is None and want_lse:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _expect(o, (B, Hq, Nq, d), torch.bfloat16, "o")
    _expect(lse, (B, Hq, Nq), torch.float32, "lse")
    need = fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _require_gpu(q, k, v, o, lse, workspace)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    _check(lib().fa_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, scale,
                           int(bool(causal)), FA_BF16, _ptr(workspace), nbytes, _stream(stream, q.device)))
    return o, lse


def fa_fwd_ext(q, k, v, o=None, lse=None, *, scale=None, causal=False, window=(-1, -1), cu_seqlens=None,
               max_seqlen=None, want_lse=True, stream=None):
    """Attention forward with grouped key/value heads, a sliding window (left, right) (a
    negative bound: no limit) and packed variable-length sequences.

    Without cu_seqlens: q [B, Hq, N, d], k, v [B, Hkv, N, d] (bfloat16, Hkv divides Hq). With
    cu_seqlens (int32 GPU tensor of B + 1 offsets from 0 to N): q [1, Hq, N, d], k, v
    [1, Hkv, N, d]; max_seqlen is the longest sequence (read back from cu_seqlens, which
    synchronises, when not given). Returns (o, lse) shaped like q and [batch, Hq, N]."""
    Bq, Hq, N, d = _bhnd(q)
    Bk, Hkv, Nk, dk = _bhnd(k)
    if tuple(v.shape) != tuple(k.shape) or Bk != Bq or Nk != N or dk != d:
        raise ValueError("k and v must be [B, Hkv, N, d] with the batch, length and head dim of q")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("fa_fwd_ext takes bfloat16 tensors")
    if cu_seqlens is not None:
        if Bq != 1:
            raise ValueError("packed sequences: the batch dimension must be 1")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor of B + 1 offsets")
        B = cu_seqlens.numel() - 1
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if B > 0 else 0
    else:
        B, max_seqlen = Bq, 0
    o = torch.empty_like(q) if o is None else o
    if lse is None and want_lse:
        lse = torch.empty((Bq, Hq, N), dtype=torch.float32, device=q.device)
    _expect(o, (Bq, Hq, N, d), torch.bfloat16, "o")
    _expect(lse, (Bq, Hq, N), torch.float32, "lse")
    _require_gpu(q, k, v, o, lse, cu_seqlens)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    _check(lib().fa_fwd_ext(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, d, scale,
                            int(bool(causal)), int(window[0]), int(window[1]), _ptr(cu_seqlens), int(max_seqlen),
                            FA_BF16, _stream(stream, q.device)))
    return o, lse


def fa_decode_noalloc(q, k, v, o, lse=None, *, scale=None, causal=False, stream=None):
    """fa_decode with the library's static scratch instead of a workspace: the C entry point
    allocates nothing. o (bfloat16 [B, Hq, Nq, d]) must be given; lse (float32 [B, Hq, Nq]) is
    optional. Calls that overlap in time on one GPU share the scratch and race."""
    B, Hq, Nq, d = _bhnd(q)
    Bk, Hkv, Nk, dk = _bhnd(k)
    if tuple(v.shape) != tuple(k.shape) or Bk != B or dk != d:
        raise ValueError("k and v must be [B, Hkv, Nk, d] with the batch and head dim of q")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise ValueError("fa_decode_noalloc takes bfloat16 tensors")
    if o is None:
        raise ValueError("fa_decode_noalloc writes into a given output tensor")
    _expect(o, (B, Hq, Nq, d), torch.bfloat16, "o")
    _expect(lse, (B, Hq, Nq), torch.float32, "lse")
    _require_gpu(q, k, v, o, lse)
    scale = (1.0 / d ** 0.5) if scale is None else float(scale)
    _check(lib().fa_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, scale,
                                   int(bool(causal)), FA_BF16, _stream(stream, q.device)))
    return o, lse
