"""The C ABI without a GPU: the library loads, exports what include/fa.h declares, and
rejects bad arguments on the host before anything is launched (no compute call here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def L():
    from exact_attention_06_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from exact_attention_06_amd.build import build

        build()
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(["fa_fwd", "fa_prep_fp8", "fa_fwd_fp8", "fa_bwd", "fa_fwd_ext",
                                           "fa_decode_workspace_size", "fa_decode", "fa_decode_noalloc",
                                           "fa_status_string", "fa_version"])


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_version_and_status_strings(L):
    from exact_attention_06_amd import _lib

    assert L.fa_version() == 500
    for code, name in _lib.STATUS_NAMES.items():
        s = _lib.status_string(code)
        assert s and s != "unknown status", name
    assert _lib.status_string(12345) == "unknown status"


P = 0x10000   # a 16-byte aligned fake device address: never dereferenced, validation fails first


def fwd(L, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=128, scale=0.088, causal=0, dtype=1):
    return L.fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, None)


def test_fwd_argument_errors(L):
    assert fwd(L, d=96) == -4
    assert fwd(L, d=32) == -4
    assert fwd(L, scale=0.0) == -6
    assert fwd(L, scale=-1.0) == -6
    assert fwd(L, scale=float("inf")) == -6
    assert fwd(L, scale=float("nan")) == -6
    assert fwd(L, causal=2) == -8
    assert fwd(L, dtype=2) == -5
    assert fwd(L, B=-1) == -3
    assert fwd(L, N=-5) == -3
    assert fwd(L, B=1 << 16, H=1 << 16, N=1) == -3     # B*H*N beyond the int32 row range
    assert fwd(L, N=1 << 21, d=256) == -3               # one head's fp32 bytes reach 2^31
    assert L.fa_prep_fp8(P, P, P, None, 1, 1, 1 << 21, 256, None) == -3
    assert fwd(L, q=None) == -1
    assert fwd(L, o=None) == -1
    assert fwd(L, k=P + 8) == -2
    assert fwd(L, lse=P + 4) == -2


def test_empty_problem_is_ok_without_launch(L):
    # nothing to do: no pointer is touched and no kernel is launched
    assert fwd(L, q=None, k=None, v=None, o=None, lse=None, N=0) == 0
    assert fwd(L, q=None, k=None, v=None, o=None, lse=None, B=0) == 0
    assert L.fa_prep_fp8(None, None, None, None, 0, 4, 64, 128, None) == 0
    assert L.fa_fwd_fp8(None, None, None, None, None, None, None, None, 2, 0, 64, 128, 0.1, 0, None) == 0


def test_fp8_argument_errors(L):
    assert L.fa_prep_fp8(P, P, P, None, 1, 1, 64, 100, None) == -4
    assert L.fa_prep_fp8(None, P, P, None, 1, 1, 64, 128, None) == -1
    assert L.fa_prep_fp8(P + 4, P, P, None, 1, 1, 64, 128, None) == -2
    assert L.fa_fwd_fp8(P, P, P, P, P, P, P, P, 1, 1, 64, 128, 0.0, 0, None) == -6
    assert L.fa_fwd_fp8(P, P, P, None, P, P, P, P, 1, 1, 64, 128, 0.1, 0, None) == -1
    assert L.fa_fwd_fp8(P, P, P, P + 2, P, P, P, P, 1, 1, 64, 128, 0.1, 0, None) == -2
    assert L.fa_fwd_fp8(P, P, P, P, P, P, P, P, 1, 1, 64, 128, 0.1, 3, None) == -8


def test_python_binding_rejects_cpu_tensors(L):
    import torch

    from exact_attention_06_amd import fa_fwd

    q = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa_fwd(q, q, q, o=torch.empty_like(q), lse=torch.empty(1, 1, 64))


def test_python_binding_checks_given_outputs(L):
    """Outputs the caller passes in are checked for shape and dtype before anything is
    launched (an undersized one would be written past its end)."""
    import torch

    from exact_attention_06_amd import fa_bwd, fa_decode, fa_fwd, fa_fwd_ext, fa_fwd_fp8, fa_prep_fp8

    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16)
    lse = torch.empty(1, 2, 64)
    with pytest.raises(ValueError, match="o must be"):
        fa_fwd(q, q, q, o=torch.empty(1, 2, 32, 64, dtype=torch.bfloat16), lse=lse)
    with pytest.raises(ValueError, match="o must be"):
        fa_fwd(q, q, q, o=torch.empty(1, 2, 64, 64), lse=lse)            # float32 for bf16 inputs
    with pytest.raises(ValueError, match="lse must be"):
        fa_fwd(q, q, q, o=torch.empty_like(q), lse=torch.empty(2, 64))
    with pytest.raises(ValueError, match="dk must be"):
        fa_bwd(q, q, q, q, q, lse, dq=torch.empty_like(q), dk=torch.empty(1, 2, 64, 32, dtype=torch.bfloat16),
               dv=torch.empty_like(q), delta=torch.empty(2, 1, 2, 64))
    with pytest.raises(ValueError, match="lse must be"):
        fa_decode(q[:, :, :4], q, q, o=torch.empty_like(q[:, :, :4]), lse=torch.empty(1, 2, 64))
    with pytest.raises(ValueError, match="o must be"):
        fa_fwd_ext(q, q[:, :1], q[:, :1], o=torch.empty(1, 1, 64, 64, dtype=torch.bfloat16))
    x = torch.zeros(1, 2, 64, 64)
    with pytest.raises(ValueError, match="s must be"):
        fa_prep_fp8(x, x8=torch.empty(1, 2, 64, 64, dtype=torch.uint8), s=torch.empty(1, 2, 2))
    c8 = torch.zeros(1, 2, 64, 64, dtype=torch.uint8)
    sc = torch.ones(1, 2, 1)
    with pytest.raises(ValueError, match="o must be"):
        fa_fwd_fp8(c8, c8, c8, sc, sc, sc, o=torch.empty(1, 2, 64, 64, dtype=torch.bfloat16))   # it writes float32


def test_python_binding_rejects_mixed_devices():
    from types import SimpleNamespace

    from exact_attention_06_amd._lib import _require_gpu

    def fake(dev):
        return SimpleNamespace(is_cuda=True, is_contiguous=lambda: True, device=dev)

    _require_gpu(fake("cuda:0"), None, fake("cuda:0"))
    with pytest.raises(ValueError, match="one device"):
        _require_gpu(fake("cuda:0"), fake("cuda:1"))


def bwd(L, ptrs=None, B=1, H=1, N=128, d=128, scale=0.088, causal=0, dtype=1):
    p = [P] * 10 if ptrs is None else ptrs
    return L.fa_bwd(*p, B, H, N, d, scale, causal, dtype, None)


def test_bwd_argument_errors(L):
    assert bwd(L, d=256) == -4          # the backward supports d = 64 and 128
    assert bwd(L, d=96) == -4
    assert bwd(L, dtype=0) == -5        # bfloat16 only
    assert bwd(L, scale=0.0) == -6
    assert bwd(L, causal=3) == -8
    assert bwd(L, N=-1) == -3
    for i in range(10):                 # q k v o dout lse dq dk dv delta
        p = [P] * 10
        p[i] = None
        assert bwd(L, p) == -1, i
        p[i] = P + 4
        assert bwd(L, p) == -2, i
    assert bwd(L, [None] * 10, N=0) == 0   # empty: nothing touched, nothing launched


def dec(L, ptrs=None, B=2, Hq=8, Hkv=2, Nq=1, Nk=4096, d=128, scale=0.088, causal=0, dtype=1, ws_bytes=None):
    p = [P] * 5 if ptrs is None else ptrs[:5]
    ws = P if ptrs is None else ptrs[5]
    if ws_bytes is None:
        ws_bytes = L.fa_decode_workspace_size(B, Hq, Hkv, Nq, Nk, d)
    return L.fa_decode(*p, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, ws, ws_bytes, None)


def test_decode_workspace_size(L):
    # split over the keys: one fp32 state (d values, max, sum) per split and query row
    n = L.fa_decode_workspace_size(2, 8, 2, 1, 4096, 128)
    assert n > 0 and n % (4 * (128 + 2)) == 0
    rows = 2 * 8 * 1
    assert (n // (4 * (128 + 2))) % rows == 0          # whole splits of every row
    assert L.fa_decode_workspace_size(2, 8, 2, 1, 64, 128) == 0      # two tiles: one split, no workspace
    assert L.fa_decode_workspace_size(2, 8, 3, 1, 4096, 128) == 0    # invalid shape
    assert L.fa_decode_workspace_size(0, 8, 2, 1, 4096, 128) == 0    # empty


def test_decode_argument_errors(L):
    assert dec(L, d=256) == -4
    assert dec(L, dtype=0) == -5
    assert dec(L, scale=float("nan")) == -6
    assert dec(L, causal=2) == -8
    assert dec(L, Hkv=3) == -3            # Hkv must divide Hq
    assert dec(L, Hkv=0) == -3
    assert dec(L, Nq=5, Nk=4) == -3       # more queries than keys
    need = L.fa_decode_workspace_size(2, 8, 2, 1, 4096, 128)
    assert dec(L, ws_bytes=need - 1) == -8
    for i in range(4):                    # q k v o
        p = [P] * 6
        p[i] = None
        assert dec(L, p) == -1, i
        p[i] = P + 4
        assert dec(L, p) == -2, i
    p = [P] * 6
    p[4] = None                           # lse is optional: only the other checks apply
    p[5] = P + 8
    assert dec(L, p) == -2                # misaligned workspace
    p[5] = None
    assert dec(L, p) == -1                # the workspace is required when its size is > 0
    assert dec(L, [None] * 6, Nq=0) == 0  # empty: nothing touched, nothing launched


def ext(L, ptrs=None, B=2, Hq=8, Hkv=2, N=256, d=128, scale=0.088, causal=1, left=-1, right=-1, cu=None,
        max_seqlen=0, dtype=1):
    p = [P] * 5 if ptrs is None else ptrs
    return L.fa_fwd_ext(*p, B, Hq, Hkv, N, d, scale, causal, left, right, cu, max_seqlen, dtype, None)


def test_fwd_ext_argument_errors(L):
    assert ext(L, d=256) == -4            # 64 and 128
    assert ext(L, dtype=0) == -5          # bfloat16 only
    assert ext(L, scale=-1.0) == -6
    assert ext(L, causal=7) == -8
    assert ext(L, Hkv=3) == -3            # Hkv must divide Hq
    assert ext(L, Hkv=0) == -3
    assert ext(L, N=-5) == -3
    assert ext(L, cu=P, max_seqlen=257) == -3    # longer than N
    assert ext(L, cu=P, max_seqlen=-1) == -3
    assert ext(L, cu=P + 2, max_seqlen=100) == -2  # int32 offsets: 4-byte aligned
    for i in range(4):                    # q k v o
        p = [P] * 5
        p[i] = None
        assert ext(L, p) == -1, i
        p[i] = P + 8
        assert ext(L, p) == -2, i
    assert ext(L, [None] * 5, N=0) == 0                      # empty: nothing launched
    assert ext(L, [None] * 5, cu=P, max_seqlen=0) == 0       # packed, every sequence empty


def test_decode_noalloc_argument_errors(L):
    """The allocation-free decoding entry point checks its arguments like fa_decode, before it
    looks up its scratch or launches anything (nothing here reaches the GPU)."""
    def dn(ptrs=None, B=2, Hq=8, Hkv=2, Nq=1, Nk=4096, d=128, scale=0.088, causal=0, dtype=1):
        p = [P] * 5 if ptrs is None else ptrs
        return L.fa_decode_noalloc(*p, B, Hq, Hkv, Nq, Nk, d, scale, causal, dtype, None)

    assert dn(d=256) == -4
    assert dn(dtype=0) == -5
    assert dn(scale=0.0) == -6
    assert dn(causal=3) == -8
    assert dn(Hkv=3) == -3
    assert dn(Nq=9, Nk=8) == -3
    for i in range(4):                    # q k v o
        p = [P] * 5
        p[i] = None
        assert dn(p) == -1, i
        p[i] = P + 4
        assert dn(p) == -2, i
    assert dn([None] * 5, Nq=0) == 0      # empty: nothing touched, nothing launched
    # every shape's workspace fits the static scratch (8,486,400 bytes, the largest any shape needs)
    assert L.fa_decode_workspace_size(255, 1, 1, 32, 512, 128) == 8486400
