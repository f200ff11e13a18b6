// C ABI of the attention library (declared in include/fa.h): argument checks on the host,
// then dispatch to the gfx950 kernels. No allocation, no synchronisation, no fallback: an
// unsupported argument is an error code, never a silent slower path.
#include <cmath>
#include <cstdint>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

constexpr int kVersion = 500;   // 0.5.0: fa_decode_noalloc

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool headdim_ok(int d) { return d == 64 || d == 128 || d == 256; }

// common shape/scale checks; returns FA_OK or the first error
int check_common(int B, int H, int N, int d, float scale, int causal) {
    if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
    if (!headdim_ok(d)) return FA_ERR_HEADDIM;
    if (!(std::isfinite(scale) && scale > 0.f)) return FA_ERR_SCALE;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    // element offsets are computed in 64-bit; the grid and per-head row counts must fit int32,
    // and the bytes of one head of fp32 data (buffer ranges and offsets inside a head) too
    const long long rows = (long long)B * H * (long long)N;
    if (rows > 0x7fffffffLL) return FA_ERR_SHAPE;
    if ((long long)N * d * 4 > 0x7fffffffLL) return FA_ERR_SHAPE;
    return FA_OK;
}

// decode shapes: returns FA_OK or the first error
int check_decode(int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal) {
    if (B < 0 || Hq < 0 || Hkv < 1 || Nq < 0 || Nk < 0 || Hq % Hkv != 0 || Nq > Nk) return FA_ERR_SHAPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (!(std::isfinite(scale) && scale > 0.f)) return FA_ERR_SCALE;
    if (causal != 0 && causal != 1) return FA_ERR_ARG;
    // rows of q / o and of the key/value cache fit int32, one head of K or V fits a buffer range
    if ((long long)B * Hq * (long long)Nq > 0x7fffffffLL) return FA_ERR_SHAPE;
    if ((long long)B * Hkv * (long long)Nk > 0x7fffffffLL) return FA_ERR_SHAPE;
    if ((long long)Nk * d * 2 > 0x7fffffffLL) return FA_ERR_SHAPE;
    return FA_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d, float scale,
           int causal, int dtype, void* stream) {
    int st = check_common(B, H, N, d, scale, causal);
    if (st != FA_OK) return st;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
    if ((long long)B * H * N == 0) return FA_OK;
    if (!q || !k || !v || !o) return FA_ERR_NULLPTR;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
        return FA_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == FA_BF16) return from_hip(fa::launch_fwd_bf16(q, k, v, o, lse, B * H, N, d, scale, causal != 0, s));
    return from_hip(fa::launch_fwd_f32(q, k, v, o, lse, B * H, N, d, scale, causal != 0, s));
}

int fa_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int N,
               int d, float scale, int causal, int window_left, int window_right, const int* cu_seqlens,
               int max_seqlen, int dtype, void* stream) {
    if (B < 0 || Hkv < 1 || Hq < 0 || Hq % Hkv != 0) return FA_ERR_SHAPE;
    const int nb = cu_seqlens != nullptr ? 1 : B;   // batch dimension of the tensors
    int st = check_common(nb, Hq, N, d, scale, causal);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16) return FA_ERR_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if (cu_seqlens != nullptr && (max_seqlen < 0 || max_seqlen > N)) return FA_ERR_SHAPE;
    const int rows_n = cu_seqlens != nullptr ? max_seqlen : N;
    // workgroups: B Hq rows of ceil(rows_n / 128) query blocks
    if ((long long)B * Hq * ((rows_n + 127) / 128) > 0x7fffffffLL) return FA_ERR_SHAPE;
    if ((long long)B * Hq * rows_n == 0) return FA_OK;
    if (!q || !k || !v || !o) return FA_ERR_NULLPTR;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)) ||
        (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
        return FA_ERR_ALIGN;
    return from_hip(fa::launch_fwd_ext_bf16(q, k, v, o, lse, B, Hq, Hkv, N, max_seqlen, d, scale, causal != 0,
                                            window_left, window_right, cu_seqlens, static_cast<hipStream_t>(stream)));
}

int fa_prep_fp8(const float* x, void* x8, float* sc, const float* signs, int B, int H, int N, int d, void* stream) {
    int st = check_common(B, H, N, d, 1.f, 0);
    if (st != FA_OK) return st;
    if ((long long)B * H * N == 0) return FA_OK;
    if (!x || !x8 || !sc) return FA_ERR_NULLPTR;
    if (!aligned16(x) || !aligned16(x8) || !aligned16(sc) || (signs && !aligned16(signs))) return FA_ERR_ALIGN;
    return from_hip(fa::launch_prep_fp8(x, x8, sc, signs, B * H, N, d, static_cast<hipStream_t>(stream)));
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* sq, const float* sk, const float* sv,
               void* o, float* lse, int B, int H, int N, int d, float scale, int causal, void* stream) {
    int st = check_common(B, H, N, d, scale, causal);
    if (st != FA_OK) return st;
    if ((long long)B * H * N == 0) return FA_OK;
    if (!q8 || !k8 || !v8 || !sq || !sk || !sv || !o) return FA_ERR_NULLPTR;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o) || (lse && !aligned16(lse)))
        return FA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(sq) | reinterpret_cast<uintptr_t>(sk) | reinterpret_cast<uintptr_t>(sv)) & 3u)
        return FA_ERR_ALIGN;
    return from_hip(fa::launch_fwd_fp8(q8, k8, v8, sq, sk, sv, o, lse, B * H, N, d, scale, causal != 0,
                                       static_cast<hipStream_t>(stream)));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse, void* dq,
           void* dk, void* dv, float* delta, int B, int H, int N, int d, float scale, int causal, int dtype,
           void* stream) {
    int st = check_common(B, H, N, d, scale, causal);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16) return FA_ERR_DTYPE;
    if (d != 64 && d != 128) return FA_ERR_HEADDIM;
    if ((long long)B * H * N == 0) return FA_OK;
    if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta) return FA_ERR_NULLPTR;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(lse) ||
        !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(delta))
        return FA_ERR_ALIGN;
    return from_hip(fa::launch_bwd_bf16(q, k, v, o, dout, lse, dq, dk, dv, delta, B * H, N, d, scale, causal != 0,
                                        static_cast<hipStream_t>(stream)));
}

size_t fa_decode_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    if (check_decode(B, Hq, Hkv, Nq, Nk, d, 1.f, 0) != FA_OK) return 0;
    if ((long long)B * Hq * Nq == 0) return 0;
    return fa::decode_plan(B, Hq, Hkv, Nq, Nk, d).ws_bytes;
}

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Nq,
              int Nk, int d, float scale, int causal, int dtype, void* workspace, size_t workspace_bytes,
              void* stream) {
    int st = check_decode(B, Hq, Hkv, Nq, Nk, d, scale, causal);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16) return FA_ERR_DTYPE;
    if ((long long)B * Hq * Nq == 0) return FA_OK;
    if (!q || !k || !v || !o) return FA_ERR_NULLPTR;
    const size_t need = fa::decode_plan(B, Hq, Hkv, Nq, Nk, d).ws_bytes;
    if (need > 0 && !workspace) return FA_ERR_NULLPTR;
    if (workspace_bytes < need) return FA_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)) ||
        (workspace && !aligned16(workspace)))
        return FA_ERR_ALIGN;
    return from_hip(fa::launch_decode_bf16(q, k, v, o, lse, workspace, B, Hq, Hkv, Nq, Nk, d, scale, causal != 0,
                                           static_cast<hipStream_t>(stream)));
}

int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                      int Nq, int Nk, int d, float scale, int causal, int dtype, void* stream) {
    int st = check_decode(B, Hq, Hkv, Nq, Nk, d, scale, causal);
    if (st != FA_OK) return st;
    if (dtype != FA_BF16) return FA_ERR_DTYPE;
    if ((long long)B * Hq * Nq == 0) return FA_OK;
    if (!q || !k || !v || !o) return FA_ERR_NULLPTR;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
        return FA_ERR_ALIGN;
    if (fa::decode_plan(B, Hq, Hkv, Nq, Nk, d).ws_bytes > fa::kDecodeScratchBytes) return FA_ERR_SCRATCH;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if (fa::decode_scratch(s, &ws) != hipSuccess) return FA_ERR_LAUNCH;
    return from_hip(fa::launch_decode_bf16(q, k, v, o, lse, ws, B, Hq, Hkv, Nq, Nk, d, scale, causal != 0, s));
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_NULLPTR: return "a required pointer is NULL";
        case FA_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case FA_ERR_SHAPE: return "invalid shape (negative size, too many rows, or N*d*4 >= 2^31)";
        case FA_ERR_HEADDIM: return "unsupported head dimension (64, 128 or 256; the backward and decoding: 64 or 128)";
        case FA_ERR_DTYPE: return "unsupported dtype";
        case FA_ERR_SCALE: return "scale must be finite and > 0";
        case FA_ERR_LAUNCH: return "kernel launch failed";
        case FA_ERR_ARG: return "invalid argument (causal not 0/1, or a workspace smaller than required)";
        case FA_ERR_SCRATCH: return "the problem needs more scratch than the library's static buffer holds";
        default: return "unknown status";
    }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
