// Host-side declarations shared by the launchers and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace fa {

// bf16 Q, K, V, O [BH, N, d]; lse [BH, N] or null. d in {64, 128, 256}.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                           float scale, bool causal, hipStream_t stream);

// Short sequences (bf16, 1 <= N <= 128, d in {64, 128}): the whole key/value range of a head in
// one workgroup's LDS; same arguments as launch_fwd_bf16. short_fwd_applies: whether it takes
// the problem.
bool short_fwd_applies(int N, int d);
hipError_t launch_fwd_short_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                                 float scale, bool causal, hipStream_t stream);

// Grouped heads, sliding window, packed sequences (bf16, d in {64, 128}). Without cu_seqlens:
// q, o [B, Hq, N, d], k, v [B, Hkv, N, d], lse [B, Hq, N]. With cu_seqlens (device int32, B + 1
// offsets into N tokens): q, o [Hq, N, d], k, v [Hkv, N, d], lse [Hq, N], every sequence at most
// max_seqlen long. left / right < 0: no limit on that side.
hipError_t launch_fwd_ext_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                               int Hkv, int N, int max_seqlen, int d, float scale, bool causal, int left, int right,
                               const int* cu_seqlens, hipStream_t stream);

// fp32 Q, K, V, O [BH, N, d]; lse [BH, N] or null. d in {64, 128, 256}.
hipError_t launch_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                          float scale, bool causal, hipStream_t stream);

// fp32 x [BH, N, d] -> e4m3 codes x8 [BH, N, d], scales s [BH, ceil(N/64)]; signs [d] or null.
hipError_t launch_prep_fp8(const float* x, void* x8, float* s, const float* signs, int BH, int N, int d,
                           hipStream_t stream);

// e4m3 q8, k8, v8 [BH, N, d] with scales [BH, ceil(N/64)] -> fp32 O [BH, N, d], lse [BH, N] or null.
hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* sq, const float* sk,
                          const float* sv, void* o, float* lse, int BH, int N, int d, float scale, bool causal,
                          hipStream_t stream);

// bf16 backward: q, k, v, o, dout [BH, N, d], lse [BH, N] from the forward -> dq, dk, dv
// [BH, N, d] bf16; delta [2, BH, N] fp32 workspace (-D = -rowsum(dO o O), then -LSE log2 e).
// d in {64, 128}.
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, float* delta, int BH, int N, int d,
                           float scale, bool causal, hipStream_t stream);

// Split-key decoding: how the keys are cut (the same for a given shape, so that the caller's
// workspace size can be asked for first). ncg column groups of 32 query rows, ntiles 32-key
// tiles, tps tiles per split, nsplit splits; ws_bytes of fp32 workspace (0 with one split).
struct DecodePlan {
    int ncg, ntiles, tps, nsplit;
    size_t ws_bytes;
};
DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d);

// The largest decode_plan(...).ws_bytes of any shape: a plan splits only when its B Hkv ncg
// groups are fewer than the 256 workgroups it aims for, into at most ceil(256 / groups) splits,
// so groups x splits <= 510; each holds at most 32 ncg rows of d + 2 fp32 values (d <= 128).
constexpr size_t kDecodeScratchBytes = (size_t)510 * 32 * (128 + 2) * 4;   // 8,486,400 bytes

// Address of this GPU's copy of the static decode scratch (kDecodeScratchBytes, for
// fa_decode_noalloc): the GPU of `stream` (the current one for the null stream); looked up
// once per GPU with that GPU current, then cached.
hipError_t decode_scratch(hipStream_t stream, void** ptr);

// bf16 q [B, Hq, Nq, d], k, v [B, Hkv, Nk, d] -> o [B, Hq, Nq, d] bf16, lse [B, Hq, Nq] or null;
// ws: decode_plan(...).ws_bytes of workspace. d in {64, 128}.
hipError_t launch_decode_bf16(const void* q, const void* k, const void* v, void* o, float* lse, void* ws, int B,
                              int Hq, int Hkv, int Nq, int Nk, int d, float scale, bool causal, hipStream_t stream);

}  // namespace fa
