// FP8 (OCP e4m3) path: the incoherent-rotation + block-quantisation kernel and the fused
// attention forward on e4m3 inputs.
//
// Sources: "FlashAttention 2 & 3: Work Partitioning, Warp Specialization & FP8", sections
// "FP8 attention and incoherent processing" (rotate Q and K by M = (1/sqrt(d)) H D before
// quantising; scale = amax / 448) and "What stays in higher precision" (FP8 operands,
// FP32 accumulation, softmax statistics and output accumulator in high precision);
// "FlashAttention-3: How Warp Specialization ..." page, section 4 "Technique 3" (block-wise
// scales: the score tile is s_Q s_K (Q8 K8^T); P is converted to FP8 after the online
// rescale).
//
// prep_fp8_kernel: one workgroup per 64-row block of one (batch, head). Each thread holds a
// quarter of one row in registers; the fast Walsh-Hadamard transform runs its first
// log2(d/4) butterfly stages inside the thread and the last two across the 4 threads of the
// row (lane xor 1, 2). Then the signs and 1/sqrt(d) are applied, the block amax is reduced,
// s = amax / 448 and the codes are e4m3(clamp(x / s, +-448)) with the hardware RNE convert.
// Memory-bound: reads 4 bytes and writes 1 byte per element.
//
// The FP8 forward itself is the shared fused kernel (fa_fwd_kernel.h) instantiated for e4m3
// Q, K, V: e4m3 QK^T on the matrix cores with the block scales folded into the softmax FMA,
// V expanded exactly to bf16 in LDS with its block scale carried by P, bf16 P.
#include "fa_common.h"
#include "fa_fwd_kernel.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kPrepThreads = 256;
constexpr int kRowsPerScale = 64;
constexpr float kE4m3Max = 448.f;

// ------------------------------------------------------------------------------------------
// rotation + quantisation
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kPrepThreads) void prep_fp8_kernel(const float* __restrict__ X, uint8_t* __restrict__ X8,
                                                            float* __restrict__ S, const float* __restrict__ signs,
                                                            int N, int nsb, float inv_sqrt_d) {
    constexpr int NV = D / 4;   // values per thread
    __shared__ float wmax[kPrepThreads / kWave];
    const int tid = threadIdx.x;
    const int blk = blockIdx.x;            // (bh, sb) flattened
    const int bh = blk / nsb;
    const int sb = blk - bh * nsb;
    const int row = sb * kRowsPerScale + (tid >> 2);
    const int qd = tid & 3;
    const bool ok = row < N;
    const size_t base = ((size_t)bh * N + (ok ? row : 0)) * D + qd * NV;

    float x[NV];
#pragma unroll
    for (int i = 0; i < NV; i += 4) {
        f32x4 v = ok ? *(const f32x4*)(X + base + i) : f32x4{};
        x[i] = v[0]; x[i + 1] = v[1]; x[i + 2] = v[2]; x[i + 3] = v[3];
    }
    if (signs != nullptr) {
        // in-thread butterflies: strides 1 .. NV/2
#pragma unroll
        for (int st = 1; st < NV; st <<= 1)
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if ((i & st) == 0) {
                    const float a = x[i], b = x[i + st];
                    x[i] = a + b;
                    x[i + st] = a - b;
                }
        // cross-thread butterflies: strides NV and 2 NV (partner lane xor 1, xor 2)
#pragma unroll
        for (int m = 1; m <= 2; m <<= 1) {
            const bool upper = (qd & m) != 0;
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const float other = __shfl_xor(x[i], m);
                x[i] = upper ? (other - x[i]) : (x[i] + other);
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) x[i] = (x[i] * inv_sqrt_d) * signs[qd * NV + i];
    }
    // block amax
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) am = fmaxf(am, fabsf(x[i]));
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) am = fmaxf(am, __shfl_xor(am, m));
    if ((tid & 63) == 0) wmax[tid >> 6] = am;
    __syncthreads();
    am = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s = (am == 0.f) ? 1.f : __fdiv_rn(am, kE4m3Max);
    if (tid == 0) S[(size_t)bh * nsb + sb] = s;
    if (!ok) return;
    uint8_t* out = X8 + base;
#pragma unroll
    for (int i = 0; i < NV; i += 16) {
        i32x4 pk;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float y[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float t = __fdiv_rn(x[i + 4 * w + u], s);
                t = t > kE4m3Max ? kE4m3Max : (t < -kE4m3Max ? -kE4m3Max : t);   // saturate, keep NaN
                y[u] = t;
            }
            int word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
            pk[w] = word;
        }
        *(i32x4*)(out + i) = pk;
    }
}

template <int D>
hipError_t launch_prep(const float* x, void* x8, float* s, const float* signs, int BH, int N, hipStream_t stream) {
    const int nsb = (N + kRowsPerScale - 1) / kRowsPerScale;
    const long long total = (long long)BH * nsb;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prep_fp8_kernel<D>), dim3((unsigned)total), dim3(kPrepThreads), 0, stream, x, (uint8_t*)x8, s,
                       signs, N, nsb, 1.0f / sqrtf((float)D));
    return hipGetLastError();
}

#ifndef FA_F8_D128_NQ
#define FA_F8_D128_NQ 1
#endif
#ifndef FA_F8_D128_BC
#define FA_F8_D128_BC 32
#endif
#ifndef FA_F8_D128_MINB
#define FA_F8_D128_MINB (FA_F8_D128_NQ == 2 ? 1 : 2)
#endif

template <int D, int BC, int NQ, int MINB, bool PIPE>
hipError_t dispatch_fp8(const void* q8, const void* k8, const void* v8, const float* sq, const float* sk,
                        const float* sv, void* o, float* lse, int BH, int N, float scale, bool causal,
                        hipStream_t stream) {
    constexpr InKind K = InKind::FP8;
    return causal ? launch_fwd_kernel<K, D, BC, NQ, true, 8, MINB, PIPE>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale,
                                                                         stream)
                  : launch_fwd_kernel<K, D, BC, NQ, false, 8, MINB, PIPE>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale,
                                                                          stream);
}

}  // namespace

hipError_t launch_prep_fp8(const float* x, void* x8, float* s, const float* signs, int BH, int N, int d,
                           hipStream_t stream) {
    switch (d) {
        case 64: return launch_prep<64>(x, x8, s, signs, BH, N, stream);
        case 128: return launch_prep<128>(x, x8, s, signs, BH, N, stream);
        case 256: return launch_prep<256>(x, x8, s, signs, BH, N, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* sq, const float* sk,
                          const float* sv, void* o, float* lse, int BH, int N, int d, float scale, bool causal,
                          hipStream_t stream) {
    // key blocks of 64 keys (one scale block) or, for d = 128, 32 (half of one; fewer live
    // registers, as for bf16); conditional rescale threshold 2^8
    switch (d) {
        case 64: return dispatch_fp8<64, 64, 1, 2, true>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, causal, stream);
        case 128: return dispatch_fp8<128, FA_F8_D128_BC, FA_F8_D128_NQ, FA_F8_D128_MINB, true>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, causal, stream);
        case 256: return dispatch_fp8<256, 64, 1, 1, false>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, causal, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
