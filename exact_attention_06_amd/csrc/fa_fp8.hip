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
// prep_fp8_kernel: one workgroup per 64-row block of one (batch, head). The 4 threads of a
// lane quad share one row: thread q holds the elements 16 k + 4 q + j (j < 4), so each load
// instruction of a quad reads 64 contiguous bytes. The fast Walsh-Hadamard transform pairs
// elements along one index bit per butterfly stage, in any order: the bits of j and k are
// stages inside the thread, the two bits of q are stages across the quad (DPP quad
// permutations, no LDS), all in fp64; then one multiply by +-1/sqrt(d) applies the signs and
// the normalisation and the result is rounded once to fp32 (the definition's x M to within
// ~1e-16 relative; an fp32 transform rounds at every stage and moves a few values per
// million to the neighbouring E4M3 code). The block amax is reduced, s = amax / 448, and
// the codes are e4m3(x / s) with the hardware RNE convert. x / s is the correctly rounded
// fp32 quotient, computed from r = RN(1/s) as q0 = x r, q = q0 + (x - q0 s) r (two FMAs;
// Markstein's correction gives RN(x / s) for normal operands; the sign is copied from x so that
// -0 stays -0) instead of a full division.
// No clamp is needed for a normal s: |x| <= amax gives |x / s| <= 448 (1 + 2^-23), which the
// convert rounds to 448; only a subnormal s (amax below ~5e-36) can exceed that, and such
// blocks take a clamping branch. NaN inputs stay NaN.
// Memory-bound: reads 4 bytes and writes 1 byte per element.
//
// The FP8 forward itself is the shared fused kernel (fa_fwd_kernel.h) instantiated for e4m3
// Q, K, V: e4m3 QK^T on the matrix cores with the block scales folded into the softmax FMA,
// V expanded exactly to fp16 in LDS with its block scale carried by P, fp16 P and an fp32 O.
#include <cmath>

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
// value of lane l ^ 1 / l ^ 2 within each quad of lanes (DPP quad permutations; every lane
// has a source, so the move can be folded into the instruction that uses it)
__device__ __forceinline__ float quad_xor1(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}
// the same for an fp64 value (its two 32-bit halves)
template <int CTRL>
__device__ __forceinline__ double quad_xor_d(double x) {
    const int lo = __builtin_amdgcn_mov_dpp(__double2loint(x), CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_mov_dpp(__double2hiint(x), CTRL, 0xF, 0xF, true);
    return __hiloint2double(hi, lo);
}

// workgroups per CU the register budget is held to: the kernel streams memory, and the loads
// of more resident workgroups hide more latency (d = 128: 5, where the compiler would otherwise
// take 108 registers and leave room for 4)
template <int D>
constexpr int kPrepMinBlocks = D <= 64 ? 8 : D <= 128 ? 5 : 2;

template <int D>
__global__ __launch_bounds__(kPrepThreads, kPrepMinBlocks<D>) void prep_fp8_kernel(const float* __restrict__ X, uint8_t* __restrict__ X8,
                                                            float* __restrict__ S, const float* __restrict__ signs,
                                                            int N, int nsb, double inv_sqrt_d) {
    constexpr int NV = D / 4;   // values per thread: x[4 k + j] is element 16 k + 4 qd + j
    __shared__ float wmax[kPrepThreads / kWave];
    const int tid = threadIdx.x;
    const int blk = blockIdx.x;            // (bh, sb) flattened
    const int bh = blk / nsb;
    const int sb = blk - bh * nsb;
    const int row = sb * kRowsPerScale + (tid >> 2);
    const int qd = tid & 3;                // quarter of the row; the 4 quarters are one lane quad
    const bool ok = row < N;
    const size_t base = ((size_t)bh * N + (ok ? row : 0)) * D + 4 * qd;   // element 16 k + 4 qd + j

    // rows past N (ragged last block) read as zero through the buffer's range check
    const __amdgpu_buffer_rsrc_t rX =
        __builtin_amdgcn_make_buffer_rsrc((void*)(X + (size_t)bh * N * D), (short)0, N * D * 4, kBufferConfig);
    const int off = (row * D + 4 * qd) * 4;
    float x[NV];
#pragma unroll
    for (int i = 0; i < NV; i += 4) {
        const f32x4 v = __builtin_bit_cast(f32x4, buffer_load16(rX, off + 16 * i));
        x[i] = v[0]; x[i + 1] = v[1]; x[i + 2] = v[2]; x[i + 3] = v[3];
    }
    if (signs != nullptr) {
        // the rotation in fp64, rounded once to fp32: the partial sums of the transform are exact
        // in fp64 for fp32 inputs of moderate range, so the result is x M to within ~1e-16
        // relative, the float64 product of the definition, and rounds to the same fp32 value
        // except within ~1e-15 of a rounding midpoint
        double y[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) y[i] = (double)x[i];
        // in-thread butterflies: register strides 1 .. NV/2 (element bits 0, 1 and 4 ..)
#pragma unroll
        for (int st = 1; st < NV; st <<= 1)
#pragma unroll
            for (int i = 0; i < NV; ++i)
                if ((i & st) == 0) {
                    const double a = y[i], b = y[i + st];
                    y[i] = a + b;
                    y[i + st] = a - b;
                }
        // cross-thread butterflies: element bits 2 and 3 (lane xor 1, xor 2); the lower
        // partner keeps x + y, the upper one y - x, i.e. (+-x) + y, one fused multiply-add
        // (the product by +-1 is exact, so it rounds as the sum alone)
        const double sg1 = (qd & 1) ? -1.0 : 1.0;
        const double sg2 = (qd & 2) ? -1.0 : 1.0;
#pragma unroll
        for (int i = 0; i < NV; ++i) y[i] = __fma_rn(y[i], sg1, quad_xor_d<0xB1>(y[i]));
#pragma unroll
        for (int i = 0; i < NV; ++i) y[i] = __fma_rn(y[i], sg2, quad_xor_d<0x4E>(y[i]));
        // signs and 1/sqrt(d) in one multiply (+-c is exact), then the one rounding to fp32
#pragma unroll
        for (int i = 0; i < NV; i += 4) {
            const f32x4 sv = *(const f32x4*)(signs + 4 * i + 4 * qd);
#pragma unroll
            for (int u = 0; u < 4; ++u) x[i + u] = (float)(y[i + u] * ((double)sv[u] * inv_sqrt_d));
        }
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
    const float r = __fdiv_rn(1.f, s);     // RN(1/s)
    const bool tiny = s < 1.17549435e-38f; // subnormal scale: quotients may exceed 448
    if (tid == 0) S[(size_t)bh * nsb + sb] = s;
    if (!ok) return;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const float q0 = __fmul_rn(x[i], r);
        // RN(x / s); the correction turns a -0 quotient into +0, so the sign is taken from x
        // (s > 0: x / s has the sign of x, and E4M3 keeps -0 as its own code)
        x[i] = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q0, s, x[i]), r, q0), x[i]);
    }
    if (tiny) {   // uniform per block, rare
#pragma unroll
        for (int i = 0; i < NV; ++i)
            x[i] = x[i] > kE4m3Max ? kE4m3Max : (x[i] < -kE4m3Max ? -kE4m3Max : x[i]);   // keeps NaN
    }
    uint8_t* out = X8 + base;
#pragma unroll
    for (int i = 0; i < NV; i += 4) {
        const float* y = x + i;
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
        *(int*)(out + 4 * i) = word;
    }
}

template <int D>
hipError_t launch_prep(const float* x, void* x8, float* s, const float* signs, int BH, int N, hipStream_t stream) {
    const int nsb = (N + kRowsPerScale - 1) / kRowsPerScale;
    const long long total = (long long)BH * nsb;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((prep_fp8_kernel<D>), dim3((unsigned)total), dim3(kPrepThreads), 0, stream, x, (uint8_t*)x8, s,
                       signs, N, nsb, 1.0 / std::sqrt((double)D));
    return hipGetLastError();
}

template <int D, int BC, int NQ, int MINB, bool PIPE, int WAVES = 4, int DSPLIT = 1>
hipError_t dispatch_fp8(const void* q8, const void* k8, const void* v8, const float* sq, const float* sk,
                        const float* sv, void* o, float* lse, int BH, int N, float scale, bool causal,
                        hipStream_t stream) {
    constexpr InKind K = InKind::FP8;
    return causal ? launch_fwd_kernel<K, D, BC, NQ, true, 8, MINB, PIPE, WAVES, false, DSPLIT>(
                        q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, stream)
                  : launch_fwd_kernel<K, D, BC, NQ, false, 8, MINB, PIPE, WAVES, false, DSPLIT>(
                        q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, stream);
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
    // key blocks of 64 keys (one scale block) or, for d = 128 and 256, 32 (half of one; fewer
    // live registers, as for bf16); conditional rescale threshold 2^8. d = 128: 8 waves (256
    // queries) share each K/V tile, one workgroup per CU; the 4 KB e4m3 K tile is loaded by
    // four of them, and all eight expand V (+1.4% over 4-wave workgroups). d = 256: 8 waves in
    // pairs that split the head dimension (each wave holds Q and O for 128 columns, the
    // d = 128 footprint), one workgroup of 128 queries per CU, as for bf16
    switch (d) {
        case 64: return dispatch_fp8<64, 64, 1, 2, true>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, causal, stream);
        case 128: return dispatch_fp8<128, 32, 1, 1, true, 8>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, causal, stream);
        case 256:
            return dispatch_fp8<256, 32, 1, 1, true, 8, 2>(q8, k8, v8, sq, sk, sv, o, lse, BH, N, scale, causal, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
