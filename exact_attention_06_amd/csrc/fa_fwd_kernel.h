// The fused attention forward kernel shared by the bf16 and the e4m3 (FP8) inputs.
//
// Algorithm: the FA2 loop order ("FlashAttention 2 & 3: Work Partitioning, Warp
// Specialization & FP8", sections "Edit 1" to "Edit 3"): one workgroup owns 128 queries of
// one (batch, head) and streams every key/value block of that head through LDS, keeping the
// online-softmax state ("Learn: The Memory Wall & FlashAttention", section 5.1: running max
// m, running sum l, unnormalised accumulator o) in registers; the division by l happens once
// at the end, together with the logsumexp L = m + log l.
//
// CDNA4 mapping:
// - 4 waves x 32 queries. Each wave computes S^T = K_j Q_i^T (keys x queries) on the matrix
//   cores (bf16: v_mfma_f32_32x32x16_bf16; FP8: v_mfma_scale_f32_32x32x64_f8f6f4 with unit
//   MX scales), so the scores of one query sit in one lane (16 per 32-key tile) and its
//   partner lane l^32: row max and row sum are in-register reductions plus one
//   v_permlane32_swap. A wave's queries never interact with another wave's (split-Q).
// - K rows are fed to the MFMA in the order swap_bits23, so the S^T result registers are
//   already the B operand (P^T) of O^T += V_j^T P^T in bf16; P never leaves registers.
// - V^T is read from the row-major bf16 V tile with ds_read_b64_tr_b16 (8 keys of one d
//   column per lane in two reads).
// - K/V tiles are double-buffered in LDS: the global loads of block j+1 are issued before
//   the math on block j and written to the other buffer after it; one barrier per block.
// - The accumulator is rescaled only when a row maximum grows by more than 2^TAU (the
//   conditional rescaling of the FA4 section of the memory-wall page). The result stays
//   exact (numerator and denominator use the same reference); P is bounded by 2^TAU.
// - Causal: key blocks entirely above the workgroup's diagonal are never visited; a wave
//   whose 32 queries all precede a key block skips its math; only blocks that straddle the
//   diagonal are masked element by element. Each head's query blocks are walked heaviest
//   first, and the XCD-aware remap keeps a head's blocks on one XCD (one L2).
//
// FP8 inputs ("FlashAttention-3: How Warp Specialization ...", section 4 "Technique 3";
// "FlashAttention 2 & 3", section "What stays in higher precision"):
// - Q8 and K8 are e4m3 with one fp32 scale per 64 rows; 64-key blocks match the scale
//   blocks, so the score of the block is s_Q s_K (Q8 K8^T) and s_Q s_K is folded into the
//   FMA that subtracts the running max;
// - V stays e4m3 in HBM and is expanded exactly to bf16 when it is written to LDS (every
//   e4m3 value is a bf16 value); its block scale rides on P: P_j is computed as
//   exp2(S ct - m + log2(s_V(j) / max s_V)) in the same FMA (no extra per-element work),
//   the row sum divides the ratio back out once per block, and max s_V is applied with the
//   final division. P is rounded to bf16, not e4m3, for the PV product: with e4m3 P the
//   output error on inputs with outliers is an order of magnitude above the 6e-2 budget.
#pragma once

#include "fa_common.h"

namespace fa {

enum class InKind { BF16, FP8 };

constexpr int kBR = 128;        // queries per workgroup
constexpr int kThreads = 256;   // 4 waves

template <InKind KIND, int D, int BC>
struct FwdCfg {
    static constexpr bool F8 = KIND == InKind::FP8;
    static constexpr int IN_BYTES = F8 ? 1 : 2;            // bytes per element in HBM
    static constexpr int ROW_BYTES = D * IN_BYTES;          // bytes per K/V row in HBM
    static constexpr int KP = ROW_BYTES + 16;               // LDS pitch of K rows (bytes): 4-bank shift
    static constexpr int VP = D + 16;                       // LDS pitch of bf16 V rows (elements): 8-bank shift
    static constexpr int QK_K = F8 ? 64 : 16;               // contraction length of one QK MFMA
    static constexpr int KSTEPS = D / QK_K;
    static constexpr int MT = BC / 32;                      // 32-key tiles per block
    static constexpr int DT = D / 32;                       // 32-wide d tiles of O^T
    static constexpr int CH = BC / 16;                      // 16-key chunks of the PV product
    static constexpr int CPT = BC * ROW_BYTES / 16 / kThreads;   // 16-byte chunks per thread per tensor
    static_assert(CPT >= 1 && CPT * kThreads * 16 == BC * ROW_BYTES, "tile must split evenly");
    static constexpr int K_BYTES = BC * KP;
    static constexpr int V_BYTES = BC * VP * 2;
};

template <InKind KIND>
struct QOperand;
template <>
struct QOperand<InKind::BF16> { typedef bf16x8 type; };
template <>
struct QOperand<InKind::FP8> { typedef i32x8 type; };

template <InKind KIND, int D, int BC, bool CAUSAL, int TAU, int MINB>
__global__ __launch_bounds__(kThreads, MINB) void fwd_kernel(
    const void* __restrict__ Qv, const void* __restrict__ Kv, const void* __restrict__ Vv,
    const float* __restrict__ SQ, const float* __restrict__ SK, const float* __restrict__ SV,
    bf16_t* __restrict__ O, float* __restrict__ LSE, int N, int numQB, int nsb, float c2 /* scale*log2(e) */) {
    using C = FwdCfg<KIND, D, BC>;
    using QT = typename QOperand<KIND>::type;
    constexpr float tau = (float)TAU;
    __shared__ __attribute__((aligned(16))) uint8_t smK[2][C::K_BYTES];
    __shared__ __attribute__((aligned(16))) bf16_t smV[2][BC * C::VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;        // lane half
    const int col = lane & 31;      // query column owned by this lane

    const int w = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = w / numQB;
    const int qi = w - bh * numQB;
    const int qb = CAUSAL ? (numQB - 1 - qi) : qi;
    const int q0 = qb * kBR;
    const int q0w = q0 + wave * 32;
    const int qrow = q0w + col;

    const size_t head_off = (size_t)bh * N * D;   // elements
    const uint8_t* Qh = (const uint8_t*)Qv + head_off * C::IN_BYTES;
    const uint8_t* Kh = (const uint8_t*)Kv + head_off * C::IN_BYTES;
    const uint8_t* Vh = (const uint8_t*)Vv + head_off * C::IN_BYTES;

    const int nkb_all = (N + BC - 1) / BC;
    int nkb = nkb_all;
    if (CAUSAL) nkb = min(nkb_all, (min(q0 + kBR, N) - 1) / BC + 1);

    // score scale (log2 units); FP8 adds the Q block scale of this wave
    float cq = c2;
    float svmax = 1.f;   // FP8: largest V block scale of this head
    if constexpr (C::F8) {
        cq *= (q0w < N) ? SQ[(size_t)bh * nsb + q0w / 64] : 1.f;
        float mx = 0.f;
        for (int i = lane; i < nkb_all; i += kWave) mx = fmaxf(mx, SV[(size_t)bh * nsb + i]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
        svmax = mx;
    }

    // ---- Q^T operand (B of S^T = K Q^T): lane holds query `qrow`; step s covers head-dim
    // elements [QK_K s + (QK_K/2) h, +QK_K/2)
    QT qf[C::KSTEPS];
    {
        const bool ok = qrow < N;
        const uint8_t* qp = Qh + (size_t)(ok ? qrow : 0) * C::ROW_BYTES + (C::QK_K / 2) * C::IN_BYTES * h;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            const uint8_t* p = qp + s * C::QK_K * C::IN_BYTES;
            if constexpr (C::F8) {
                const i32x4 lo = ok ? *(const i32x4*)p : i32x4{};
                const i32x4 hi = ok ? *(const i32x4*)(p + 16) : i32x4{};
                qf[s] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                qf[s] = ok ? *(const bf16x8*)p : bf16x8{};
            }
        }
    }

    // ---- K/V staging: each thread moves CPT 16-byte chunks of K and of V per block
    i32x4 kst[C::CPT], vst[C::CPT];
    auto load_tile = [&](int kb) {
#pragma unroll
        for (int r = 0; r < C::CPT; ++r) {
            const int x = tid + kThreads * r;
            const int row = x / (C::ROW_BYTES / 16);
            const int c16 = x % (C::ROW_BYTES / 16);
            const int grow = kb + row;
            if (grow < N) {
                kst[r] = *(const i32x4*)(Kh + (size_t)grow * C::ROW_BYTES + 16 * c16);
                vst[r] = *(const i32x4*)(Vh + (size_t)grow * C::ROW_BYTES + 16 * c16);
            } else {
                kst[r] = i32x4{};
                vst[r] = i32x4{};
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int r = 0; r < C::CPT; ++r) {
            const int x = tid + kThreads * r;
            const int row = x / (C::ROW_BYTES / 16);
            const int c16 = x % (C::ROW_BYTES / 16);
            *(i32x4*)(&smK[buf][row * C::KP + 16 * c16]) = kst[r];
            if constexpr (C::F8) {
                // 16 e4m3 values -> 16 bf16 values, exact (the convert's scale operand only
                // contributes its power of two, so it is left at 1 and s_V is applied to P)
                i32x4 lo, hi;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vst[r][u], 1.f, false);
                    const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(vst[r][u], 1.f, true);
                    const int wa = __builtin_bit_cast(int, a);
                    const int wb = __builtin_bit_cast(int, b);
                    if (u < 2) { lo[2 * u] = wa; lo[2 * u + 1] = wb; }
                    else { hi[2 * (u - 2)] = wa; hi[2 * (u - 2) + 1] = wb; }
                }
                *(i32x4*)(&smV[buf][row * C::VP + 16 * c16]) = lo;
                *(i32x4*)(&smV[buf][row * C::VP + 16 * c16 + 8]) = hi;
            } else {
                *(i32x4*)(&smV[buf][row * C::VP + 8 * c16]) = vst[r];
            }
        }
    };

    // ---- online-softmax state (log2 domain: m is a running max of S * scale * log2 e)
    f32x16 acc[C::DT];
#pragma unroll
    for (int e = 0; e < C::DT; ++e) acc[e] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // per-lane key offsets of the 16 result registers within a 32-key tile
    int koff[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) koff[i] = swap_bits23(mfma32_row(i, h));
    const int krow_a = swap_bits23(col);   // key row this lane feeds into A-operand row `col`

    load_tile(0);
    store_tile(0);
    __syncthreads();

    for (int j = 0; j < nkb; ++j) {
        const int buf = j & 1;
        const int kb = j * BC;
        if (j + 1 < nkb) load_tile(kb + BC);

        const bool active = (q0w < N) && (!CAUSAL || kb <= q0w + 31);
        if (active) {
            const uint8_t* sk = smK[buf];
            const bf16_t* sv = smV[buf];
            // ---- S^T = K_j Q_i^T
            f32x16 st[C::MT];
#pragma unroll
            for (int t = 0; t < C::MT; ++t) {
                st[t] = f32x16{};
                const uint8_t* kp = sk + (32 * t + krow_a) * C::KP + (C::QK_K / 2) * C::IN_BYTES * h;
#pragma unroll
                for (int s = 0; s < C::KSTEPS; ++s) {
                    const uint8_t* p = kp + s * C::QK_K * C::IN_BYTES;
                    if constexpr (C::F8) {
                        const i32x4 lo = *(const i32x4*)p;
                        const i32x4 hi = *(const i32x4*)(p + 16);
                        const i32x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                        st[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[s], st[t], 0, 0, 0, 127, 0,
                                                                                 127);
                    } else {
                        const bf16x8 a = *(const bf16x8*)p;
                        st[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], st[t], 0, 0, 0);
                    }
                }
            }
            float ct = cq;
            if constexpr (C::F8) ct *= SK[(size_t)bh * nsb + j];
            // ---- masks: ragged tail of keys, causal diagonal
            const bool need_mask = (kb + BC > N) || (CAUSAL && kb + BC - 1 > q0w);
            if (need_mask) {
#pragma unroll
                for (int t = 0; t < C::MT; ++t)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kb + 32 * t + koff[i];
                        const bool hide = (key >= N) || (CAUSAL && key > qrow);
                        if (hide) st[t][i] = -INFINITY;
                    }
            }
            // ---- block row max, conditional rescale
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < C::MT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[t][i]);
            mx = pair_max(mx) * ct;
            const float m_new = fmaxf(m_run, mx);
            const bool grow = m_new > m_run + tau;
            if (wave_any(grow)) {
                const float m_ref = grow ? m_new : m_run;
                const float alpha = (m_ref == -INFINITY) ? 1.f : fast_exp2(m_run - m_ref);
                m_run = m_ref;
                l_run *= alpha;
#pragma unroll
                for (int e = 0; e < C::DT; ++e)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[e][i] *= alpha;
            }
            // ---- P = exp2(S ct - m), partial row sums, bf16 operand of the PV product
            // (FP8: P carries r = s_V(j) / max s_V, divided back out of the row sum)
            float bias = (m_run == -INFINITY) ? 0.f : -m_run;
            float inv_r = 1.f;
            if constexpr (C::F8) {
                const float r = SV[(size_t)bh * nsb + j] / svmax;
                bias += __log2f(r);
                inv_r = svmax / SV[(size_t)bh * nsb + j];
            }
            bf16x8 pf[C::CH];
            float lsum = 0.f;
#pragma unroll
            for (int t = 0; t < C::MT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(__builtin_fmaf(st[t][i], ct, bias));
                    lsum += p;
                    pf[2 * t + i / 8][i % 8] = (bf16_t)p;
                }
            if constexpr (C::F8) lsum *= inv_r;
            l_run += lsum;
            // ---- O^T += V_j^T P^T : A = V^T (d rows x 16 keys) via transposing LDS reads
            const int g = lane >> 4;       // 16-lane group
            const int L = lane & 15;
            const int vrow = 8 * (g >> 1) + (L >> 2);
            const int vcol = 16 * (g & 1) + 4 * (L & 3);
#pragma unroll
            for (int ch = 0; ch < C::CH; ++ch) {
#pragma unroll
                for (int e = 0; e < C::DT; ++e) {
                    const bf16_t* vp = sv + (16 * ch + vrow) * C::VP + 32 * e + vcol;
                    // keys 16ch + 8h + 0..3 and + 4..7 of column d, concatenated as whole vectors
                    // (element-wise assembly of the two halves is mis-compiled by the toolchain)
                    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(FA_LDS(bf16x4, vp));
                    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(FA_LDS(bf16x4, vp + 4 * C::VP));
                    const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ch], acc[e], 0, 0, 0);
                }
            }
        }
        if (j + 1 < nkb) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O~ / l, LSE = (m + log2 l) ln 2
    const float l_tot = pair_sum(l_run);   // lanes l and l^32 hold the two halves of a row's sum
    if (qrow < N) {
        const float inv = l_tot > 0.f ? svmax / l_tot : 0.f;
        bf16_t* op = O + head_off + (size_t)qrow * D + 4 * h;
#pragma unroll
        for (int e = 0; e < C::DT; ++e)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                bf16x4 ov;
#pragma unroll
                for (int b = 0; b < 4; ++b) ov[b] = (bf16_t)(acc[e][4 * a + b] * inv);
                *(bf16x4*)(op + 32 * e + 8 * a) = ov;
            }
        if (LSE != nullptr && h == 0)
            LSE[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

template <InKind KIND, int D, int BC, bool CAUSAL, int TAU, int MINB>
hipError_t launch_fwd_kernel(const void* q, const void* k, const void* v, const float* sq, const float* sk,
                             const float* sv, void* o, float* lse, int BH, int N, float scale, hipStream_t stream) {
    const int numQB = (N + kBR - 1) / kBR;
    const int nsb = (N + 63) / 64;
    const long long total = (long long)BH * numQB;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_kernel<KIND, D, BC, CAUSAL, TAU, MINB>), dim3((unsigned)total), dim3(kThreads), 0,
                       stream, q, k, v, sq, sk, sv, (bf16_t*)o, lse, N, numQB, nsb, scale * kLog2e);
    return hipGetLastError();
}

}  // namespace fa
