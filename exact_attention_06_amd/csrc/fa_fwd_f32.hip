// fp32 attention forward: the same fused online-softmax kernel as the bf16 one, but with
// every product and every stored value in fp32 (v_mfma_f32_32x32x2_f32, fp32 LDS tiles,
// fp32 O). It exists for callers that need fp32 end to end; it is not tuned for speed.
//
// Work split and recurrence as in the bf16 kernel ("FlashAttention 2 & 3" page, sections
// "Edit 1" to "Edit 3"; "Learn: The Memory Wall & FlashAttention", section 5.1):
// 4 waves x 32 queries per workgroup, S^T = K_j Q_i^T per 32-key block, online softmax
// state in registers, one division at the end. Differences from the bf16 kernel:
// - one k = 2 product per MFMA: lane half h carries head-dim coordinate s + (d/2) h at
//   step s (A and B agree on it, which is all the contraction needs);
// - the PV product takes 2 keys per MFMA; result register c of lane half h is the key the
//   instruction pairs with lane half h, so the V^T operand is V[key(c, h)][d], one fp32
//   LDS read per product, and K rows need no permutation;
// - single-buffered K/V tiles;
// - small grids take fwd_f32_split_kernel (keys split over the waves, states merged).
#include "fa_common.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kBR = 128;
constexpr int kThreads = 256;
constexpr int kBC = 32;   // keys per block
constexpr int kSmallGrid = 256;   // one workgroup per compute unit

template <int D, bool CAUSAL, int MINB>
__global__ __launch_bounds__(kThreads, MINB) void fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V, float* __restrict__ O,
    float* __restrict__ LSE, int N, int numQB, float c2) {
    constexpr int KP = D + 4;          // K pitch (floats): +16 bytes
    constexpr int VP = D + 4;
    constexpr int HALF = D / 2;
    constexpr int DT = D / 32;
    __shared__ __attribute__((aligned(16))) float smK[kBC * KP];
    __shared__ __attribute__((aligned(16))) float smV[kBC * VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int col = lane & 31;

    const int w = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = w / numQB;
    const int qi = w - bh * numQB;
    const int qb = CAUSAL ? (numQB - 1 - qi) : qi;
    const int q0 = qb * kBR;
    const int q0w = q0 + wave * 32;
    const int qrow = q0w + col;

    const size_t head_off = (size_t)bh * N * D;
    const float* Qh = Q + head_off;
    const float* Kh = K + head_off;
    const float* Vh = V + head_off;

    const int nkb_all = (N + kBC - 1) / kBC;
    int nkb = nkb_all;
    if (CAUSAL) nkb = min(nkb_all, (min(q0 + kBR, N) - 1) / kBC + 1);

    // Q operand: lane half h holds d = HALF*h + s
    float qf[HALF];
    {
        const bool ok = qrow < N;
        const float* qp = Qh + (size_t)(ok ? qrow : 0) * D + HALF * h;
#pragma unroll
        for (int s = 0; s < HALF; s += 4) {
            f32x4 x = *(const f32x4*)(qp + s);
            if (!ok) x = f32x4{};
            qf[s] = x[0]; qf[s + 1] = x[1]; qf[s + 2] = x[2]; qf[s + 3] = x[3];
        }
    }

    f32x16 acc[DT];
#pragma unroll
    for (int e = 0; e < DT; ++e) acc[e] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    for (int j = 0; j < nkb; ++j) {
        const int kb = j * kBC;
        // ---- load the K/V block (16-byte chunks; rows past N are zero)
        for (int x = tid; x < kBC * D / 4; x += kThreads) {
            const int row = x / (D / 4);
            const int c4 = x % (D / 4);
            const int grow = kb + row;
            f32x4 kv = f32x4{}, vv = f32x4{};
            if (grow < N) {
                kv = *(const f32x4*)(Kh + (size_t)grow * D + 4 * c4);
                vv = *(const f32x4*)(Vh + (size_t)grow * D + 4 * c4);
            }
            *(f32x4*)(&smK[row * KP + 4 * c4]) = kv;
            *(f32x4*)(&smV[row * VP + 4 * c4]) = vv;
        }
        __syncthreads();

        const bool active = (q0w < N) && (!CAUSAL || kb <= q0w + 31);
        if (active) {
            // ---- S^T = K_j Q_i^T (one 32-key tile)
            f32x16 st = f32x16{};
            const float* kp = smK + col * KP + HALF * h;
#pragma unroll
            for (int s = 0; s < HALF; s += 4) {
                const f32x4 a = *(const f32x4*)(kp + s);
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    st = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u], qf[s + u], st, 0, 0, 0);
            }
            const bool need_mask = (kb + kBC > N) || (CAUSAL && kb + kBC - 1 > q0w);
            if (need_mask) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kb + mfma32_row(i, h);
                    if (key >= N || (CAUSAL && key > qrow)) st[i] = -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[i]);
            mx = pair_max(mx) * c2;
            const float m_new = fmaxf(m_run, mx);
            const bool grow = m_new > m_run + kRescaleTau;
            if (wave_any(grow)) {
                const float m_ref = grow ? m_new : m_run;
                const float alpha = (m_ref == -INFINITY) ? 1.f : fast_exp2(m_run - m_ref);
                m_run = m_ref;
                l_run *= alpha;
#pragma unroll
                for (int e = 0; e < DT; ++e)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[e][i] *= alpha;
            }
            const float msub = (m_run == -INFINITY) ? 0.f : m_run;
            float p[16];
            float lsum = 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                p[i] = fast_exp2(__builtin_fmaf(st[i], c2, -msub));
                lsum += p[i];
            }
            l_run += lsum;
            // ---- O^T += V_j^T P^T, 2 keys per product: key(c, h) = mfma32_row(c, h)
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const float* vp = smV + mfma32_row(c, h) * VP + col;
#pragma unroll
                for (int e = 0; e < DT; ++e)
                    acc[e] = __builtin_amdgcn_mfma_f32_32x32x2f32(vp[32 * e], p[c], acc[e], 0, 0, 0);
            }
        }
        __syncthreads();
    }

    const float l_tot = pair_sum(l_run);
    if (qrow < N) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float* op = O + head_off + (size_t)qrow * D + 4 * h;
#pragma unroll
        for (int e = 0; e < DT; ++e)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                f32x4 ov;
#pragma unroll
                for (int b = 0; b < 4; ++b) ov[b] = acc[e][4 * a + b] * inv;
                *(f32x4*)(op + 32 * e + 8 * a) = ov;
            }
        if (LSE != nullptr && h == 0)
            LSE[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

// Small problems (fewer 128-query blocks than compute units): 32 queries per workgroup, the
// key blocks dealt round-robin to its W waves (8 at d = 64, 4 at d = 128, as the LDS allows),
// each with its own tiles (synchronised within
// the wave only) and its own online-softmax state; the four states are then combined in LDS
// with the online-softmax merge ("FlashAttention-3 & GPU Kernel Optimization", section
// "Online softmax tiling mathematics"): m = max m_w, O = sum 2^(m_w - m) O~_w / sum
// 2^(m_w - m) l_w. A wave thus walks 1/W of the keys, which is what bounds these
// latency-bound launches.
template <int D>
constexpr int split_waves() { return D <= 64 ? 8 : 4; }

template <int D, bool CAUSAL, int kSplitWaves = split_waves<D>()>
__global__ __launch_bounds__(64 * kSplitWaves, 1) void fwd_f32_split_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V, float* __restrict__ O,
    float* __restrict__ LSE, int N, int numQT, float c2) {
    constexpr int KP = D + 4;
    constexpr int VP = D + 4;
    constexpr int HALF = D / 2;
    constexpr int DT = D / 32;
    constexpr int TILE = kBC * KP + kBC * VP;          // one wave's K and V tiles (floats)
    static_assert(kSplitWaves * DT * 16 * 64 + 2 * kSplitWaves * 64 <= kSplitWaves * TILE, "merge fits in the tiles");
    __shared__ __attribute__((aligned(16))) float sm[kSplitWaves * TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int col = lane & 31;
    const int bh = blockIdx.x / numQT;
    const int qt = blockIdx.x - bh * numQT;
    const int q0 = (CAUSAL ? numQT - 1 - qt : qt) * 32;   // causal: longest rows first
    const int qrow = q0 + col;
    float* const smK = sm + wave * TILE;
    float* const smV = smK + kBC * KP;

    const size_t head_off = (size_t)bh * N * D;
    const float* Qh = Q + head_off;
    const float* Kh = K + head_off;
    const float* Vh = V + head_off;
    int nkb = (N + kBC - 1) / kBC;
    if (CAUSAL) nkb = min(nkb, (min(q0 + 32, N) - 1) / kBC + 1);

    float qf[HALF];
    {
        const bool ok = qrow < N;
        const float* qp = Qh + (size_t)(ok ? qrow : 0) * D + HALF * h;
#pragma unroll
        for (int s = 0; s < HALF; s += 4) {
            f32x4 x = *(const f32x4*)(qp + s);
            if (!ok) x = f32x4{};
            qf[s] = x[0]; qf[s + 1] = x[1]; qf[s + 2] = x[2]; qf[s + 3] = x[3];
        }
    }
    f32x16 acc[DT];
#pragma unroll
    for (int e = 0; e < DT; ++e) acc[e] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    for (int j = wave; j < nkb; j += kSplitWaves) {
        const int kb = j * kBC;
        // this wave's K/V block (rows past N are zero)
        for (int x = lane; x < kBC * D / 4; x += kWave) {
            const int row = x / (D / 4);
            const int c4 = x % (D / 4);
            const int grow = kb + row;
            f32x4 kv = f32x4{}, vv = f32x4{};
            if (grow < N) {
                kv = *(const f32x4*)(Kh + (size_t)grow * D + 4 * c4);
                vv = *(const f32x4*)(Vh + (size_t)grow * D + 4 * c4);
            }
            *(f32x4*)(&smK[row * KP + 4 * c4]) = kv;
            *(f32x4*)(&smV[row * VP + 4 * c4]) = vv;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave reads what its lanes wrote
        __builtin_amdgcn_wave_barrier();

        f32x16 st = f32x16{};
        const float* kp = smK + col * KP + HALF * h;
#pragma unroll
        for (int s = 0; s < HALF; s += 4) {
            const f32x4 a = *(const f32x4*)(kp + s);
#pragma unroll
            for (int u = 0; u < 4; ++u) st = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u], qf[s + u], st, 0, 0, 0);
        }
        if ((kb + kBC > N) || (CAUSAL && kb + kBC - 1 > q0)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kb + mfma32_row(i, h);
                if (key >= N || (CAUSAL && key > qrow)) st[i] = -INFINITY;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[i]);
        mx = pair_max(mx) * c2;
        const float m_new = fmaxf(m_run, mx);
        const bool grow = m_new > m_run + kRescaleTau;
        if (wave_any(grow)) {
            const float m_ref = grow ? m_new : m_run;
            const float alpha = (m_ref == -INFINITY) ? 1.f : fast_exp2(m_run - m_ref);
            m_run = m_ref;
            l_run *= alpha;
#pragma unroll
            for (int e = 0; e < DT; ++e)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[e][i] *= alpha;
        }
        const float msub = (m_run == -INFINITY) ? 0.f : m_run;
        float p[16];
        float lsum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[i] = fast_exp2(__builtin_fmaf(st[i], c2, -msub));
            lsum += p[i];
        }
        l_run += lsum;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const float* vp = smV + mfma32_row(c, h) * VP + col;
#pragma unroll
            for (int e = 0; e < DT; ++e)
                acc[e] = __builtin_amdgcn_mfma_f32_32x32x2f32(vp[32 * e], p[c], acc[e], 0, 0, 0);
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // the tile reads are done before the next block's writes
        __builtin_amdgcn_wave_barrier();
    }

    // ---- merge: every wave leaves (m, l, O~) in LDS, lane-major; wave 0 combines them. A
    // wave that saw no visible key has m = -inf and weight 0.
    __syncthreads();   // every wave is done with its tiles
    float* const mo = sm;                                    // [wave][e][i][lane]
    float* const ml = sm + kSplitWaves * DT * 16 * 64;       // [wave][m | l][lane]
#pragma unroll
    for (int e = 0; e < DT; ++e)
#pragma unroll
        for (int i = 0; i < 16; ++i) mo[((wave * DT + e) * 16 + i) * 64 + lane] = acc[e][i];
    ml[(wave * 2) * 64 + lane] = m_run;
    ml[(wave * 2 + 1) * 64 + lane] = l_run;
    __syncthreads();
    if (wave == 0) {
        float mw[kSplitWaves], m_all = -INFINITY;
#pragma unroll
        for (int w = 0; w < kSplitWaves; ++w) {
            mw[w] = ml[(w * 2) * 64 + lane];
            m_all = fmaxf(m_all, mw[w]);
        }
        float sw[kSplitWaves], l_part = 0.f;
#pragma unroll
        for (int w = 0; w < kSplitWaves; ++w) {
            sw[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - m_all);
            l_part += sw[w] * ml[(w * 2 + 1) * 64 + lane];
        }
        const float l_tot = pair_sum(l_part);   // lanes l and l^32 hold the two halves of a row's sum
        if (qrow < N) {
            const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
            float* op = O + head_off + (size_t)qrow * D + 4 * h;
#pragma unroll
            for (int e = 0; e < DT; ++e)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f32x4 ov;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        float x = 0.f;
#pragma unroll
                        for (int w = 0; w < kSplitWaves; ++w) x += sw[w] * mo[((w * DT + e) * 16 + 4 * a + b) * 64 + lane];
                        ov[b] = x * inv;
                    }
                    *(f32x4*)(op + 32 * e + 8 * a) = ov;
                }
            if (LSE != nullptr && h == 0) LSE[(size_t)bh * N + qrow] = l_tot > 0.f ? (m_all + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
}

template <int D, bool CAUSAL>
hipError_t launch_split(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, float scale,
                        hipStream_t stream) {
    const int numQT = (N + 31) / 32;
    hipLaunchKernelGGL((fwd_f32_split_kernel<D, CAUSAL>), dim3((unsigned)(BH * numQT)), dim3(64 * split_waves<D>()), 0, stream,
                       (const float*)q, (const float*)k, (const float*)v, (float*)o, lse, N, numQT, scale * kLog2e);
    return hipGetLastError();
}

template <int D, bool CAUSAL, int MINB>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, float scale,
                  hipStream_t stream) {
    const int numQB = (N + kBR - 1) / kBR;
    const long long total = (long long)BH * numQB;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, MINB>), dim3((unsigned)total), dim3(kThreads), 0, stream,
                       (const float*)q, (const float*)k, (const float*)v, (float*)o, lse, N, numQB, scale * kLog2e);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                          float scale, bool causal, hipStream_t stream) {
    // fewer 128-query blocks than compute units: split each block's keys over its waves
    if (d <= 128 && (long long)BH * ((N + kBR - 1) / kBR) < kSmallGrid) {
        if (d == 64) return causal ? launch_split<64, true>(q, k, v, o, lse, BH, N, scale, stream)
                                   : launch_split<64, false>(q, k, v, o, lse, BH, N, scale, stream);
        return causal ? launch_split<128, true>(q, k, v, o, lse, BH, N, scale, stream)
                      : launch_split<128, false>(q, k, v, o, lse, BH, N, scale, stream);
    }
    switch (d) {
        case 64:
            return causal ? launch<64, true, 2>(q, k, v, o, lse, BH, N, scale, stream)
                          : launch<64, false, 2>(q, k, v, o, lse, BH, N, scale, stream);
        case 128:
            return causal ? launch<128, true, 1>(q, k, v, o, lse, BH, N, scale, stream)
                          : launch<128, false, 1>(q, k, v, o, lse, BH, N, scale, stream);
        case 256:
            return causal ? launch<256, true, 1>(q, k, v, o, lse, BH, N, scale, stream)
                          : launch<256, false, 1>(q, k, v, o, lse, BH, N, scale, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace fa
