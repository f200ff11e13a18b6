// bf16 attention forward for short sequences (N <= 128, d = 64 or 128): one workgroup per
// (batch, head) holds the head's whole key and value range in LDS.
//
// With N <= 128 the streaming kernel's workgroup runs only a few key blocks, each waiting for
// the tile loads of the next, and the bytes in flight over the chip (two 16 KB tiles per
// workgroup) are too few to cover the memory latency: such problems are bound by memory
// latency, not bandwidth. Here K and V of the head (at most 2 x 32 KB) are requested at once
// and waited for once. The softmax is then computed exactly in two passes over scores held in
// registers ("Learn: The Memory Wall & FlashAttention", section 3, the three-loop safe
// softmax with the row max taken over all keys first): S for every key block, the row max,
// then P = exp2(S c - m), the row sum and O = P V; no running rescale is needed.
//
// Layouts are those of the streaming kernels: 4 waves x 32 queries; S^T = K Q^T with the key
// tiles read as MFMA rows, O^T += V^T P^T with V read through the transposing LDS read (the
// tile helpers shared with the backward).
#include "fa_fwd_kernel.h"   // kBufferConfig
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int kShortRows = 128;   // the longest sequence one workgroup holds (4 key blocks of 32)

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_short_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                                                          const bf16_t* __restrict__ V, bf16_t* __restrict__ O,
                                                          float* __restrict__ LSE, int N, float c2 /* scale*log2(e) */) {
    using C = TileCfg<D, 32, 4>;
    constexpr int NB = kShortRows / 32;   // key blocks held
    __shared__ __attribute__((aligned(1024))) uint8_t sK[NB * C::TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sV[NB * C::TB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    const int bh = blockIdx.x;
    const size_t head = (size_t)bh * N * D;
    const int q0w = 32 * wave;
    const int qrow = q0w + col;

    // every key and value row of the head, in one go (rows past N read as zero)
    const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc((void*)(K + head), (short)0, N * C::ROW, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc((void*)(V + head), (short)0, N * C::ROW, kBufferConfig);
    TileAddr<D, 32, 4> ta;
    ta.init(wave, lane);
    const int nkb = (N + 31) / 32;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        if (j < nkb) {
            ta.load(rK, sK + j * C::TB, 32 * j, wave);
            ta.load(rV, sV + j * C::TB, 32 * j, wave);
        }
    }
    bf16x8 qf[C::KSTEPS];
    load_resident<D>(qf, Q + head, qrow, N, h);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // the key blocks this wave's queries see (causal: up to its last query)
    const int nkw = CAUSAL ? min(nkb, (min(q0w + 32, N) - 1) / 32 + 1) : nkb;
    // register i of block j holds key 32 j + 16(i/8) + 8h + i%8 of query qrow; it is visible
    // iff that offset from 8h is at most lim
    const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - 8 * h;

    // pass 1: scores and the row max
    f32x16 st[NB];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        if (j < nkw) {
            st[j] = f32x16{};
#pragma unroll
            for (int s = 0; s < C::KSTEPS; ++s)
                st[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row_operand(sK + j * C::TB, s), qf[s], st[j], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int off = 32 * j + 16 * (i / 8) + (i % 8);
                st[j][i] = off > lim ? -INFINITY : st[j][i];
                mx = fmaxf(mx, st[j][i]);
            }
        }
    }
    // lanes l and l^32 hold the two halves of a row; every row sees at least one key
    const float m2 = pair_max(mx) * c2;

    // pass 2: P = exp2(S c - m), the row sum (of fp32 P) and O^T += V^T P^T
    f32x16 acc[C::DT];
#pragma unroll
    for (int e = 0; e < C::DT; ++e) acc[e] = f32x16{};
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        if (j < nkw) {
            // causal: the first rows see only a few keys, where rounding P to bf16 would cost up to
            // 2^-9 of the largest value's magnitude; P is carried as P_hi + P_lo (two bf16 terms)
            // and each block takes two PV products (the kernel is bound by memory, not MFMA)
            bf16x8 pf[2], plo[CAUSAL ? 2 : 1];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(__builtin_fmaf(st[j][i], c2, -m2));
                lsum += p;
                const bf16_t ph = (bf16_t)p;
                pf[i / 8][i % 8] = ph;
                if constexpr (CAUSAL) plo[i / 8][i % 8] = (bf16_t)(p - (float)ph);   // p - ph is exact
            }
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int e = 0; e < C::DT; ++e) {
                    const bf16x8 a = ta.tr_operand(sV + j * C::TB, e, ch);
                    acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[ch], acc[e], 0, 0, 0);
                    if constexpr (CAUSAL) acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, plo[ch], acc[e], 0, 0, 0);
                }
        }
    }
    const float l_tot = pair_sum(lsum);
    if (LSE != nullptr && h == 0 && qrow < N) LSE[(size_t)bh * N + qrow] = (m2 + __log2f(l_tot)) * kLn2;

    // O = O~ / l, staged per wave in the K tiles once every wave is done reading them
    __syncthreads();
    store_rows<D>(acc, 1.f / l_tot, sK + wave * C::TB, O + head, q0w, N, lane);
}

template <int D>
hipError_t launch_short(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, float scale,
                        bool causal, hipStream_t stream) {
    const float c2 = scale * kLog2e;
    if (causal)
        hipLaunchKernelGGL((fwd_short_kernel<D, true>), dim3(BH), dim3(256), 0, stream, (const bf16_t*)q,
                           (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)o, lse, N, c2);
    else
        hipLaunchKernelGGL((fwd_short_kernel<D, false>), dim3(BH), dim3(256), 0, stream, (const bf16_t*)q,
                           (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)o, lse, N, c2);
    return hipGetLastError();
}

}  // namespace

bool short_fwd_applies(int N, int d) { return N >= 1 && N <= kShortRows && (d == 64 || d == 128); }

hipError_t launch_fwd_short_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                                 float scale, bool causal, hipStream_t stream) {
    if (!short_fwd_applies(N, d)) return hipErrorInvalidValue;
    return d == 64 ? launch_short<64>(q, k, v, o, lse, BH, N, scale, causal, stream)
                   : launch_short<128>(q, k, v, o, lse, BH, N, scale, causal, stream);
}

}  // namespace fa
