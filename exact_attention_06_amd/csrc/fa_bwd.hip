// bf16 attention backward: dQ, dK, dV from Q, K, V, O, dO and the forward's logsumexp.
//
// Source: "FlashAttention 2 & 3: Work Partitioning, Warp Specialization & FP8", section
// "The backward pass: recompute, and the one identity that makes it tile-able": the
// probabilities are rebuilt from the saved logsumexp, P = exp(S - L); dV = P^T dO,
// dP = dO V^T, D = rowsum(dO o O), dS = P o (dP - D), dQ = scale dS K, dK = scale dS^T Q.
// The same page (section "Edit 3" and the backward section) parallelises the backward over
// key blocks so that dK and dV accumulate locally, and names fp32 atomics or a separate pass
// for dQ; this file takes the separate pass (deterministic, no atomics):
//
// 1. bwd_delta_kernel: -D = -rowsum(dO o O) in fp32, one row per group of d/8 lanes, and the
//    exp2 bias -LSE log2(e) of every row (both into the caller's workspace). The dP products
//    start their accumulators from -D, so that they yield dP - D with no subtraction.
// 2. bwd_dq_kernel, parallel over 128-query blocks (the forward's layout): each wave keeps
//    Q^T and dO^T of its 32 queries in registers as MFMA B operands and streams 32-key blocks
//    of K and V through LDS. S^T = K Q^T and dP^T = V dO^T put one query in each lane pair;
//    P^T = exp2(S^T c - L log2 e) and dS^T = P^T o (dP^T - D) stay in registers and are the B
//    operand (bf16) of dQ^T += K^T dS^T, whose A operand K^T comes from the LDS transpose read.
// 3. bwd_dkdv_kernel (d = 64), parallel over 128-key blocks: each wave keeps K^T and V^T of
//    its 32 keys in registers and streams 32-query blocks of Q and dO through LDS. S = Q K^T and
//    dP = dO V^T put one key in each lane pair; P and dS (bf16) are the B operands of
//    dV^T += dO^T P and dK^T += Q^T dS, with dO^T and Q^T from the LDS transpose read.
//    At d = 128 the same work runs in bwd_dkdv_pair_kernel: 8 waves in pairs, one of each
//    pair holding K (S, P, dV) and the other V (dP, dS, dK), P passed through LDS.
//
// Every step loop issues the next tiles' loads at its top and waits for them only at its end
// (row values are loaded a step ahead, tile slots are separate LDS objects); causal waves or
// pairs work only on the blocks their own rows reach and take part in the rest of the
// workgroup's loads and barriers.
//
// MFMA layouts as in fa_common.h. The rows of the A operand of S / S^T are fed in the order
// swap_bits23, so that result registers 8u .. 8u+7 of lane half h hold rows 16u + 8h + 0..7:
// exactly the B operand of a 32x32x16 product over those 16 rows. Tiles are row-major bf16 in
// LDS, loaded straight from HBM (buffer_load ... lds; rows past N read as zero), 16-byte
// chunks XOR-swizzled (tile_slot) so that both the row reads and the transposing reads are
// free of bank conflicts.
#include "fa_common.h"
#include "fa_fwd_kernel.h"   // kBufferConfig
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int kBwdThreads = 256;   // 4 waves
constexpr int kBwdRows = 32;       // rows per streamed tile of the dq kernel (keys)
// waves of the dq kernel: 128 queries per workgroup, two workgroups per CU (256 queries per
// workgroup measured 7.25 vs 7.10 ms for the whole backward at 8k)
constexpr int kDqWaves = 4;

// ------------------------------------------------------------------------------------------
// -D = -rowsum(dO o O)
// ------------------------------------------------------------------------------------------
// also nl2 = -LSE log2(e), the exp2 bias of P = exp2(S c - LSE log2 e), read per query by the
// dK / dV passes
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_delta_kernel(const bf16_t* __restrict__ O,
                                                                const bf16_t* __restrict__ dO,
                                                                const float* __restrict__ LSE,
                                                                float* __restrict__ delta, float* __restrict__ nl2,
                                                                long long rows) {
    constexpr int LPR = D / 8;           // lanes per row, 8 bf16 each
    constexpr int RPW = kWave / LPR;     // rows per wave
    const int lane = threadIdx.x & 63;
    const long long row = ((long long)blockIdx.x * (kBwdThreads / kWave) + (threadIdx.x >> 6)) * RPW + lane / LPR;
    const int c = lane % LPR;
    float acc = 0.f;
    if (row < rows) {
        const bf16x8 a = *(const bf16x8*)(O + row * D + 8 * c);
        const bf16x8 b = *(const bf16x8*)(dO + row * D + 8 * c);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = __builtin_fmaf((float)a[j], (float)b[j], acc);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (c == 0 && row < rows) {
        delta[row] = -acc;
        nl2[row] = -LSE[row] * kLog2e;
    }
}

// ------------------------------------------------------------------------------------------
// shared pieces of the two MFMA kernels
// ------------------------------------------------------------------------------------------

template <int V>
using BIC = std::integral_constant<int, V>;

// ------------------------------------------------------------------------------------------
// dQ: parallel over 128-query blocks
// ------------------------------------------------------------------------------------------
// 4 waves (128 queries per workgroup), two workgroups per CU
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kDqWaves, 2) void bwd_dq_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dl,
    bf16_t* __restrict__ dQ, int N, int numQB, float c2 /* scale*log2(e) */, float scale) {
    constexpr int WAVES = kDqWaves;
    using C = TileCfg<D, kBwdRows, WAVES>;
    constexpr int BR = 32 * WAVES;
    constexpr int BC = kBwdRows;
    __shared__ __attribute__((aligned(1024))) uint8_t sK0[C::TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sK1[C::TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sV0[C::TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sV1[C::TB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    int bh, qi;   // causal: heaviest blocks first, across the XCD's heads
    work_item(xcd_remap(blockIdx.x, gridDim.x), gridDim.x, numQB, CAUSAL ? 0 : 1, bh, qi);
    const int qb = CAUSAL ? (numQB - 1 - qi) : qi;
    const int q0 = qb * BR;
    const int q0w = q0 + 32 * wave;
    const int qrow = q0w + col;
    const size_t head = (size_t)bh * N * D;

    const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc((void*)(K + head), (short)0, N * C::ROW, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc((void*)(V + head), (short)0, N * C::ROW, kBufferConfig);
    TileAddr<D, kBwdRows, WAVES> ta;
    ta.init(wave, lane);

    bf16x8 qf[C::KSTEPS], df[C::KSTEPS];
    load_resident<D>(qf, Q + head, qrow, N, h);
    load_resident<D>(df, dO + head, qrow, N, h);
    const float lse2 = qrow < N ? LSE[(size_t)bh * N + qrow] * kLog2e : 0.f;
    const float ndlt = qrow < N ? Dl[(size_t)bh * N + qrow] : 0.f;   // -D of this lane's query

    int nkb = (N + BC - 1) / BC;
    if (CAUSAL) nkb = min(nkb, (min(q0 + BR, N) - 1) / BC + 1);
    // causal: the wave computes only the key blocks its own 32 queries reach (nkb_c) and masks
    // only those that straddle its own diagonal (from nfull on); it loads its share of the
    // workgroup's later blocks, which the other waves need, and takes part in their barriers.
    // Blocks [0, nfull) need no mask for any query of the wave.
    const int nkb_c = CAUSAL ? min(nkb, (min(q0w + 32, N) - 1) / BC + 1) : nkb;
    const int nfull = CAUSAL ? min(N / BC, (q0w + 1) / BC) : N / BC;

    f32x16 acc[C::DT];
#pragma unroll
    for (int e = 0; e < C::DT; ++e) acc[e] = f32x16{};
    const int key8h = 8 * h;

    auto step = [&](int j, auto b_c, auto mask_c) __attribute__((always_inline)) {
        constexpr int B = decltype(b_c)::value;
        constexpr bool MASK = decltype(mask_c)::value != 0;
        const int kb = j * BC;
        if (j + 1 < nkb) {
            ta.load(rK, (B ? sK0 : sK1), kb + BC, wave);
            ta.load(rV, (B ? sV0 : sV1), kb + BC, wave);
        }
        // issue the loads here: left to itself the scheduler sinks them to the end of the step,
        // just before the wait for them
        __builtin_amdgcn_sched_barrier(0);
        // S^T = K Q^T and dP^T = V dO^T (keys x queries)
        // dP^T - D: the product starts from -D (the query's, in every register)
        f32x16 st{}, dpt;
#pragma unroll
        for (int i = 0; i < 16; ++i) dpt[i] = ndlt;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row_operand((B ? sK1 : sK0), s), qf[s], st, 0, 0, 0);
            dpt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row_operand((B ? sV1 : sV0), s), df[s], dpt, 0, 0, 0);
        }
        // register i holds key kb + 16(i/8) + 8h + i%8 of query qrow
        bf16x8 dsf[2];
        const int lim = (CAUSAL ? min(qrow, N - 1) : N - 1) - kb - key8h;   // last visible key offset
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float p = fast_exp2(__builtin_fmaf(st[i], c2, -lse2));
            if constexpr (MASK) p = (16 * (i / 8) + (i % 8)) > lim ? 0.f : p;
            dsf[i / 8][i % 8] = (bf16_t)(p * dpt[i]);
        }
        // dQ^T += K^T dS^T
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int e = 0; e < C::DT; ++e)
                acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.tr_operand((B ? sK1 : sK0), e, ch), dsf[ch], acc[e], 0, 0, 0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    ta.load(rK, sK0, 0, wave);
    ta.load(rV, sV0, 0, wave);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int j = 0;
    for (; j + 1 < nkb_c && j + 1 < nfull; j += 2) {
        step(j, BIC<0>{}, BIC<0>{});
        step(j + 1, BIC<1>{}, BIC<0>{});
    }
    for (; j < nkb_c; j += 2) {
        if (j >= nfull) step(j, BIC<0>{}, BIC<1>{});
        else step(j, BIC<0>{}, BIC<0>{});
        if (j + 1 < nkb_c) step(j + 1, BIC<1>{}, BIC<1>{});
    }
    if constexpr (CAUSAL) {
        // blocks past this wave's queries: loads and barriers only (every wave passes nkb)
        for (int jj = nkb_c; jj < nkb; ++jj) {
            if (jj + 1 < nkb) {
                const bool odd = (jj & 1) != 0;   // block jj + 1 goes to buffer (jj + 1) & 1
                ta.load(rK, odd ? sK0 : sK1, (jj + 1) * BC, wave);
                ta.load(rV, odd ? sV0 : sV1, (jj + 1) * BC, wave);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    // dQ = scale dQ~ (each wave stages its tile in one of the four tile buffers)
    uint8_t* const stg = wave == 0 ? sK0 : wave == 1 ? sK1 : wave == 2 ? sV0 : sV1;
    store_rows<D>(acc, scale, stg, dQ + head, q0w, N, lane);
}

// ------------------------------------------------------------------------------------------
// dK, dV: parallel over 128-key blocks
// ------------------------------------------------------------------------------------------
// Both gradients in one pass, 32 queries per step (d = 64: two waves per SIMD fit both
// accumulators; d = 128 takes the wave-pair kernel below)
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dkdv_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ NL2, const float* __restrict__ Dl,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int N, int numKB, float c2, float scale) {
    static_assert(D <= 64, "both accumulators of a wave fit two waves per SIMD only at d <= 64");
    constexpr int BQ = 32;
    using C = TileCfg<D, BQ>;
    constexpr int BK = 128;
    constexpr int QT = BQ / 32;   // 32-query tiles per step
    __shared__ __attribute__((aligned(1024))) uint8_t sQ0[C::TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sQ1[C::TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sD0[C::TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sD1[C::TB];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    int bh, kbi;   // causal: low key blocks see the most queries and come first (across the XCD's heads)
    work_item(xcd_remap(blockIdx.x, gridDim.x), gridDim.x, numKB, CAUSAL ? 0 : 1, bh, kbi);
    const int k0 = kbi * BK;
    const int k0w = k0 + 32 * wave;
    const int krow = k0w + col;
    const size_t head = (size_t)bh * N * D;

    const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc((void*)(Q + head), (short)0, N * C::ROW, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rO = __builtin_amdgcn_make_buffer_rsrc((void*)(dO + head), (short)0, N * C::ROW, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rL = __builtin_amdgcn_make_buffer_rsrc((void*)(NL2 + (size_t)bh * N), (short)0, N * 4, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rDl = __builtin_amdgcn_make_buffer_rsrc((void*)(Dl + (size_t)bh * N), (short)0, N * 4, kBufferConfig);
    TileAddr<D, BQ> ta;
    ta.init(wave, lane);

    bf16x8 kf[C::KSTEPS], vf[C::KSTEPS];
    load_resident<D>(kf, K + head, krow, N, h);
    load_resident<D>(vf, V + head, krow, N, h);

    const int nqb = (N + BQ - 1) / BQ;
    const int i0 = CAUSAL ? min(k0, N) / BQ : 0;   // queries before the first key see none of it
    f32x16 dk[C::DT], dv[C::DT];
#pragma unroll
    for (int e = 0; e < C::DT; ++e) {
        dk[e] = f32x16{};
        dv[e] = f32x16{};
    }

    // -LSE log2(e) and -D of the queries this lane half holds in query block i: tile tt, rows
    // i BQ + 32 tt + 16u + 8h + 0..7. Loaded one step ahead (rows past N read as zero): the
    // loads for block i + 1 are issued at the start of step i, ahead of its tile loads, and
    // complete by its end, so no step waits for them
    f32x4 lq_n[QT][4], dq_n[QT][4];
    auto load_rows = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int tt = 0; tt < QT; ++tt)
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int v2 = 0; v2 < 2; ++v2) {
                    const int off = 4 * (i * BQ + 32 * tt + 16 * u + 8 * h + 4 * v2);
                    lq_n[tt][2 * u + v2] = __builtin_bit_cast(f32x4, buffer_load16(rL, off));
                    dq_n[tt][2 * u + v2] = __builtin_bit_cast(f32x4, buffer_load16(rDl, off));
                }
    };

    auto step = [&](int i, auto b_c, auto mask_c) __attribute__((always_inline)) {
        constexpr int B = decltype(b_c)::value;
        constexpr bool MASK = decltype(mask_c)::value != 0;
        const int q0 = i * BQ;
        f32x4 lq[QT][4], dq[QT][4];
#pragma unroll
        for (int tt = 0; tt < QT; ++tt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                lq[tt][r] = lq_n[tt][r];
                dq[tt][r] = dq_n[tt][r];
            }
        load_rows(i + 1);
        // the next tiles, issued here (left to itself the scheduler sinks the loads to the end
        // of the step, just before the wait for them)
        __builtin_amdgcn_sched_barrier(0);
        if (i + 1 < nqb) {
            ta.load(rQ, (B ? sQ0 : sQ1), q0 + BQ, wave);
            ta.load(rO, (B ? sD0 : sD1), q0 + BQ, wave);
        }
        __builtin_amdgcn_sched_barrier(0);
        // S = Q K^T and dP = dO V^T (queries x keys), per 32-query tile
        f32x16 s[QT], dp[QT];
#pragma unroll
        for (int tt = 0; tt < QT; ++tt) {
            s[tt] = f32x16{};
            // dP - D: the product starts from -D (register r of query tile tt: dq[tt][r / 4][r % 4])
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[tt][r] = dq[tt][r / 4][r % 4];
#pragma unroll
            for (int st = 0; st < C::KSTEPS; ++st) {
                s[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row_operand((B ? sQ1 : sQ0), st, tt), kf[st], s[tt], 0, 0, 0);
                dp[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row_operand((B ? sD1 : sD0), st, tt), vf[st], dp[tt], 0, 0, 0);
            }
        }
#pragma unroll
        for (int tt = 0; tt < QT; ++tt) {
            // register r holds query q0 + 32 tt + 16(r/8) + 8h + r%8 of key krow
            bf16x8 pf[2], dsf[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float p = fast_exp2(__builtin_fmaf(s[tt][r], c2, lq[tt][r / 4][r % 4]));   // lq: -LSE log2 e
                if constexpr (MASK) {
                    const int q = q0 + 32 * tt + 16 * (r / 8) + 8 * h + (r % 8);
                    p = (q >= N || (CAUSAL && q < krow)) ? 0.f : p;
                }
                pf[r / 8][r % 8] = (bf16_t)p;
                dsf[r / 8][r % 8] = (bf16_t)(p * dp[tt][r]);
            }
            // dV^T += dO^T P, dK^T += Q^T dS over the 32 queries of tile tt
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
#pragma unroll
                for (int e = 0; e < C::DT; ++e) {
                    dv[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.tr_operand((B ? sD1 : sD0), e, 2 * tt + ch), pf[ch], dv[e], 0, 0, 0);
                    dk[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.tr_operand((B ? sQ1 : sQ0), e, 2 * tt + ch), dsf[ch], dk[e], 0, 0, 0);
                }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    if (i0 < nqb) {
        load_rows(i0);
        ta.load(rQ, sQ0, i0 * BQ, wave);
        ta.load(rO, sD0, i0 * BQ, wave);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // query blocks that need a mask: the ones that reach below the last key of the
        // workgroup (causal: a masked prefix) and the ragged last one (a masked tail); the
        // blocks in between run in a loop without branches, so that the accumulators keep
        // their registers (branches between step variants inside the loop make the compiler
        // copy them on every iteration). Block i uses tile slot (i - i0) & 1.
        const int nfree_hi = N / BQ;                                              // full blocks end here
        const int lo = CAUSAL ? min(nqb, (k0 + BK + BQ - 1) / BQ) : i0;   // blocks from here see all keys
        const int hi = max(lo, nfree_hi);
        // causal: query blocks before iw see none of this wave's keys; for the wave they are
        // loads and barriers only (the other waves need the tiles)
        const int iw = CAUSAL ? min(lo, max(i0, k0w / BQ)) : i0;
        for (int i = i0; i < iw; ++i) {
            load_rows(i + 1);
            if (i + 1 < nqb) {
                const bool odd = ((i - i0) & 1) != 0;   // block i + 1 goes to slot (i + 1 - i0) & 1
                ta.load(rQ, odd ? sQ0 : sQ1, (i + 1) * BQ, wave);
                ta.load(rO, odd ? sD0 : sD1, (i + 1) * BQ, wave);
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
        auto run = [&](int a, int b, auto mask_c) __attribute__((always_inline)) {   // blocks [a, b), all masked or all not
            if (a >= b) return;
            if ((a - i0) & 1) step(a++, BIC<1>{}, mask_c);
            for (; a + 1 < b; a += 2) {
                step(a, BIC<0>{}, mask_c);
                step(a + 1, BIC<1>{}, mask_c);
            }
            if (a < b) step(a, BIC<0>{}, mask_c);
        };
        run(iw, lo, BIC<1>{});
        run(lo, hi, BIC<0>{});
        run(hi, nqb, BIC<1>{});
    }

    // dK = scale dK~, dV = dV~; each wave stages its 32-key tile in one of the tile buffers
    uint8_t* const stg = wave == 0 ? sQ0 : wave == 1 ? sQ1 : wave == 2 ? sD0 : sD1;
    store_rows<D>(dk, scale, stg, dK + head, k0w, N, lane);
    store_rows<D>(dv, 1.f, stg, dV + head, k0w, N, lane);
}

// ------------------------------------------------------------------------------------------
// dK, dV with wave pairs
// ------------------------------------------------------------------------------------------
// One 128-key block per workgroup of 8 waves; waves p and p + 4 share the keys k0 + 32p .. +31.
// Wave p (the P wave) keeps K resident; in step i it adds dV^T += dO^T P of block i - 1, then
// computes S = Q K^T and P of block i and leaves P (fp32, the lane layout of S) in LDS, so its
// exponentials overlap its partner's dK products. Wave p + 4 (the dS wave)
// keeps V resident and runs one block behind: dP = dO V^T for block i - 1, dS = P o (dP - D)
// with the P its partner left, dK^T += Q^T dS. Four products per query block (two separate
// dV and dK passes take five), every Q / dO tile is loaded once for both gradients, and each
// wave holds one accumulator, so two waves fit on a SIMD. A tile is in use for three steps
// (being loaded, read by the P waves, read by the dS waves): three slots each for Q, dO and
// each pair's P, block i in slot (i - u) mod 3. The unmasked blocks from u on run unrolled by
// three, so that every LDS address is a per-lane register plus an immediate; the few masked
// blocks (and the first) compute their slot at run time. Masks (causal diagonal, ragged tail) act on P
// only: a masked P is 0, and so is dS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void bwd_dkdv_pair_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ NL2, const float* __restrict__ Dl,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int N, int numKB, float c2, float scale) {
    constexpr int W = 8;
    constexpr int BQ = 32, BK = 128;
    // a 32-row tile is TB / 1 KB load regions: 8 at d = 128 (every wave loads a region of both
    // the Q and the dO tile), 4 at d = 64 (the P waves load the Q tile, the dS waves the dO tile)
    constexpr int LW = TileCfg<D, BQ, 1>::TB / 1024 >= W ? W : W / 2;
    using C = TileCfg<D, BQ, LW>;
    constexpr int TB = C::TB;          // one 32-row tile
    static_assert(C::LOADS == 1, "one load region per wave and tile");
    constexpr int PT = 64 * 16 * 4;    // one P tile: 16 fp32 per lane, stored as 4 planes of 16 B per lane
    // one LDS object per tile slot (three each for Q and dO), so that the compiler can tell
    // that reads of one slot do not touch the DMA writes still in flight into another (with
    // one array it waits for every tile load before each transposing read); and the P tiles
    __shared__ __attribute__((aligned(1024))) uint8_t sQ0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sQ1[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sQ2[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sD0[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sD1[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sD2[TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sP[12 * PT];
    static_assert(6 * TB + 12 * PT >= W * TB && 12 * PT >= (W - 6) * TB, "the output staging reuses the slots");
    auto qslot = [&](int t) __attribute__((always_inline)) { return t == 0 ? sQ0 : t == 1 ? sQ1 : sQ2; };
    auto dslot = [&](int t) __attribute__((always_inline)) { return t == 0 ? sD0 : t == 1 ? sD1 : sD2; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = wave & 3;
    const bool pwave = wave < 4;
    const int h = lane >> 5, col = lane & 31;
    int bh, kbi;   // causal: low key blocks see the most queries and come first (across the XCD's heads)
    work_item(xcd_remap(blockIdx.x, gridDim.x), gridDim.x, numKB, CAUSAL ? 0 : 1, bh, kbi);
    const int k0 = kbi * BK;
    const int k0w = k0 + 32 * pair;
    const int krow = k0w + col;
    const size_t head = (size_t)bh * N * D;

    const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc((void*)(Q + head), (short)0, N * C::ROW, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rO = __builtin_amdgcn_make_buffer_rsrc((void*)(dO + head), (short)0, N * C::ROW, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rL = __builtin_amdgcn_make_buffer_rsrc((void*)(NL2 + (size_t)bh * N), (short)0, N * 4, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rDl = __builtin_amdgcn_make_buffer_rsrc((void*)(Dl + (size_t)bh * N), (short)0, N * 4, kBufferConfig);
    TileAddr<D, BQ, LW> ta;
    const int lwave = LW == W ? wave : (wave & 3);   // this wave's load region
    ta.init(lwave, lane);

    bf16x8 kv[C::KSTEPS];   // K (P wave) or V (dS wave) of the pair's 32 keys
    load_resident<D>(kv, (pwave ? K : V) + head, krow, N, h);
    f32x16 acc[C::DT];      // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
    for (int e = 0; e < C::DT; ++e) acc[e] = f32x16{};

    const int nqb = (N + BQ - 1) / BQ;
    const int i0 = CAUSAL ? min(k0, N) / BQ : 0;   // queries before the first key see none of it
    // blocks [i0, lo) reach below the last key of the workgroup (causal: masked), blocks from
    // lo on see all of its keys; blocks from N / BQ on are ragged (masked)
    const int lo = CAUSAL ? min(nqb, (k0 + BK + BQ - 1) / BQ) : i0;
    const int hi = max(lo, N / BQ);
    const int u = max(lo, i0 + 1);   // first block of the unrolled loops (the first block is peeled)
    // causal: query blocks before ip see none of this pair's keys; for the pair they are
    // loads and barriers only (the other pairs need the tiles)
    const int ip = CAUSAL ? min(nqb, max(i0, k0w / BQ)) : i0;
    uint8_t* const pbuf = sP + 3 * PT * pair;
    auto slot = [&](int i) __attribute__((always_inline)) { return ((i - u) % 3 + 3) % 3; };
    auto load_tiles = [&](int i, int t) __attribute__((always_inline)) {
        if (LW == W || pwave) ta.load(rQ, qslot(t), i * BQ, lwave);
        if (LW == W || !pwave) ta.load(rO, dslot(t), i * BQ, lwave);
    };
    // four values per lane from a per-query fp32 vector: registers 4v .. 4v+3 of tile rows
    // q0 + 16(v/2) + 8h + 4(v%2) + 0..3
    auto row_vals = [&](__amdgpu_buffer_rsrc_t r, int q0, f32x4 (&x)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            x[v] = __builtin_bit_cast(f32x4, buffer_load16(r, 4 * (q0 + 16 * (v / 2) + 8 * h + 4 * (v % 2))));
    };

    // the row values of the wave's next step, loaded one step ahead (see the dK/dV kernel):
    // -LSE log2(e) (P wave) or -D (dS wave)
    f32x4 rv_n[4];

    bf16x8 pf[2];   // P wave: P of the previous block, the B operand of its dV product
    auto dv_update = [&](const uint8_t* td) __attribute__((always_inline)) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int e = 0; e < C::DT; ++e)
                acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.tr_operand(td, e, ch), pf[ch], acc[e], 0, 0, 0);
    };
    // P wave, step i: dV of block i - 1 (unless FIRST), then S and P of query block i in slot
    // SL (-1: computed here); register r of S holds query i BQ + 16(r/8) + 8h + r%8 of key krow
    auto step_p = [&](int i, auto sl_c, auto mask_c, auto first_c) __attribute__((always_inline)) {
        constexpr int SL = decltype(sl_c)::value;
        constexpr bool MASK = decltype(mask_c)::value != 0;
        constexpr bool FIRST = decltype(first_c)::value != 0;
        const int t = SL >= 0 ? SL : slot(i);
        const int q0 = i * BQ;
        // the next step's row values ahead of the tile loads: vector-memory counters retire in
        // order, so a wait for values loaded after the tiles would also wait for the tiles
        f32x4 lq[4];   // -LSE log2(e)
#pragma unroll
        for (int v = 0; v < 4; ++v) lq[v] = rv_n[v];
        row_vals(rL, q0 + BQ, rv_n);
        __builtin_amdgcn_sched_barrier(0);
        // (the unrolled steps, SL >= 0, always have a next block: no branch around the loads)
        if (SL >= 0 || i + 1 < nqb) load_tiles(i + 1, SL >= 0 ? (SL + 1) % 3 : slot(i + 1));
        __builtin_amdgcn_sched_barrier(0);   // and issued early, not sunk to the end of the step
        if constexpr (!FIRST) dv_update(dslot(SL >= 0 ? (SL + 2) % 3 : slot(i - 1)));
        const uint8_t* tq = qslot(t);
        f32x16 sc{};
#pragma unroll
        for (int st = 0; st < C::KSTEPS; ++st)
            sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row_operand(tq, st), kv[st], sc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float p = fast_exp2(__builtin_fmaf(sc[r], c2, lq[r / 4][r % 4]));
            if constexpr (MASK) {
                const int q = q0 + 16 * (r / 8) + 8 * h + (r % 8);
                p = (q >= N || (CAUSAL && q < krow)) ? 0.f : p;
            }
            sc[r] = p;
            pf[r / 8][r % 8] = (bf16_t)p;
        }
        uint8_t* pb = pbuf + PT * t + 16 * lane;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *(f32x4*)(pb + 1024 * j) = f32x4{sc[4 * j], sc[4 * j + 1], sc[4 * j + 2], sc[4 * j + 3]};
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    // dS wave, query block i in slot SL (one step after the P wave's)
    auto step_ds = [&](int i, auto sl_c) __attribute__((always_inline)) {
        constexpr int SL = decltype(sl_c)::value;
        const int t = SL >= 0 ? SL : slot(i);
        const int q0 = i * BQ;
        f32x4 dl[4];   // -D, in the register layout of dP (the next step's loaded as above)
#pragma unroll
        for (int v = 0; v < 4; ++v) dl[v] = rv_n[v];
        row_vals(rDl, q0 + BQ, rv_n);
        __builtin_amdgcn_sched_barrier(0);
        if (SL >= 0 || i + 2 < nqb) load_tiles(i + 2, SL >= 0 ? (SL + 2) % 3 : slot(i + 2));
        __builtin_amdgcn_sched_barrier(0);
        const uint8_t* tq = qslot(t);
        const uint8_t* td = dslot(t);
        // dP - D: the product starts from -D (loaded a step ago)
        f32x16 dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = dl[r / 4][r % 4];
#pragma unroll
        for (int st = 0; st < C::KSTEPS; ++st)
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row_operand(td, st), kv[st], dp, 0, 0, 0);
        const uint8_t* pb = pbuf + PT * t + 16 * lane;
        f32x4 pv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) pv[j] = *(const f32x4*)(pb + 1024 * j);
        bf16x8 dsf[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) dsf[r / 8][r % 8] = (bf16_t)(pv[r / 4][r % 4] * dp[r]);
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int e = 0; e < C::DT; ++e)
                acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.tr_operand(tq, e, ch), dsf[ch], acc[e], 0, 0, 0);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    if (i0 < nqb) {
        // both kinds of wave take part in every tile load and in every barrier: nqb - i0 + 1
        // steps after the first load, the P waves' blocks in steps 0 .. nqb - i0 - 1, the dS
        // waves' in steps 1 .. nqb - i0
        row_vals(pwave ? rL : rDl, i0 * BQ, rv_n);
        load_tiles(i0, slot(i0));
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        // each loop runs without branches between step variants (a branch there makes the
        // compiler copy the accumulators on every iteration)
        int i = i0;
        if (pwave) {
            for (; i < ip; ++i) {   // blocks before the pair's keys
                row_vals(rL, (i + 1) * BQ, rv_n);
                if (i + 1 < nqb) load_tiles(i + 1, slot(i + 1));
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
            if (i < nqb) {
                step_p(i++, BIC<-1>{}, BIC<1>{}, BIC<1>{});
                for (; i < u; ++i) step_p(i, BIC<-1>{}, BIC<1>{}, BIC<0>{});
                for (; i + 3 <= hi; i += 3) {
                    step_p(i, BIC<0>{}, BIC<0>{}, BIC<0>{});
                    step_p(i + 1, BIC<1>{}, BIC<0>{}, BIC<0>{});
                    step_p(i + 2, BIC<2>{}, BIC<0>{}, BIC<0>{});
                }
                // the rest (masking blocks below hi is harmless), then dV of the last block
                for (; i < nqb; ++i) step_p(i, BIC<-1>{}, BIC<1>{}, BIC<0>{});
                dv_update(dslot(slot(nqb - 1)));
            }
            __syncthreads();
        } else {
            if (i0 + 1 < nqb) load_tiles(i0 + 1, slot(i0 + 1));
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            for (; i < ip; ++i) {   // blocks before the pair's keys, one step behind the P wave
                row_vals(rDl, (i + 1) * BQ, rv_n);
                if (i + 2 < nqb) load_tiles(i + 2, slot(i + 2));
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
            }
            for (; i < u; ++i) step_ds(i, BIC<-1>{});
            for (; i + 3 <= nqb; i += 3) {
                step_ds(i, BIC<0>{});
                step_ds(i + 1, BIC<1>{});
                step_ds(i + 2, BIC<2>{});
            }
            for (; i < nqb; ++i) step_ds(i, BIC<-1>{});
        }
    }

    // dV = dV~, dK = scale dK~; each wave stages its 32-key tile in its own 32-row slot
    uint8_t* const stg = wave < 3 ? qslot(wave) : wave < 6 ? dslot(wave - 3) : sP + (wave - 6) * TB;
    store_rows<D>(acc, pwave ? 1.f : scale, stg, (pwave ? dV : dK) + head, k0w, N, lane);
}

// dK and dV: one pass per 128-key block; d = 64 in one wave per 32 keys (a wave pair's 8
// products per step are too few to pay for the per-step barrier of 8 waves and the P
// exchange: 2.89 vs 2.22 ms at B=8 H=16 N=4k), d = 128 in wave pairs
template <int D, bool CAUSAL>
void launch_dkdv(const bf16_t* Qb, const bf16_t* Kb, const bf16_t* Vb, const bf16_t* dOb, const float* nl2,
                 const float* delta, bf16_t* dk, bf16_t* dv, int N, int nb, long long total, float c2, float scale,
                 hipStream_t stream) {
    if constexpr (D > 64) {
        hipLaunchKernelGGL((bwd_dkdv_pair_kernel<D, CAUSAL>), dim3((unsigned)total), dim3(512), 0, stream, Qb, Kb, Vb,
                           dOb, nl2, delta, dk, dv, N, nb, c2, scale);
    } else {
        hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)total), dim3(kBwdThreads), 0, stream, Qb, Kb,
                           Vb, dOb, nl2, delta, dk, dv, N, nb, c2, scale);
    }
}

template <int D>
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, float* delta, int BH, int N, float scale, bool causal,
                      hipStream_t stream) {
    const long long rows = (long long)BH * N;
    {
        constexpr int rows_per_block = (kBwdThreads / kWave) * (kWave / (D / 8));
        const long long blocks = (rows + rows_per_block - 1) / rows_per_block;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)blocks), dim3(kBwdThreads), 0, stream,
                           (const bf16_t*)o, (const bf16_t*)dout, lse, delta, delta + rows, rows);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const float c2 = scale * kLog2e;
    const int nb = (N + 127) / 128;
    const long long total = (long long)BH * nb;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    const bf16_t *Qb = (const bf16_t*)q, *Kb = (const bf16_t*)k, *Vb = (const bf16_t*)v, *dOb = (const bf16_t*)dout;
    constexpr int DQW = kDqWaves;
    const int nbq = (N + 32 * DQW - 1) / (32 * DQW);
    const long long totalq = (long long)BH * nbq;
    if (causal) {
        launch_dkdv<D, true>(Qb, Kb, Vb, dOb, delta + rows, delta, (bf16_t*)dk, (bf16_t*)dv, N, nb, total, c2, scale, stream);
        hipLaunchKernelGGL((bwd_dq_kernel<D, true>), dim3((unsigned)totalq), dim3(64 * DQW), 0, stream, Qb, Kb,
                           Vb, dOb, lse, delta, (bf16_t*)dq, N, nbq, c2, scale);
    } else {
        launch_dkdv<D, false>(Qb, Kb, Vb, dOb, delta + rows, delta, (bf16_t*)dk, (bf16_t*)dv, N, nb, total, c2, scale, stream);
        hipLaunchKernelGGL((bwd_dq_kernel<D, false>), dim3((unsigned)totalq), dim3(64 * DQW), 0, stream, Qb, Kb,
                           Vb, dOb, lse, delta, (bf16_t*)dq, N, nbq, c2, scale);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o, const void* dout,
                           const float* lse, void* dq, void* dk, void* dv, float* delta, int BH, int N, int d,
                           float scale, bool causal, hipStream_t stream) {
    switch (d) {
        case 64: return launch_bwd<64>(q, k, v, o, dout, lse, dq, dk, dv, delta, BH, N, scale, causal, stream);
        case 128: return launch_bwd<128>(q, k, v, o, dout, lse, dq, dk, dv, delta, BH, N, scale, causal, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
