// The fused attention forward kernel shared by the bf16 and the e4m3 (FP8) inputs.
//
// Algorithm: the FA2 loop order ("FlashAttention 2 & 3: Work Partitioning, Warp
// Specialization & FP8", sections "Edit 1" to "Edit 3"): one workgroup owns 128 (or 256)
// queries of one (batch, head) and streams every key/value block of that head through LDS, keeping the
// online-softmax state ("Learn: The Memory Wall & FlashAttention", section 5.1: running max
// m, running sum l, unnormalised accumulator o) in registers; the division by l happens once
// at the end, together with the logsumexp L = m + log l.
//
// CDNA4 mapping:
// - 4 or 8 waves x 32 queries (at d = 256, 8 waves in pairs that split the head dimension).
//   Each wave computes S^T = K_j Q_i^T (keys x queries) on the matrix
//   cores (bf16: v_mfma_f32_32x32x16_bf16; FP8: v_mfma_scale_f32_32x32x64_f8f6f4 with unit
//   MX scales), so the scores of one query sit in one lane (16 per 32-key tile) and its
//   partner lane l^32: row max and row sum are in-register reductions plus one
//   v_permlane32_swap. A wave's queries never interact with another wave's (split-Q).
// - K rows are fed to the MFMA in the order swap_bits23, so the S^T result registers are
//   already the B operand (P^T) of O^T += V_j^T P^T in bf16 (FP8: fp16); P never leaves
//   registers.
// - V^T is read from the row-major 16-bit V tile with ds_read_b64_tr_b16 (8 keys of one d
//   column per lane in two reads).
// - K/V blocks go from HBM straight into LDS (buffer_load ... lds, no staging registers;
//   FP8 V passes through registers to be expanded); rows past N read as zero through the
//   buffer's range check. Tiles are unpadded and
//   XOR-swizzled in 16-byte chunks so that the MFMA operand reads and the transposing V
//   reads are free of bank conflicts.
// - Two-stage software pipeline: while the softmax of block j runs on the vector ALUs, the
//   scores of block j+1 are computed on the matrix cores (the same idea as the
//   intra-warpgroup overlap on the FA2/FA3 pages), then O += P_j V_j. K is double-buffered
//   one block ahead of V; one barrier per block.
// - The accumulator is rescaled only when a row maximum grows by more than 2^TAU (the
//   conditional rescaling of the FA4 section of the memory-wall page). The result stays
//   exact (numerator and denominator use the same reference); P is bounded by 2^TAU.
// - Causal: key blocks entirely above the workgroup's diagonal are never visited; a wave
//   computes only the blocks its own queries reach and masks element by element only the
//   blocks that straddle its own diagonal (it still helps load the workgroup's later blocks).
//   Each head's query blocks are walked heaviest first, and the XCD-aware remap keeps a
//   head's blocks on one XCD (one L2).
//
// FP8 inputs ("FlashAttention-3: How Warp Specialization ...", section 4 "Technique 3";
// "FlashAttention 2 & 3", section "What stays in higher precision"):
// - Q8 and K8 are e4m3 with one fp32 scale per 64 rows; a key block (32 or 64 keys) and a
//   32-query tile each lie inside one scale block, so the score of the block is
//   s_Q s_K (Q8 K8^T) and s_Q s_K is folded into the FMA that subtracts the running max;
// - V stays e4m3 in HBM and is expanded exactly to fp16 when it is written to LDS (every
//   e4m3 value is an fp16 value); its block scale rides on P: P_j is computed as
//   exp2(S ct - m + log2(s_V(j) / max s_V)) in the same FMA (no extra per-element work),
//   the row sum divides the ratio back out once per block, and max s_V is applied with the
//   final division. P is rounded to fp16 (11 significant bits), not e4m3, for the PV product
//   (v_mfma_f32_32x32x16_f16, the bf16 rate): the outliers put values of magnitude up to ~70
//   into V, and with e4m3 P (or bf16 P) one dominant probability's rounding alone moves such
//   an output by more than the 6e-2 budget. For the same reason O is written in fp32.
#pragma once

#include <algorithm>
#include <type_traits>

#include "fa_common.h"

namespace fa {

enum class InKind { BF16, FP8 };

// buffer resource word 3 for raw (untyped) 32-bit-offset buffer loads on gfx950
constexpr int kBufferConfig = 0x00020000;

template <InKind KIND, int D, int BC, int NT>
struct FwdCfg {
    static constexpr bool F8 = KIND == InKind::FP8;
    static constexpr int IN_BYTES = F8 ? 1 : 2;            // bytes per element in HBM
    static constexpr int ROW_BYTES = D * IN_BYTES;          // bytes per K row (HBM and LDS)
    static constexpr int KCPR = ROW_BYTES / 16;             // 16-byte chunks per K row
    static constexpr int VROW_BYTES = D * 2;                // bytes per bf16 V row in LDS
    static constexpr int VCPR = VROW_BYTES / 16;
    static constexpr int QK_K = F8 ? 64 : 16;               // contraction length of one QK MFMA
    static constexpr int KSTEPS = D / QK_K;
    static constexpr int MT = BC / 32;                      // 32-key tiles per block
    static constexpr int DT = D / 32;                       // 32-wide d tiles of O^T
    static constexpr int CH = BC / 16;                      // 16-key chunks of the PV product
    static constexpr int K_BYTES = BC * ROW_BYTES;
    static constexpr int V_BYTES = BC * VROW_BYTES;
    // direct loads per thread; a K tile smaller than one 1 KB region per wave is loaded by its
    // first K_BYTES / 1024 waves, one region each
    static constexpr bool K_PART = K_BYTES < 16 * NT;
    static constexpr int K_LOADS = K_PART ? 1 : K_BYTES / 16 / NT;
    static constexpr int V_LOADS = F8 ? BC * D / 8 / NT : V_BYTES / 16 / NT;   // FP8: 8-byte loads
    static_assert(K_PART ? K_BYTES % 1024 == 0 : K_LOADS * NT * 16 == K_BYTES, "K tile must split evenly");
    static_assert(V_LOADS >= 1, "V tile must split evenly");
    // FP8: a key block lies inside one 64-row scale block of K and V
    static_assert(!F8 || 64 % BC == 0, "FP8 key blocks must divide the 64-row scale blocks");
    static constexpr int KSWZ = (KCPR < 16 ? KCPR : 16) - 1;   // XOR mask of the K swizzle
    static constexpr int VSWZ = VCPR - 1;
};

// swizzled 16-byte chunk position of chunk c in K row r / bf16 V row r. An MFMA operand read
// serves 16 lanes per cycle from the 64 banks (256 bytes) of LDS; those lanes read rows
// swap_bits23(0..15) at one chunk position. Rows of 256 bytes or more: the XOR with
// swap_bits23(r) puts the 16 rows on 16 different chunk positions. Shorter rows (e4m3 at
// d = 128, bf16 at d = 64: 128 bytes; e4m3 at d = 64: 64 bytes) share a 256-byte bank line with
// the RPB - 1 rows next to them, so rows that agree modulo RPB must differ in the XOR:
// r / RPB, distinct over the 16 / RPB rows of each residue.
template <int MASK>
__device__ __forceinline__ int k_slot(int r, int c) {
    constexpr int RPB = 16 / (MASK + 1);   // rows per 256-byte bank line (MASK + 1 chunks per row)
    if constexpr (RPB > 1) return c ^ ((r / RPB) & MASK);
    return c ^ (swap_bits23(r) & MASK);
}
template <int MASK>
__device__ __forceinline__ int v_slot(int r, int c) { return c ^ ((2 * (r & 3) ^ 8 * (r & 1)) & MASK); }

template <InKind KIND>
struct QOperand;
template <>
struct QOperand<InKind::BF16> { typedef bf16x8 type; };
template <>
struct QOperand<InKind::FP8> { typedef i32x8 type; };

template <int V>
using IC = std::integral_constant<int, V>;

// Extended problems (EXT kernels): grouped key/value heads, a sliding window and packed
// variable-length sequences. A workgroup's (batch or sequence, head) index is seq Hq + h; query
// head h reads key/value head h / g. Window: query i sees key j iff i - left <= j <= i + right
// (a negative bound: no limit; the causal mask sets right = 0). With cu (cu[s], cu[s+1] the
// token range of sequence s; the batch dimension is then 1) positions count from the start of
// the sequence and keys of other sequences are never visited. ntot: tokens per (batch, head)
// row of the tensors (N, or the total of the packed sequences); nseq: the number of packed
// sequences (with cu).
struct FwdExt {
    int Hq, g, left, right, ntot;
    const int* cu;
    int nseq;
};

// Query blocks of packed sequence s: ceil(rows / BR), at most numQB (the grid's longest
// sequence); offsets clamped to [0, ntot] as where the kernel reads them.
template <int BR>
__device__ __forceinline__ int packed_blocks(const int* cu, int s, int ntot, int numQB) {
    const int a = min(max(cu[s], 0), ntot);
    const int n = min(max(cu[s + 1], a), ntot) - a;
    return min((n + BR - 1) / BR, numQB);
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

// index of the k-th set bit (k < popcount(m)) of a wave-uniform 64-bit mask
__device__ __forceinline__ int kth_set_bit(uint64_t m, int k, int lane) {
    const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    return __ffsll((long long)__builtin_amdgcn_ballot_w64(((m >> lane) & 1) != 0 && rank == k)) - 1;
}

// Packed sequences: the grid enumerates only query blocks that exist (a grid of every sequence
// times the longest one's blocks leaves most workgroups empty, and the hardware's dispatch order
// then places the live ones on a fraction of the CUs). Work item r is block rank r / Hq, head
// r % Hq; blocks are ranked by block index, highest first (for the causal mask the costliest
// ones), then by sequence. Every lane takes part; the results are wave-uniform. Returns false
// past the last block.
template <int BR>
__device__ bool packed_item(const FwdExt& ext, int numQB, int r, int lane, int& seq, int& hq, int& qb) {
    const int rb = r / ext.Hq;
    hq = r - rb * ext.Hq;
    if (ext.nseq <= kWave) {
        // one sequence per lane: walk the block levels down from the top, counting the
        // sequences that have a block at each level (a ballot per level)
        const int nb = lane < ext.nseq ? packed_blocks<BR>(ext.cu, lane, ext.ntot, numQB) : 0;
        int above = 0;   // blocks ranked before level l
        for (int l = numQB - 1; l >= 0; --l) {
            const uint64_t m = __builtin_amdgcn_ballot_w64(nb > l);
            const int c = __popcll(m);
            if (rb < above + c) {
                qb = l;
                seq = kth_set_bit(m, rb - above, lane);
                return true;
            }
            above += c;
        }
        return false;
    }
    // any number of sequences: blocks with an index above level l are
    // sum over s of max(0, blocks(s) - l - 1); binary search for the level
    auto above = [&](int l) {
        int c = 0;
        for (int s = lane; s < ext.nseq; s += kWave) c += max(0, packed_blocks<BR>(ext.cu, s, ext.ntot, numQB) - l - 1);
        return wave_sum(c);
    };
    if (rb >= above(-1)) return false;
    // the lowest level l with above(l) <= rb (above is non-increasing, above(numQB - 1) = 0)
    int lo = 0, hi = numQB - 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (above(mid) <= rb) hi = mid; else lo = mid + 1;
    }
    qb = lo;
    // the k-th sequence (in order) that has block qb
    int k = rb - above(qb);
    for (int base = 0; base < ext.nseq; base += kWave) {
        const int s = base + lane;
        const uint64_t m = __builtin_amdgcn_ballot_w64(s < ext.nseq && packed_blocks<BR>(ext.cu, s, ext.ntot, numQB) > qb);
        const int c = __popcll(m);
        if (k < c) {
            seq = base + kth_set_bit(m, k, lane);
            return true;
        }
        k -= c;
    }
    return false;   // not reached for consistent counts
}

// WAVES: waves per workgroup (each owns 32 NQ queries; all share the K/V tiles).
// NQ: 32-query tiles per wave (the workgroup owns WAVES * 32 * NQ queries). With NQ = 2 every K
// and V^T operand read from LDS feeds two MFMAs, which halves the LDS traffic per FLOP.
// PIPE: compute the scores of block j+1 while the softmax of block j runs (needs registers
// for two score tiles); without it each block's scores are computed just before its softmax.
// DSPLIT = 2: the head dimension is split over a pair of waves (waves 2w and 2w+1 own the same
// 32 NQ queries). Each wave holds Q and the O accumulator for its half of d, computes its
// half of the score contraction, and the two partial score tiles are exchanged through LDS at
// the block barrier and added (fp32 addition commutes, so both waves see bit-identical scores
// and take identical softmax decisions); each wave then accumulates its half of O. At
// d = 256 this keeps a wave's registers at the d = 128 footprint, where a whole-d wave needs
// more than the 256 VGPRs and the compiler copies the accumulator between register files.
template <InKind KIND, int D, int BC, int NQ, bool CAUSAL, int TAU, int MINB, bool PIPE, int WAVES, bool EXT = false,
          int DSPLIT = 1>
__global__ __launch_bounds__(64 * WAVES, MINB) void fwd_kernel(
    const void* __restrict__ Qv, const void* __restrict__ Kv, const void* __restrict__ Vv,
    const float* __restrict__ SQ, const float* __restrict__ SK, const float* __restrict__ SV,
    void* __restrict__ Ov, float* __restrict__ LSE, int N, int numQB, int nsb, float c2 /* scale*log2(e) */,
    int hgroup, FwdExt ext) {
    static_assert(!(EXT && KIND == InKind::FP8), "extended problems take bf16 inputs");
    constexpr int NT = 64 * WAVES;    // threads per workgroup
    using C = FwdCfg<KIND, D, BC, NT>;
    using QT = typename QOperand<KIND>::type;
    // operands of the PV product: bf16 P and V, or (FP8 inputs) fp16 P and V
    using PT = typename std::conditional<C::F8, f16x8, bf16x8>::type;
    using PE = typename std::conditional<C::F8, _Float16, bf16_t>::type;
    constexpr float tau = (float)TAU;
    static_assert(DSPLIT == 1 || (DSPLIT == 2 && PIPE && WAVES % 2 == 0), "d split: pipelined, wave pairs");
    constexpr int BR = WAVES / DSPLIT * 32 * NQ;   // queries per workgroup
    constexpr int KST = C::KSTEPS / DSPLIT;        // QK steps of one wave
    constexpr int DTW = C::DT / DSPLIT;            // 32-wide d tiles of O^T of one wave
    constexpr int XB = C::MT * NQ * 4096;          // bytes of one wave's partial score tiles
    // separate objects per buffer, so that the compiler can tell that LDS reads of one
    // buffer do not depend on the DMA writes still in flight into the other one
    __shared__ __attribute__((aligned(1024))) uint8_t smK0[C::K_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t smK1[C::K_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t smV0[C::V_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t smV1[C::V_BYTES];
    // d split: partial score tiles of block parity 0 / 1, one XB region per wave
    __shared__ __attribute__((aligned(1024))) uint8_t smX0[DSPLIT > 1 ? WAVES * XB : 16];
    __shared__ __attribute__((aligned(1024))) uint8_t smX1[DSPLIT > 1 ? WAVES * XB : 16];
    uint8_t* const smK[2] = {smK0, smK1};
    uint8_t* const smV[2] = {smV0, smV1};

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, kept in an SGPR
    const int qwave = wave / DSPLIT;   // the wave's query tile(s)
    const int hd = wave % DSPLIT;      // the wave's part of the head dimension
    const int h = lane >> 5;        // lane half
    const int col = lane & 31;      // query column owned by this lane in each query tile

    int bh, qi;
    if (EXT && ext.cu != nullptr) {
        // packed sequences of unequal lengths: the costliest blocks of every sequence and head
        // are dispatched first and spread over all XCDs (the contiguous per-XCD ranges of the
        // remap would put a long sequence on one or two XCDs)
        int seq, hq, qbk;
        if (!packed_item<BR>(ext, numQB, blockIdx.x, lane, seq, hq, qbk)) return;
        bh = __builtin_amdgcn_readfirstlane(seq * ext.Hq + hq);
        qbk = __builtin_amdgcn_readfirstlane(qbk);
        qi = CAUSAL ? numQB - 1 - qbk : qbk;
    } else {
        // causal: each XCD's heads in groups of hgroup (launch_fwd_kernel), each group ordered
        // by query block first (costliest blocks first)
        work_item(xcd_remap(blockIdx.x, gridDim.x), gridDim.x, numQB, CAUSAL ? hgroup : 1, bh, qi);
    }
    const int qb = CAUSAL ? (numQB - 1 - qi) : qi;
    const int q0 = qb * BR;
    const int q0w = q0 + qwave * 32 * NQ;
    int qrow[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) qrow[n] = q0w + 32 * n + col;

    // rows of this head (sequence) and the row index of its row 0 in Q / O / LSE and in K / V
    size_t qbase = (size_t)bh * N, kvbase = (size_t)bh * N;
    if constexpr (EXT) {
        const int seq = bh / ext.Hq;
        const int hq = bh - seq * ext.Hq;
        int start = 0;
        if (ext.cu != nullptr) {   // offsets clamped to [0, ntot]: never a read outside the tensors
            start = min(max(ext.cu[seq], 0), ext.ntot);
            N = min(max(ext.cu[seq + 1], start), ext.ntot) - start;
        }
        const int bb = ext.cu != nullptr ? 0 : seq;
        qbase = ((size_t)bb * ext.Hq + hq) * ext.ntot + start;
        kvbase = ((size_t)bb * (ext.Hq / ext.g) + hq / ext.g) * ext.ntot + start;
        if (q0 >= N) return;   // the grid covers the longest sequence (uniform per workgroup)
    }
    const size_t head_off = qbase * D;   // elements
    const uint8_t* Qh = (const uint8_t*)Qv + head_off * C::IN_BYTES;
    const uint8_t* Kh = (const uint8_t*)Kv + kvbase * D * C::IN_BYTES;
    const uint8_t* Vh = (const uint8_t*)Vv + kvbase * D * C::IN_BYTES;
    // buffer resources over this head's K and V: reads past row N return zero
    const __amdgpu_buffer_rsrc_t rK =
        __builtin_amdgcn_make_buffer_rsrc((void*)Kh, (short)0, N * C::ROW_BYTES, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rV =
        __builtin_amdgcn_make_buffer_rsrc((void*)Vh, (short)0, N * C::ROW_BYTES, kBufferConfig);

    const int nkb_all = (N + BC - 1) / BC;
    int nkb = nkb_all;
    if (CAUSAL) nkb = min(nkb_all, (min(q0 + BR, N) - 1) / BC + 1);
    // EXT: key blocks [jlo, nkb) reach the window of some query of the workgroup; blocks
    // below jfree reach below some query's window (masked)
    int jlo = 0, jfree = 0;
    const int right = CAUSAL ? 0 : (EXT ? ext.right : -1);
    if constexpr (EXT) {
        const int qlast = min(q0 + BR, N) - 1;
        if (right >= 0) nkb = min(nkb_all, (qlast + right) / BC + 1);
        if (ext.left >= 0) {
            jlo = max(0, q0 - ext.left) / BC;
            jfree = max(0, qlast - ext.left + BC - 1) / BC;
        }
    }

    // score scale (log2 units); FP8 adds the Q block scale of each query tile
    float cq[NQ];
    float svmax = 1.f;   // FP8: largest V block scale of this head
    float l2svmax = 0.f;  // and its log2
#pragma unroll
    for (int n = 0; n < NQ; ++n) cq[n] = c2;
    if constexpr (C::F8) {
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int qt0 = q0w + 32 * n;
            cq[n] *= (qt0 < N) ? SQ[(size_t)bh * nsb + qt0 / 64] : 1.f;
        }
        float mx = 0.f;
        for (int i = lane; i < nsb; i += kWave) mx = fmaxf(mx, SV[(size_t)bh * nsb + i]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m));
        svmax = mx;
        l2svmax = __log2f(mx);
    }

    // ---- Q^T operands (B of S^T = K Q^T): in tile n the lane holds query qrow[n]; step s
    // covers head-dim elements [QK_K s + (QK_K/2) h, +QK_K/2)
    QT qf[NQ][KST];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
        const bool ok = qrow[n] < N;
        const uint8_t* qp = Qh + (size_t)(ok ? qrow[n] : 0) * C::ROW_BYTES + (C::QK_K / 2) * C::IN_BYTES * h +
                            hd * KST * C::QK_K * C::IN_BYTES;
#pragma unroll
        for (int s = 0; s < KST; ++s) {
            const uint8_t* p = qp + s * C::QK_K * C::IN_BYTES;
            if constexpr (C::F8) {
                const i32x4 lo = ok ? *(const i32x4*)p : i32x4{};
                const i32x4 hi = ok ? *(const i32x4*)(p + 16) : i32x4{};
                qf[n][s] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            } else {
                qf[n][s] = ok ? *(const bf16x8*)p : bf16x8{};
            }
        }
    }

    // ---- per-thread source offsets of the direct-to-LDS tile loads. One load instruction of
    // a wave fills one 1 KB region of the tile (RPL rows); load i of wave w fills region
    // w + 4 i: lane L writes row RPL (w + 4 i) + L / CPR, swizzled slot L % CPR, so it fetches
    // source chunk slot ^ f(row). The rows of one thread's loads are 4 RPL apart; when that is
    // a multiple of the swizzle period (16 rows for K, 4 for V) every load of the thread has
    // the same swizzle, and its offsets are one register plus constants (fewer live VGPRs).
    constexpr int KRPL = 1024 / C::ROW_BYTES;
    constexpr bool KUNI = (WAVES * KRPL) % 16 == 0;
    constexpr int KN = KUNI ? 1 : C::K_LOADS;
    int koff[KN];
#pragma unroll
    for (int i = 0; i < KN; ++i) {
        const int r = KRPL * (wave + WAVES * i) + lane / C::KCPR;
        koff[i] = r * C::ROW_BYTES + 16 * k_slot<C::KSWZ>(r, lane % C::KCPR);
    }
    auto koff_of = [&](int i) { return KUNI ? koff[0] + WAVES * KRPL * C::ROW_BYTES * i : koff[i]; };
    constexpr int VRPL = 1024 / C::VROW_BYTES;
    int voff0;
    if constexpr (C::F8) {
        // register-staged: load i of a thread reads the 8 e4m3 values x = tid + NT i of the
        // tile (row x / (D/8), fp16 chunk x % (D/8) once expanded); NT is a multiple of D/8, so
        // rows of successive loads are NT / (D/8) apart. 16 consecutive lanes then write 16
        // consecutive fp16 chunks of one row (or two 128-byte rows), all 64 banks once.
        voff0 = (tid / (D / 8)) * C::ROW_BYTES + 8 * (tid % (D / 8));
    } else {
        const int r = VRPL * wave + lane / C::VCPR;
        voff0 = r * C::ROW_BYTES + 16 * v_slot<C::VSWZ>(r, lane % C::VCPR);
    }
    auto voff_of = [&](int i) {
        if constexpr (C::F8) return voff0 + (NT / (D / 8)) * C::ROW_BYTES * i;
        return voff0 + WAVES * VRPL * C::ROW_BYTES * i;   // rows WAVES VRPL apart keep the V swizzle
    };
    auto load_k = [&](int kb, uint8_t* dst) {
        if constexpr (C::K_PART) {
            if (wave < C::K_BYTES / 1024) lds_dma16(rK, dst + 1024 * wave, koff_of(0) + kb * C::ROW_BYTES);
        } else {
#pragma unroll
            for (int i = 0; i < C::K_LOADS; ++i)
                lds_dma16(rK, dst + 1024 * (wave + WAVES * i), koff_of(i) + kb * C::ROW_BYTES);
        }
    };
    i32x2 vst[C::F8 ? C::V_LOADS : 1];   // FP8 V staging
    auto load_v = [&](int kb, uint8_t* dst) {
#pragma unroll
        for (int i = 0; i < C::V_LOADS; ++i) {
            if constexpr (C::F8)
                vst[i] = buffer_load8(rV, voff_of(i) + kb * C::ROW_BYTES);
            else
                lds_dma16(rV, dst + 1024 * (wave + WAVES * i), voff_of(i) + kb * C::ROW_BYTES);
        }
    };
    // FP8: expand the staged e4m3 V chunks exactly to fp16 and store them swizzled
    auto store_v = [&](uint8_t* dst) {
        if constexpr (C::F8) {
#pragma unroll
            for (int i = 0; i < C::V_LOADS; ++i) {
                const int x = tid + NT * i;
                const int r = x / (D / 8);
                const int c = x % (D / 8);   // 8 e4m3 values = fp16 chunk c
                i32x4 w;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    w[2 * u] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vst[i][u], 1.f, false));
                    w[2 * u + 1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vst[i][u], 1.f, true));
                }
                *(i32x4*)(dst + r * C::VROW_BYTES + 16 * v_slot<C::VSWZ>(r, c)) = w;
            }
        }
    };

    // ---- per-lane LDS read addresses (relative to a tile buffer). The swizzles only touch
    // the low 4 bits of a chunk index, so chunks 16 apart keep a fixed 256-byte distance and
    // only the first 16 chunks of a row need a per-lane address.
    // K operand of QK step s, 32-key tile t: row 32t + swap_bits23(col), chunk c(s, h)
    constexpr int KREADS = C::F8 ? 2 : 1;              // 16-byte reads per operand
    constexpr int KSPAN = C::F8 ? 4 : 8;               // steps per 16 chunks
    constexpr int KA = KST < KSPAN ? KST : KSPAN;
    // d split: a wave's steps are whole spans (bf16 d = 256) or a part of one span (e4m3
    // d = 256: two of its four steps)
    static_assert(DSPLIT == 1 || ((KST % KSPAN == 0 || KSPAN % KST == 0) && DTW % 4 == 0),
                  "d split: whole 16-chunk spans, or whole parts of one, per wave");
    const int khd = 256 * (hd * KST / KSPAN);   // the wave's first K chunk span
    const int vhd = 256 * (hd * DTW / 4);       // and first V^T chunk span
    int kaddr[KA][KREADS];
    {
        const int rr = swap_bits23(col);   // same swizzle for rows rr and 32t + rr
#pragma unroll
        for (int s = 0; s < KA; ++s)
#pragma unroll
            for (int u = 0; u < KREADS; ++u) {
                const int w = (hd * KST + s) % KSPAN;   // the step's place in its span
                const int c = C::F8 ? 4 * w + 2 * h + u : 2 * w + h;
                kaddr[s][u] = rr * C::ROW_BYTES + 16 * k_slot<C::KSWZ>(rr, c);
            }
    }
    // V^T operand of PV chunk ch, d tile e: rows 16ch + 8(g>>1) + (L>>2) (+4), the 8 bytes
    // of columns 32e + 16(g&1) + 4(L&3) .. +3. The swizzle depends on row & 3 = (L>>2) only.
    constexpr int VA = C::DT < 4 ? C::DT : 4;          // 4 d tiles = 16 chunks
    int vaddr[VA];
    {
        const int g = lane >> 4, L = lane & 15;
        const int vr = 8 * (g >> 1) + (L >> 2);
#pragma unroll
        for (int e = 0; e < VA; ++e) {
            const int byte = 64 * e + 32 * (g & 1) + 8 * (L & 3);
            vaddr[e] = vr * C::VROW_BYTES + 16 * v_slot<C::VSWZ>(vr, byte / 16) + (byte & 15);
        }
    }

    // ---- state. The running max starts at a finite sentinel instead of -inf, so that the
    // rescale factor exp2(m_old - m_new) and the softmax bias need no special cases: a row
    // that has seen no key yet has l = 0, and masked scores are -inf whatever the bias.
    constexpr float kNoMax = -1e30f;
    f32x16 acc[NQ][DTW];
    float m_run[NQ], l_run[NQ], m_blk[NQ];   // reference max, row sum, max of the next block
    bool grow[NQ];
#pragma unroll
    for (int n = 0; n < NQ; ++n) {
#pragma unroll
        for (int e = 0; e < DTW; ++e) acc[n][e] = f32x16{};
        m_run[n] = kNoMax;
        l_run[n] = 0.f;
        m_blk[n] = kNoMax;
        grow[n] = false;
    }
    // result register i = 4a + b of a 32-key tile holds key swap_bits23(8a + 4h + b)
    //                                                     = 16(a>>1) + 4(a&1) + b + 8h
    const int key8h = 8 * h;
    f32x16 s_buf[PIPE ? 2 : 1][C::MT][NQ];   // scores of blocks j (index j&1) and j+1

    auto qk = [&](const uint8_t* kt, f32x16 (*st)[NQ]) {
#pragma unroll
        for (int t = 0; t < C::MT; ++t)
#pragma unroll
            for (int n = 0; n < NQ; ++n) st[t][n] = f32x16{};
#pragma unroll
        for (int s = 0; s < KST; ++s)
#pragma unroll
            for (int t = 0; t < C::MT; ++t) {
                const uint8_t* p = kt + 32 * t * C::ROW_BYTES + khd + 256 * (s / KSPAN);
                if constexpr (C::F8) {
                    const i32x4 lo = *(const i32x4*)(p + kaddr[s % KSPAN][0]);
                    const i32x4 hi = *(const i32x4*)(p + kaddr[s % KSPAN][KREADS - 1]);
                    const i32x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                    for (int n = 0; n < NQ; ++n)
                        st[t][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[n][s], st[t][n], 0, 0, 0,
                                                                                    127, 0, 127);
                } else {
                    const bf16x8 a = *(const bf16x8*)(p + kaddr[s % KSPAN][0]);
#pragma unroll
                    for (int n = 0; n < NQ; ++n)
                        st[t][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[n][s], st[t][n], 0, 0, 0);
                }
            }
    };
    // d split: publish this wave's partial scores of a block (parity X), and add the partner
    // wave's. Lane l stores its 16 values of a tile as four 16-byte chunks, chunk k of all
    // lanes forming one contiguous 1 KB row (conflict-free); the partner's lane l holds the
    // same (key, query) positions.
    auto x_put = [&](f32x16 (*st)[NQ], auto x_c) {
        uint8_t* xb = (decltype(x_c)::value ? smX1 : smX0) + wave * XB + 16 * lane;
#pragma unroll
        for (int t = 0; t < C::MT; ++t)
#pragma unroll
            for (int n = 0; n < NQ; ++n)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    *(f32x4*)(xb + ((t * NQ + n) * 4 + k) * 1024) =
                        f32x4{st[t][n][4 * k], st[t][n][4 * k + 1], st[t][n][4 * k + 2], st[t][n][4 * k + 3]};
    };
    auto x_add = [&](f32x16 (*st)[NQ], auto x_c) {
        const uint8_t* xb = (decltype(x_c)::value ? smX1 : smX0) + (wave ^ 1) * XB + 16 * lane;
#pragma unroll
        for (int t = 0; t < C::MT; ++t)
#pragma unroll
            for (int n = 0; n < NQ; ++n)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const f32x4 o = *(const f32x4*)(xb + ((t * NQ + n) * 4 + k) * 1024);
#pragma unroll
                    for (int u = 0; u < 4; ++u) st[t][n][4 * k + u] += o[u];
                }
    };
    // hide keys past N and, for the causal mask, keys after the query. Called only for
    // blocks that need it (the diagonal blocks and the ragged last block), unconditionally.
    // Key kb + 8h + off is visible to query qrow iff off <= lim = (last visible key) - kb - 8h,
    // with off a compile-time constant per register: one threshold per lane and block.
    auto mask = [&](f32x16 (*st)[NQ], int kb) {
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const int lim = (right >= 0 ? min(qrow[n] + right, N - 1) : N - 1) - kb - key8h;
            // EXT window: keys before qrow - left are hidden too
            const int low = (EXT && ext.left >= 0) ? qrow[n] - ext.left - kb - key8h : -(1 << 30);
#pragma unroll
            for (int t = 0; t < C::MT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int off = 32 * t + 16 * ((i >> 2) >> 1) + 4 * ((i >> 2) & 1) + (i & 3);
                    if constexpr (EXT) st[t][n][i] = (off > lim || off < low) ? -INFINITY : st[t][n][i];
                    else st[t][n][i] = off > lim ? -INFINITY : st[t][n][i];
                }
        }
    };
    // blocks [jfree, nfull) need no mask for any query of the workgroup
    int nfull;
    if (right >= 0) nfull = min(N / BC, (q0 + right + 1) / BC);
    else nfull = N / BC;
    // causal or a window's right edge: each wave computes only the key blocks its own queries
    // reach (nkb_c) and masks only the ones that cross its own right edge (from nfull on); it
    // still loads its share of the workgroup's later blocks, which the other waves need, and
    // takes part in their barriers
    constexpr bool PER_WAVE = CAUSAL || EXT;
    int nkb_c = nkb;
    if constexpr (PER_WAVE) {
        if (right >= 0) {
            nkb_c = min(nkb, (min(q0w + 32 * NQ, N) - 1 + right) / BC + 1);
            nfull = min(N / BC, (q0w + right + 1) / BC);
        }
    }
    auto needmask = [&](int x) { return x >= nfull || (EXT && x < jfree); };
    auto kscale = [&](int jj) {
        if constexpr (C::F8) return SK[(size_t)bh * nsb + jj * BC / 64];
        return 1.f;
    };
    // row max of block jj (log2 units) and whether it moves the reference max, which happens
    // only when it exceeds the reference by more than TAU (then it becomes the new reference)
    auto row_max = [&](f32x16 (*st)[NQ], int jj) {
        const float ks = kscale(jj);
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < C::MT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[t][n][i]);
            m_blk[n] = pair_max(mx) * (cq[n] * ks);
            grow[n] = m_blk[n] > m_run[n] + tau;
        }
    };

    // one key block j (buffer parity B). With the pipeline one branch-free region holds
    // [P_j on the VALU | scores of block j+1 on the matrix cores], [O += P_j V_j on the matrix
    // cores | mask and row max of block j+1 on the VALU]. MASKN: block j+1 needs the mask.
    auto step = [&](int j, auto b_c, auto next_c, auto maskn_c) {
        constexpr int B = decltype(b_c)::value;
        constexpr bool NEXT = decltype(next_c)::value != 0;
        constexpr bool MASKN = decltype(maskn_c)::value != 0;
        auto s_cur = s_buf[PIPE ? B : 0];
        auto s_nxt = s_buf[PIPE ? (B ^ 1) : 0];
        const int kb = j * BC;
        // issue the loads of the next blocks: K_{j+2} into K_j's buffer (K_{j+1} without the
        // pipeline) and V_{j+1}
        if constexpr (PIPE) {
            if (j + 2 < nkb) load_k(kb + 2 * BC, smK[B]);
        } else {
            if (NEXT || (PER_WAVE && j + 1 < nkb)) load_k(kb + BC, smK[B ^ 1]);
        }
        // (per-wave causal: the workgroup may need block j+1 when this wave is done)
        if (NEXT || (PER_WAVE && j + 1 < nkb)) load_v(kb + BC, smV[B ^ 1]);
        if constexpr (!PIPE) {
            qk(smK[B], s_cur);
            if (needmask(j)) mask(s_cur, kb);
            row_max(s_cur, j);
        }
        if constexpr (DSPLIT > 1) {
            // the partner's half of block j's scores was published before the last barrier
            x_add(s_cur, b_c);
            if (needmask(j)) mask(s_cur, kb);
            row_max(s_cur, j);
        }
        // ---- move the reference max to block j's max where it grew past TAU, rescaling the row
        // sum and the accumulator by alpha = exp2(m_old - m_new) (rare with TAU > 0; elsewhere
        // alpha would be exactly 1, so the whole update is skipped)
        bool any_grow = false;
#pragma unroll
        for (int n = 0; n < NQ; ++n) any_grow = any_grow || grow[n];
        if (wave_any(any_grow)) {
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
                const float m_ref = grow[n] ? m_blk[n] : m_run[n];
                const float alpha = fast_exp2(m_run[n] - m_ref);
                m_run[n] = m_ref;
                l_run[n] *= alpha;
#pragma unroll
                for (int e = 0; e < DTW; ++e)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[n][e][i] *= alpha;
            }
        }
        // ---- P_j = exp2(S_j ct - m) (FP8: times s_V(j) / max s_V)
        float lbias = 0.f;
        float inv_r = 1.f;
        if constexpr (C::F8) {
            const float sv = SV[(size_t)bh * nsb + j * BC / 64];
            // log2(s_V(j) / max s_V) and its inverse ratio without divisions (the block's P
            // carries the ratio, the row sum divides it back out; both to within an ulp or two)
            lbias = __log2f(sv) - l2svmax;
            inv_r = svmax * __builtin_amdgcn_rcpf(sv);
        }
        const float ks = kscale(j);
        // causal: the wave's last block holds its diagonal. The first rows of a head see only a
        // few keys there, and rounding P to bf16 would cost up to 2^-9 of the largest value's
        // magnitude; there P is carried as P_hi + P_lo (two bf16 terms, 2^-17 relative) and the
        // block takes two PV products.
        constexpr bool SPLITP = CAUSAL && !NEXT && !C::F8;
        PT pf[NQ][C::CH];
        bf16x8 plo[SPLITP ? NQ : 1][SPLITP ? C::CH : 1];
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const float ct = cq[n] * ks;
            // (-m, not 0 - m, for bf16: the negation then rides on the FMA as a modifier)
            const float bias = C::F8 ? lbias - m_run[n] : -m_run[n];
            float lsum;
#pragma unroll
            for (int t = 0; t < C::MT; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(__builtin_fmaf(s_cur[t][n][i], ct, bias));
                    // fp32 P: the logsumexp needs the unrounded sum (started at the first term,
                    // not at 0, which would cost an add)
                    lsum = (t == 0 && i == 0) ? p : lsum + p;
                    const PE ph = (PE)p;
                    pf[n][2 * t + i / 8][i % 8] = ph;
                    if constexpr (SPLITP) plo[n][2 * t + i / 8][i % 8] = (bf16_t)(p - (float)ph);   // p - ph is exact
                }
            if constexpr (C::F8) lsum *= inv_r;
            l_run[n] += lsum;
        }
        // ---- scores of block j+1
        if constexpr (PIPE && NEXT) qk(smK[B ^ 1], s_nxt);
        if constexpr (DSPLIT > 1 && NEXT) x_put(s_nxt, IC<B ^ 1>{});
        // ---- O^T += V_j^T P_j^T
        const uint8_t* vt = smV[B];
#pragma unroll
        for (int ch = 0; ch < C::CH; ++ch)
#pragma unroll
            for (int e = 0; e < DTW; ++e) {
                const uint8_t* vp = vt + 16 * ch * C::VROW_BYTES + vhd + 256 * (e / 4) + vaddr[e % 4];
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(FA_LDS(bf16x4, vp));
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(FA_LDS(bf16x4, vp + 4 * C::VROW_BYTES));
                // concatenated as whole vectors (element-wise assembly is mis-compiled); the
                // transposing read moves 16-bit elements, so FP8's fp16 V is read the same way
                const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int n = 0; n < NQ; ++n) {
                    if constexpr (C::F8) {
                        acc[n][e] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), pf[n][ch],
                                                                          acc[n][e], 0, 0, 0);
                    } else {
                        acc[n][e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[n][ch], acc[n][e], 0, 0, 0);
                        if constexpr (SPLITP)
                            acc[n][e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, plo[n][ch], acc[n][e], 0, 0, 0);
                    }
                }
            }
        // ---- mask and row max of block j+1 (d split: at the start of step j+1, after the exchange)
        if constexpr (PIPE && NEXT && DSPLIT == 1) {
            if constexpr (MASKN) mask(s_nxt, kb + BC);
            row_max(s_nxt, j + 1);
        }
        if constexpr (C::F8) {
            if (NEXT || (PER_WAVE && j + 1 < nkb)) store_v(smV[B ^ 1]);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };

    // ---- prologue: K_jlo, V_jlo (and K_jlo+1, the scores and row max of block jlo with the
    // pipeline); jlo = 0 except for windows
    const int kb0 = jlo * BC;
    load_k(kb0, smK[0]);
    load_v(kb0, smV[0]);
    if (PIPE && nkb > jlo + 1) load_k(kb0 + BC, smK[1]);
    __builtin_amdgcn_s_waitcnt(0);
    store_v(smV[0]);
    __syncthreads();
    if constexpr (PIPE) {
        qk(smK[0], s_buf[0]);
        if constexpr (DSPLIT > 1) {
            x_put(s_buf[0], IC<0>{});
        } else {
            if (needmask(jlo)) mask(s_buf[0], kb0);
            row_max(s_buf[0], jlo);
        }
        // every wave is done with smK[0] before block 0 refills it (and has published its
        // partial scores of block 0)
        if constexpr (DSPLIT > 1) __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // blocks in pairs (block jlo + even in buffer 0); block j+1's mask is needed iff
    // j + 1 >= nfull (or, for windows, j + 1 < jfree)
    int j = jlo;
    if constexpr (EXT) {
        // the window's lower edge: the next block reaches below some query's window
        for (; j + 2 < nkb_c && j + 1 < jfree; j += 2) {
            step(j, IC<0>{}, IC<1>{}, IC<1>{});
            step(j + 1, IC<1>{}, IC<1>{}, IC<1>{});
        }
    }
    for (; j + 2 < nkb_c && j + 2 < nfull; j += 2) {
        step(j, IC<0>{}, IC<1>{}, IC<0>{});
        step(j + 1, IC<1>{}, IC<1>{}, IC<0>{});
    }
    for (; j + 2 < nkb_c; j += 2) {
        if (needmask(j + 1)) step(j, IC<0>{}, IC<1>{}, IC<1>{});
        else step(j, IC<0>{}, IC<1>{}, IC<0>{});
        step(j + 1, IC<1>{}, IC<1>{}, IC<1>{});
    }
    if (j + 1 < nkb_c) {
        if (needmask(j + 1)) step(j, IC<0>{}, IC<1>{}, IC<1>{});
        else step(j, IC<0>{}, IC<1>{}, IC<0>{});
        step(j + 1, IC<1>{}, IC<0>{}, IC<0>{});
    } else {
        step(j, IC<0>{}, IC<0>{}, IC<0>{});
    }
    if constexpr (PER_WAVE) {
        // the workgroup's blocks past this wave's queries: its share of their loads, and
        // their barriers (every wave passes nkb - jlo barriers in the loop)
        for (int jj = nkb_c; jj < nkb; ++jj) {
            const int kb = jj * BC;
            const bool odd = ((jj - jlo) & 1) != 0;   // buffer parity of block jj (selects, not a
                                                      // run-time index into the pointer pairs)
            if constexpr (PIPE) {
                if (jj + 2 < nkb) load_k(kb + 2 * BC, odd ? smK1 : smK0);
            } else {
                if (jj + 1 < nkb) load_k(kb + BC, odd ? smK0 : smK1);
            }
            if (jj + 1 < nkb) {
                uint8_t* const vn = odd ? smV0 : smV1;
                load_v(kb + BC, vn);
                store_v(vn);   // FP8: the staged V, expanded (the loads are awaited first)
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }
    }

    // ---- epilogue: O = O~ / l, LSE = (m + log2 l) ln 2.
    if constexpr (C::F8) {
        // fp32 O, straight from the accumulators: register 4a + b of d tile e holds
        // d = 32 e + 8 a + 4 h + b of query col, so each lane writes whole 16-byte runs
        float* const O = (float*)Ov;
#pragma unroll
        for (int n = 0; n < NQ; ++n) {
            const float l_tot = pair_sum(l_run[n]);   // lanes l and l^32 hold the two halves of a row's sum
            const float inv = l_tot > 0.f ? svmax / l_tot : 0.f;
            if (qrow[n] < N) {
                float* const orow = O + head_off + (size_t)qrow[n] * D + hd * (D / DSPLIT) + 4 * h;
#pragma unroll
                for (int e = 0; e < DTW; ++e)
#pragma unroll
                    for (int a = 0; a < 4; ++a)
                        *(f32x4*)(orow + 32 * e + 8 * a) =
                            f32x4{acc[n][e][4 * a] * inv, acc[n][e][4 * a + 1] * inv, acc[n][e][4 * a + 2] * inv,
                                  acc[n][e][4 * a + 3] * inv};
                if (LSE != nullptr && h == 0 && hd == 0)
                    LSE[qbase + qrow[n]] = l_tot > 0.f ? (m_run[n] + __log2f(l_tot)) * kLn2 : -INFINITY;
            }
        }
        return;
    }
    // bf16 O: each wave stages its 32 x d tile in LDS (the tile slots are free after the last
    // barrier) and writes it back in whole rows, 16 bytes per lane: a lane's own results are
    // 4-element runs scattered over the d range, which would make every store instruction touch
    // 32 rows.
    bf16_t* const O = (bf16_t*)Ov;
    constexpr int DW = D / DSPLIT;                     // columns of O this wave writes
    constexpr int OROW = DW * 2;                       // bytes per staged bf16 row
    constexpr int OSTAGE = 32 * OROW;                  // one wave's tile
    constexpr int OSW = (OROW / 16 < 16 ? OROW / 16 : 16) - 1;   // XOR mask of the 16-byte chunks
    constexpr bool KFITS = C::K_BYTES >= OSTAGE;       // V slots always fit (BC >= 32 rows)
    static_assert(C::V_BYTES >= OSTAGE, "a V slot must hold a wave's O tile");
    constexpr int LPR = OROW / 16;                     // lanes per row in the write-back
    constexpr int RPI = kWave / LPR;                   // rows per write-back instruction
    // staging slots: the V tiles, and the K tiles when they are large enough; waves take
    // turns when there are fewer slots than waves
    constexpr int NSLOT = KFITS ? 4 : 2;
    constexpr int ROUNDS = (WAVES + NSLOT - 1) / NSLOT;
    const int slot = wave % NSLOT;
    uint8_t* const stg = slot == 0 ? smV0 : slot == 1 ? smV1 : slot == 2 ? smK0 : smK1;
#pragma unroll
    for (int round = 0; round < ROUNDS; ++round) {
        if (wave / NSLOT == round) {
#pragma unroll
            for (int n = 0; n < NQ; ++n) {
                const float l_tot = pair_sum(l_run[n]);   // lanes l and l^32 hold the two halves of a row's sum
                const float inv = l_tot > 0.f ? svmax / l_tot : 0.f;
                // result register 4a + b of d tile e holds d = 32 e + 8 a + 4 h + b of query col:
                // 16-byte chunk 4 e + a of the row, half h
#pragma unroll
                for (int e = 0; e < DTW; ++e)
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        bf16x4 ov;
#pragma unroll
                        for (int b = 0; b < 4; ++b) ov[b] = (bf16_t)(acc[n][e][4 * a + b] * inv);
                        *(bf16x4*)(stg + col * OROW + 16 * ((4 * e + a) ^ (col & OSW)) + 8 * h) = ov;
                    }
                if (LSE != nullptr && h == 0 && hd == 0 && qrow[n] < N)
                    LSE[qbase + qrow[n]] = l_tot > 0.f ? (m_run[n] + __log2f(l_tot)) * kLn2 : -INFINITY;
                // the wave reads back what its other lanes wrote
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
                __builtin_amdgcn_wave_barrier();
                const int qt0 = q0w + 32 * n;
#pragma unroll
                for (int it = 0; it < 32 / RPI; ++it) {
                    const int r = RPI * it + lane / LPR;
                    const int c = lane % LPR;
                    const i32x4 v = *(const i32x4*)(stg + r * OROW + 16 * (c ^ (r & OSW)));
                    if (qt0 + r < N) *(i32x4*)((uint8_t*)(O + head_off + (size_t)(qt0 + r) * D + hd * DW) + 16 * c) = v;
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);
                __builtin_amdgcn_wave_barrier();
            }
        }
        if (round + 1 < ROUNDS) __syncthreads();
    }
}

// EXT kernels: BH = (sequences or batches) x Hq workgroup rows, N = the longest sequence (the
// grid's query blocks), ext as described at FwdExt
template <InKind KIND, int D, int BC, int NQ, bool CAUSAL, int TAU, int MINB, bool PIPE, int WAVES = 4, bool EXT = false,
          int DSPLIT = 1>
hipError_t launch_fwd_kernel(const void* q, const void* k, const void* v, const float* sq, const float* sk,
                             const float* sv, void* o, float* lse, int BH, int N, float scale, hipStream_t stream,
                             FwdExt ext = FwdExt{}) {
    constexpr int BR = WAVES / DSPLIT * 32 * NQ;
    const int numQB = (N + BR - 1) / BR;
    const int nsb = (N + 63) / 64;
    long long total = (long long)BH * numQB;
    // packed sequences: at most sum over s of ceil(n_s / BR) <= (ntot + nseq (BR - 1)) / BR
    // blocks per head (the extra workgroups of a loose bound return at once)
    if (EXT && ext.cu != nullptr)
        total = std::min(total, (long long)ext.Hq * (((long long)ext.ntot + (long long)ext.nseq * (BR - 1)) / BR));
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    // causal: heads walked block-first per XCD, all of the XCD's heads at once or, with 16 or
    // more heads per XCD, in groups of about two rounds of its workgroup slots (32 CUs x MINB):
    // fewer heads' K and V then share its L2, and each group still dispatches its costliest
    // blocks first (at least two heads per group: one alone leaves its light blocks for the
    // group's end). With 8 or fewer heads per XCD the groups measured no better. d = 256 (one
    // workgroup per CU, twice the K/V bytes per key): head by head
    int hgroup = 1;
    if (CAUSAL && D <= 128) {
        hgroup = 0;   // the XCD's whole range
        if (BH % 8 == 0 && BH / 8 >= 16) {
            const int nh = BH / 8;   // heads per XCD
            int g = std::min(nh, std::max(2, 2 * 32 * MINB / std::max(1, numQB)));
            while (nh % g != 0) --g;
            hgroup = g;
        }
    }
    hipLaunchKernelGGL((fwd_kernel<KIND, D, BC, NQ, CAUSAL, TAU, MINB, PIPE, WAVES, EXT, DSPLIT>), dim3((unsigned)total),
                       dim3(64 * WAVES), 0, stream, q, k, v, sq, sk, sv, o, lse, N, numQB, nsb, scale * kLog2e, hgroup,
                       ext);
    return hipGetLastError();
}

}  // namespace fa
