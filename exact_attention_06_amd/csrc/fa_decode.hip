// Split-key decoding: a few query positions (Nq) against a long key/value sequence (Nk), with
// grouped key/value heads.
//
// Source: "FlashAttention 2 & 3: Work Partitioning, Warp Specialization & FP8", the paragraph on
// the decode regime: with one query per sequence Q K^T is a matrix-vector product and the
// query-parallel grid has nothing to split, so the key/value sequence is split across the
// compute units, each part computes a partial softmax state and the parts are combined with
// the online-softmax merge ("FlashAttention-3 & GPU Kernel Optimization", section "Online
// softmax tiling mathematics"). The work is bound by reading K and V from HBM.
//
// Work mapping (one pass over K and V):
// - the g = Hq / Hkv query heads that share a key/value head and their Nq positions form
//   R = g Nq rows; a workgroup takes 32 of them (column group cg) as the 32 MFMA columns, so
//   K and V of a head are read once for all of its query heads (twice only when R > 32);
// - the keys are cut into nsplit ranges of whole 32-key tiles; workgroup (b, hkv, cg, split)
//   has 4 waves that take the range's tiles in turn (tile t0 + w, t0 + w + 4, ...), each
//   streaming its own tiles into its own two K and two V buffers in LDS (direct-to-LDS
//   loads). A buffer is refilled with the wave's tile after next as soon as its reads are done
//   (K after the S product, V after the PV product), and the wait at the end of a step leaves
//   those loads in flight: two tiles per wave on the way from HBM most of the time, in the
//   128 KB of LDS that four waves' buffers take;
// - per tile a wave computes S^T = K Q^T (32 keys x 32 rows; the key rows are read in the
//   swap_bits23 order, so that the result registers are the next product's B operand), the
//   online softmax per row (lane pair), and O^T += V^T P^T with V^T from the transposing read;
// - the four waves' states are merged in LDS; with one split the workgroup writes O and LSE,
//   otherwise it writes its state (m, l, O~) and decode_merge_kernel combines the splits.
//
// Causal reading: the Nq queries are the last Nq positions; row (gi, i) sees keys
// j <= Nk - Nq + i. Scores are kept in log2 units (S scale log2 e).
#include <mutex>

#include "fa_common.h"
#include "fa_fwd_kernel.h"   // kBufferConfig
#include "fa_internal.h"
#include "fa_tile.h"

// Split states of the allocation-free entry point (fa_decode_noalloc): one copy per GPU, held
// until the process ends. Host code never passes this name to a kernel (on the host it is a
// stand-in, not a device address): it uses the per-device address that hipGetSymbolAddress
// returns (fa::decode_scratch).
static __device__ __align__(256) uint8_t scratch[fa::kDecodeScratchBytes];

namespace fa {
namespace {

// workgroups a decoding launch aims for (one resident per compute unit)
constexpr int kDecTargetWG = 256;
// the static scratch holds the largest workspace this plan can ask for (see decode_plan)
static_assert(kDecodeScratchBytes == (size_t)(2 * kDecTargetWG - 2) * 32 * (128 + 2) * 4, "decode scratch bound");
constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr float kDecSentinel = -1e30f;   // running max before any visible key (finite: exp2(x - m) stays defined)

template <int V>
using DIC = std::integral_constant<int, V>;

// s_waitcnt operand: wait until at most n vector-memory operations are outstanding (the LDS
// and export counters left at their maxima)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
constexpr int kLgkm0 = 0xc07f;   // lgkmcnt(0), the other counters at their maxima

template <int D>
__global__ __launch_bounds__(kDecThreads, 1) void decode_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    bf16_t* __restrict__ O, float* __restrict__ LSE, float* __restrict__ part_o, float* __restrict__ part_ml,
    int Hq, int Hkv, int Nq, int Nk, int R, int ncg, int nsplit, int tps, float c2, int causal) {
    using C = TileCfg<D, 32, 1>;
    constexpr int TB = C::TB;
    // one array per buffer (the compiler then knows that a load into one buffer does not
    // touch the others, and waits only for the loads a read depends on); wave w's tiles at
    // offset w TB of each
    __shared__ __attribute__((aligned(1024))) uint8_t sK0[kDecWaves * TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sK1[kDecWaves * TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sV0[kDecWaves * TB];
    __shared__ __attribute__((aligned(1024))) uint8_t sV1[kDecWaves * TB];
    static_assert(16 * D * 4 == TB, "a wave's fp32 state (32 x D) fills its two K tiles");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, col = lane & 31;
    int id = blockIdx.x;
    const int split = id % nsplit;
    id /= nsplit;
    const int cg = id % ncg;
    const int bkv = id / ncg;                  // b * Hkv + hkv
    const int b = bkv / Hkv, hkv = bkv - b * Hkv;
    const int g = Hq / Hkv;

    // this lane pair's query row
    const int r = cg * 32 + col;
    const bool valid = r < R;
    const int gi = valid ? r / Nq : 0;
    const int qi = valid ? r - gi * Nq : 0;
    const size_t qrow = (size_t)(b * Hq + hkv * g + gi) * Nq + qi;
    bf16x8 qf[C::KSTEPS];
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) qf[s] = valid ? *(const bf16x8*)(Q + qrow * D + 16 * s + 8 * h) : bf16x8{};
    const int lim = causal ? Nk - Nq + qi : Nk - 1;               // last key this row sees

    const size_t head = (size_t)bkv * Nk * D;
    const __amdgpu_buffer_rsrc_t rK = __builtin_amdgcn_make_buffer_rsrc((void*)(K + head), (short)0, Nk * C::ROW, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rV = __builtin_amdgcn_make_buffer_rsrc((void*)(V + head), (short)0, Nk * C::ROW, kBufferConfig);
    TileAddr<D, 32, 1> ta;
    ta.init(0, lane);
    const int wo = wave * TB;

    const int ntiles = (Nk + 31) / 32;
    const int t0 = split * tps, t1 = min(ntiles, t0 + tps);
    // tiles below tfree are visible to every row in full
    const int tfree = ((causal ? Nk - Nq : Nk - 1) + 1) / 32;

    float m = kDecSentinel, l = 0.f;
    f32x16 acc[C::DT];
#pragma unroll
    for (int e = 0; e < C::DT; ++e) acc[e] = f32x16{};

    // tile t in buffer pair B (0 or 1; -1: par); tile t + 4 is on its way into the other pair,
    // and tile t + 8 is loaded into this pair as its K and V reads finish
    constexpr int W = kDecWaves;
    int par = 0;
    auto step = [&](int t, auto b_c, auto mask_c) __attribute__((always_inline)) {
        constexpr int BC_ = decltype(b_c)::value;
        constexpr bool MASK = decltype(mask_c)::value != 0;
        uint8_t* const kt = (BC_ == 1 ? sK1 : BC_ == 0 ? sK0 : (par ? sK1 : sK0)) + wo;
        uint8_t* const vt = (BC_ == 1 ? sV1 : BC_ == 0 ? sV0 : (par ? sV1 : sV0)) + wo;
        const bool more = t + 2 * W < t1;
        f32x16 st{};
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s)
            st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.row_operand(kt, s), qf[s], st, 0, 0, 0);
        if (more) {
            __builtin_amdgcn_s_waitcnt(kLgkm0);   // the K reads are done: refill the buffer
            ta.load(rK, kt, (t + 2 * W) * 32, 0);
        }
        // register i holds key 32 t + 16(i/8) + 8h + i%8 of this lane's row
        if constexpr (MASK) {
            const int off = lim - 32 * t - 8 * h;
#pragma unroll
            for (int i = 0; i < 16; ++i) st[i] = (16 * (i / 8) + (i % 8)) > off ? -INFINITY : st[i];
        }
        float mx = st[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, st[i]);
        mx = pair_max(mx);
        const float mnew = fmaxf(m, mx * c2);
        const float alpha = fast_exp2(m - mnew);
        m = mnew;
        bf16x8 pf[2];
        float ls = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(__builtin_fmaf(st[i], c2, -m));
            ls += p;
            pf[i / 8][i % 8] = (bf16_t)p;
        }
        l = __builtin_fmaf(l, alpha, ls);
        if (wave_any(alpha < 1.f)) {
#pragma unroll
            for (int e = 0; e < C::DT; ++e)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[e][i] *= alpha;
        }
#pragma unroll
        for (int ch = 0; ch < 2; ++ch)
#pragma unroll
            for (int e = 0; e < C::DT; ++e)
                acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta.tr_operand(vt, e, ch), pf[ch], acc[e], 0, 0, 0);
        if (more) {
            __builtin_amdgcn_s_waitcnt(kLgkm0);   // the V reads are done: refill the buffer
            ta.load(rV, vt, (t + 2 * W) * 32, 0);
            // tile t + 4 (issued a step earlier) has landed; tile t + 8's loads stay in flight
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * C::LOADS));
        } else {
            __builtin_amdgcn_s_waitcnt(0);
        }
        __builtin_amdgcn_wave_barrier();
    };

    int t = t0 + wave;
    if (t < t1) {
        ta.load(rK, sK0 + wo, t * 32, 0);
        ta.load(rV, sV0 + wo, t * 32, 0);
        if (t + W < t1) {
            ta.load(rK, sK1 + wo, (t + W) * 32, 0);
            ta.load(rV, sV1 + wo, (t + W) * 32, 0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * C::LOADS));
        } else {
            __builtin_amdgcn_s_waitcnt(0);
        }
        __builtin_amdgcn_wave_barrier();
    }
    const int tu = min(t1, tfree);
    for (; t + kDecWaves < tu; t += 2 * kDecWaves) {
        step(t, DIC<0>{}, DIC<0>{});
        step(t + kDecWaves, DIC<1>{}, DIC<0>{});
    }
    if (t < tu) {
        step(t, DIC<0>{}, DIC<0>{});
        t += kDecWaves;
        par = 1;
    }
    for (; t < t1; t += kDecWaves) {
        step(t, DIC<-1>{}, DIC<1>{});
        par ^= 1;
    }

    // ---- merge the four waves' states in LDS
    const float lw = pair_sum(l);
    __syncthreads();   // every wave is done with its tiles
    // wave w's fp32 state: row r (32 x D) in its K0 tile (r < 16) or K1 tile; (m, l) in its V0 tile
    auto stage = [&](int w, int row) __attribute__((always_inline)) {
        return (float*)((row < 16 ? sK0 : sK1) + w * TB + (row & 15) * D * 4);
    };
    float* const mls = (float*)(sV0);                              // [wave][32][2] (wave w at w TB)
    // register 4a + c of d tile e holds d = 32e + 8a + 4h + c of row col
#pragma unroll
    for (int e = 0; e < C::DT; ++e)
#pragma unroll
        for (int a = 0; a < 4; ++a)
            *(f32x4*)(stage(wave, col) + 32 * e + 8 * a + 4 * h) =
                f32x4{acc[e][4 * a], acc[e][4 * a + 1], acc[e][4 * a + 2], acc[e][4 * a + 3]};
    if (h == 0) {
        mls[wave * TB / 4 + col * 2] = m;
        mls[wave * TB / 4 + col * 2 + 1] = lw;
    }
    __syncthreads();
    // thread: row tid / 8, d values (tid % 8) * D / 8 .. + D / 8
    constexpr int DPT = D / 8;
    const int mr = tid >> 3;
    const int d0 = (tid & 7) * DPT;
    const int rr = cg * 32 + mr;
    if (rr >= R) return;
    float M = kDecSentinel;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, mls[w * TB / 4 + mr * 2]);
    float wgt[kDecWaves];
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
        const float lw_ = mls[w * TB / 4 + mr * 2 + 1];
        wgt[w] = lw_ > 0.f ? fast_exp2(mls[w * TB / 4 + mr * 2] - M) : 0.f;
        L = __builtin_fmaf(wgt[w], lw_, L);
    }
    float o[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) x = __builtin_fmaf(wgt[w], stage(w, mr)[d0 + j], x);
        o[j] = x;
    }
    const int rgi = rr / Nq, rqi = rr - rgi * Nq;
    const size_t orow = (size_t)(b * Hq + hkv * g + rgi) * Nq + rqi;
    if (nsplit == 1) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
        for (int j = 0; j < DPT; j += 8) {
            bf16x8 ov;
#pragma unroll
            for (int c = 0; c < 8; ++c) ov[c] = (bf16_t)(o[j + c] * inv);
            *(bf16x8*)(O + orow * D + d0 + j) = ov;
        }
        if (LSE != nullptr && (tid & 7) == 0) LSE[orow] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    } else {
        const size_t prow = ((size_t)bkv * nsplit + split) * R + rr;
#pragma unroll
        for (int j = 0; j < DPT; j += 4)
            *(f32x4*)(part_o + prow * D + d0 + j) = f32x4{o[j], o[j + 1], o[j + 2], o[j + 3]};
        if ((tid & 7) == 0) {
            part_ml[prow * 2] = M;
            part_ml[prow * 2 + 1] = L;
        }
    }
}

// Combine the splits' states of every output row (page-5 merge), one wave per row:
// M = max m_s, O = sum_s 2^(m_s - M) O~_s / sum_s 2^(m_s - M) l_s, LSE = (M + log2 l) ln 2.
// Lane s fetches split s's (m, l) (nsplit <= 64); the O~ rows are read with the lanes along
// d, several splits' loads in flight at once.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml, bf16_t* __restrict__ O,
                                                           float* __restrict__ LSE, int Hq, int Hkv, int Nq, int R,
                                                           int nsplit, long long rows) {
    constexpr int DPL = D / 64;   // values per lane
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const long long bkv = row / R;
    const int rr = (int)(row - bkv * R);
    const int b = (int)(bkv / Hkv), hkv = (int)(bkv - (long long)b * Hkv);
    const int g = Hq / Hkv;
    const int rgi = rr / Nq, rqi = rr - rgi * Nq;
    const size_t orow = (size_t)(b * Hq + hkv * g + rgi) * Nq + rqi;
    const size_t p0 = (size_t)bkv * nsplit * R + rr;   // row of split s: p0 + s R
    // the first splits' O~ rows are requested together with the (m, l) pairs: the merge then
    // waits for one round trip to memory, not one per dependent step
    constexpr int PRE = 4;
    const float* src = part_o + p0 * D + lane * DPL;
    float xp[PRE][DPL];
#pragma unroll
    for (int u = 0; u < PRE; ++u)
#pragma unroll
        for (int j = 0; j < DPL; ++j) xp[u][j] = u < nsplit ? src[(size_t)u * R * D + j] : 0.f;
    const bool have = lane < nsplit;
    const float ms = have ? part_ml[(p0 + (size_t)lane * R) * 2] : kDecSentinel;
    const float ls = have ? part_ml[(p0 + (size_t)lane * R) * 2 + 1] : 0.f;
    float M = ls > 0.f ? ms : kDecSentinel;
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k));
    const float w = ls > 0.f ? fast_exp2(ms - M) : 0.f;
    float L = w * ls;
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) L += __shfl_xor(L, k);
    float o[DPL] = {};
#pragma unroll
    for (int u = 0; u < PRE; ++u) {
        const float ws = __shfl(w, u);   // 0 past nsplit (those lanes hold l = 0)
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[j] = __builtin_fmaf(ws, xp[u][j], o[j]);
    }
    int s = PRE;
    for (; s + 4 <= nsplit; s += 4) {
        float x[4][DPL];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < DPL; ++j) x[u][j] = src[(size_t)(s + u) * R * D + j];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float ws = __shfl(w, s + u);
#pragma unroll
            for (int j = 0; j < DPL; ++j) o[j] = __builtin_fmaf(ws, x[u][j], o[j]);
        }
    }
    for (; s < nsplit; ++s) {
        const float ws = __shfl(w, s);
#pragma unroll
        for (int j = 0; j < DPL; ++j) o[j] = __builtin_fmaf(ws, src[(size_t)s * R * D + j], o[j]);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) O[orow * D + lane * DPL + j] = (bf16_t)(o[j] * inv);
    if (LSE != nullptr && lane == 0) LSE[orow] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

}  // namespace

DecodePlan decode_plan(int B, int Hq, int Hkv, int Nq, int Nk, int d) {
    DecodePlan p{};
    const long long R = (long long)(Hq / Hkv) * Nq;
    p.ncg = (int)((R + 31) / 32);
    p.ntiles = (Nk + 31) / 32;
    const long long groups = (long long)B * Hkv * p.ncg;
    // about kDecTargetWG workgroups (one resident per compute unit: the K/V buffers take 128 KB
    // of LDS at d = 128), at least 8 tiles (2 per wave) per split, at most 64 splits
    long long ns = groups > 0 ? (kDecTargetWG + groups - 1) / groups : 1;
    long long most = p.ntiles / 8 > 1 ? p.ntiles / 8 : 1;
    most = most < 64 ? most : 64;
    ns = ns < 1 ? 1 : (ns > most ? most : ns);
    p.tps = (int)((p.ntiles + ns - 1) / ns);
    p.nsplit = p.tps > 0 ? (p.ntiles + p.tps - 1) / p.tps : 1;
    if (p.nsplit < 1) p.nsplit = 1;
    p.ws_bytes = p.nsplit > 1 ? (size_t)B * Hkv * p.nsplit * R * (size_t)(d + 2) * 4 : 0;
    return p;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(hipStream_t stream, void** ptr) {
    int dev = 0;
    hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        // once per device, with that device current: the address of its copy of the array
        int cur = 0;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

hipError_t launch_decode_bf16(const void* q, const void* k, const void* v, void* o, float* lse, void* ws, int B,
                              int Hq, int Hkv, int Nq, int Nk, int d, float scale, bool causal, hipStream_t stream) {
    const DecodePlan p = decode_plan(B, Hq, Hkv, Nq, Nk, d);
    const int R = (Hq / Hkv) * Nq;
    const long long blocks = (long long)B * Hkv * p.ncg * p.nsplit;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    float* part_o = (float*)ws;
    float* part_ml = p.nsplit > 1 ? part_o + (size_t)B * Hkv * p.nsplit * R * d : nullptr;
    const float c2 = scale * kLog2e;
    const bf16_t *Qb = (const bf16_t*)q, *Kb = (const bf16_t*)k, *Vb = (const bf16_t*)v;
    bf16_t* Ob = (bf16_t*)o;
    switch (d) {
        case 64:
            hipLaunchKernelGGL((decode_kernel<64>), dim3((unsigned)blocks), dim3(kDecThreads), 0, stream, Qb, Kb, Vb,
                               Ob, lse, part_o, part_ml, Hq, Hkv, Nq, Nk, R, p.ncg, p.nsplit, p.tps, c2, (int)causal);
            break;
        case 128:
            hipLaunchKernelGGL((decode_kernel<128>), dim3((unsigned)blocks), dim3(kDecThreads), 0, stream, Qb, Kb,
                               Vb, Ob, lse, part_o, part_ml, Hq, Hkv, Nq, Nk, R, p.ncg, p.nsplit, p.tps, c2,
                               (int)causal);
            break;
        default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.nsplit == 1) return e;
    const long long rows = (long long)B * Hkv * R;
    const long long mblocks = (rows + 3) / 4;
    if (mblocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (d == 64)
        hipLaunchKernelGGL((decode_merge_kernel<64>), dim3((unsigned)mblocks), dim3(256), 0, stream, part_o, part_ml,
                           Ob, lse, Hq, Hkv, Nq, R, p.nsplit, rows);
    else
        hipLaunchKernelGGL((decode_merge_kernel<128>), dim3((unsigned)mblocks), dim3(256), 0, stream, part_o, part_ml,
                           Ob, lse, Hq, Hkv, Nq, R, p.nsplit, rows);
    return hipGetLastError();
}

}  // namespace fa
