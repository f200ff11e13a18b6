// Row-major bf16 tiles of 32 (or 64) rows streamed into LDS by direct-to-LDS buffer loads,
// with the per-lane addresses of the two ways the MFMA kernels read them: as A-operand rows
// (d contiguous) and through the transposing read (rows contiguous), and the write-back of a
// wave's transposed accumulator. Shared by the backward, the split-KV decoding and the
// short-sequence forward kernels.
#pragma once
#include "fa_common.h"

namespace fa {

// 16-byte chunk swizzle of the streamed tiles, which are read both as MFMA rows (16 rows at
// one chunk position) and by the transposing read (4 consecutive rows at 4 chunk positions
// per half wave). f(r) = 2(r&3) ^ 8(r&1) ^ ((r>>2)&3): the first two terms (the forward's V
// swizzle) make the transposing reads conflict-free, and they span a 2-dimensional subspace
// of the 4 low chunk bits that the last term (constant within 4 consecutive rows)
// complements, so f is a bijection on row & 15 for the row reads.
template <int MASK>
__device__ __forceinline__ int tile_slot(int r, int c) {
    return c ^ ((2 * (r & 3) ^ 8 * (r & 1) ^ ((r >> 2) & 3)) & MASK);
}
template <int D, int ROWS = 32, int W = 4>
struct TileCfg {
    static constexpr int ROW = D * 2;                    // bytes per bf16 row
    static constexpr int CPR = ROW / 16;                 // 16-byte chunks per row
    static constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;
    static constexpr int KSTEPS = D / 16;                // 32x32x16 products over d
    static constexpr int DT = D / 32;                    // 32-wide d tiles of a transposed accumulator
    static constexpr int TB = ROWS * ROW;                // bytes of one streamed tile
    static constexpr int RPL = 1024 / ROW;               // rows per 1 KB DMA region
    static constexpr int LOADS = TB / 1024 / W;          // DMA loads per thread per tile (W waves)
    static_assert(LOADS >= 1, "tile must give every thread a load");
    static constexpr int KSPAN = 8;                      // steps per 16 chunks
    static constexpr int KA = KSTEPS < KSPAN ? KSTEPS : KSPAN;
    static constexpr int EA = DT < 4 ? DT : 4;           // 4 d tiles = 16 chunks
};

// Per-lane addresses inside a swizzled 32-row tile:
// - rd[s]: A-operand row reads, row swap_bits23(col), chunk 2s + h (steps s and s+8 are 256
//   bytes apart);
// - trlo[e] / trhi[e]: transposed reads of d tile e for the 16-row chunk 0 (rows 16 apart keep
//   the swizzle): lane (g, L) reads 8 bytes of row 8(g>>1) + (L>>2) (and the row 4 below),
//   columns 32e + 16(g&1) + 4(L&3) .. +3, as ds_read_b64_tr_b16 expects.
// - dma[i]: source offsets of the tile loads (load i of wave w fills 1 KB region w + W i).
template <int D, int ROWS = 32, int W = 4>
struct TileAddr {
    using C = TileCfg<D, ROWS, W>;
    int rd[C::KA];
    int trlo[C::EA], trhi[C::EA];
    int dma[C::LOADS];
    __device__ __forceinline__ void init(int wave, int lane) {
        const int h = lane >> 5, col = lane & 31;
        const int rr = swap_bits23(col);
#pragma unroll
        for (int s = 0; s < C::KA; ++s) rd[s] = rr * C::ROW + 16 * tile_slot<C::SWZ>(rr, 2 * s + h);
        const int g = lane >> 4, L = lane & 15;
        const int r0 = 8 * (g >> 1) + (L >> 2);
#pragma unroll
        for (int e = 0; e < C::EA; ++e) {
            const int byte = 64 * e + 32 * (g & 1) + 8 * (L & 3);
            trlo[e] = r0 * C::ROW + 16 * tile_slot<C::SWZ>(r0, byte / 16) + (byte & 15);
            trhi[e] = (r0 + 4) * C::ROW + 16 * tile_slot<C::SWZ>(r0 + 4, byte / 16) + (byte & 15);
        }
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) {
            const int r = C::RPL * (wave + W * i) + lane / C::CPR;
            dma[i] = r * C::ROW + 16 * tile_slot<C::SWZ>(r, lane % C::CPR);
        }
    }
    // ROWS rows starting at row0 of the buffer r into tile dst
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint8_t* dst, int row0, int wave) const {
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) lds_dma16(r, dst + 1024 * (wave + W * i), dma[i] + row0 * C::ROW);
    }
    // A operand (32 rows x 16 d) of step s, rows 32 tt .. 32 tt + 31 of the tile
    __device__ __forceinline__ bf16x8 row_operand(const uint8_t* t, int s, int tt = 0) const {
        return *(const bf16x8*)(t + 32 * tt * C::ROW + 256 * (s / C::KSPAN) + rd[s % C::KSPAN]);
    }
    // A operand (32 d x 16 rows) of d tile e and 16-row chunk ch, from the transposed read
    __device__ __forceinline__ bf16x8 tr_operand(const uint8_t* t, int e, int ch) const {
        const uint8_t* base = t + 16 * ch * C::ROW + 256 * (e / 4);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(FA_LDS(bf16x4, base + trlo[e % 4]));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(FA_LDS(bf16x4, base + trhi[e % 4]));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);   // whole-vector concatenation
    }
};

// B operand of a wave's 32 resident rows (query or key `row`): 16 values of d per step,
// [16 s + 8 h, +8); zeros past N
template <int D>
__device__ __forceinline__ void load_resident(bf16x8 (&f)[D / 16], const bf16_t* base, int row, int N, int h) {
    const bool ok = row < N;
    const bf16_t* p = base + (size_t)(ok ? row : 0) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) f[s] = ok ? *(const bf16x8*)(p + 16 * s) : bf16x8{};
}

// Write a wave's transposed fp32 accumulator (lane = row col, register 4a+b of d tile e =
// column 32e + 8a + 4h + b) as bf16 rows times `mult`, staged through the wave's LDS tile
// `stg` (32 x d) so that the global stores are whole rows, 16 bytes per lane.
template <int D>
__device__ __forceinline__ void store_rows(const f32x16 (&acc)[D / 32], float mult, uint8_t* stg, bf16_t* out,
                                           int row0, int N, int lane) {
    using C = TileCfg<D>;
    const int h = lane >> 5, col = lane & 31;
#pragma unroll
    for (int e = 0; e < C::DT; ++e)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            bf16x4 ov;
#pragma unroll
            for (int b = 0; b < 4; ++b) ov[b] = (bf16_t)(acc[e][4 * a + b] * mult);
            *(bf16x4*)(stg + col * C::ROW + 16 * ((4 * e + a) ^ (col & C::SWZ)) + 8 * h) = ov;
        }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave reads back what its lanes wrote
    __builtin_amdgcn_wave_barrier();
    constexpr int LPR = C::ROW / 16, RPI = kWave / LPR;
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
        const int r = RPI * it + lane / LPR;
        const int c = lane % LPR;
        const i32x4 v = *(const i32x4*)(stg + r * C::ROW + 16 * (c ^ (r & C::SWZ)));
        if (row0 + r < N) *(i32x4*)((uint8_t*)(out + (size_t)(row0 + r) * D) + 16 * c) = v;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
}

}  // namespace fa
