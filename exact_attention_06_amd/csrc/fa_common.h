// Device-side building blocks shared by the attention kernels (gfx950 / CDNA4 only).
//
// Everything here is written for the 64-lane wavefront and the CDNA4 matrix
// cores. The operand and result layouts below were checked on the hardware:
//
//  v_mfma_f32_32x32x16_bf16  A (32 x 16): lane l holds row l%32, k = 8*(l/32) + j (j = 0..7)
//                            B (16 x 32): lane l holds col l%32, k = 8*(l/32) + j
//                            D (32 x 32): lane l, register i holds row 8*(i/4) + 4*(l/32) + i%4, col l%32
//  v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3, unit scales): the same with 32 bytes per lane,
//                            k = 32*(l/32) + j (j = 0..31); same D layout
//  ds_read_b64_tr_b16        per group of 16 lanes, lane i element e receives element i%4 of
//                            the 8 bytes addressed by lane 4*e + i/4 of the group
//  ds_read_b64_tr_b8         per group of 16 lanes, lane i byte e receives byte i%8 of the
//                            8 bytes addressed by lane 2*e + i/8 of the group
//  v_permlane32_swap(x, x)   returns {x[l], x[l+32]} in low lanes and {x[l-32], x[l]} in high lanes
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;

#define FA_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// Largest amount (in log2 units) by which a new block maximum may exceed the
// running reference maximum before the accumulator is rescaled. Skipping
// smaller rescales keeps the result exact (the same stale reference is used in
// numerator and denominator); it only bounds the probabilities by 2^kRescaleTau.
constexpr float kRescaleTau = 8.0f;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// max / sum of x over lanes l and l^32 (the two lanes that hold one query row)
__device__ __forceinline__ float pair_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Key-row permutation within a 32-row MFMA tile: swap bits 2 and 3 of the row index.
// Feeding K row sigma(r) into A-operand row r makes the 32x32 result registers 8u..8u+7
// of lane half h hold keys 16u + 8h + 0..7, i.e. exactly the B operand of the next
// 32x32x16 product over those 16 keys.
__device__ __forceinline__ int swap_bits23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// 4-lane-group-of-the-result row index of register i for lane half h (D layout above)
__device__ __forceinline__ constexpr int mfma32_row(int i, int h) { return 8 * (i / 4) + 4 * h + (i % 4); }

// Buffer loads over a resource whose range check turns reads past the end into zeros.
// The builtins are wrapped in plain device functions: called directly from the kernel
// template with per-thread offsets they make the host compilation pass drop the kernel's
// launch stub (a silent substitution failure in clang), which leaves the library with an
// undefined symbol.
// lds_dma16: 16 bytes per lane from r + voff straight into LDS at lds + 16 * lane
// (lds must be the same for the whole wave).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ i32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}
__device__ __forceinline__ i32x2 buffer_load8(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
}

// XCD-aware work index: the dispatcher hands consecutive workgroup ids to the 8 XCDs in
// turn; remap so that each XCD walks a contiguous range of work items (a contiguous range
// of heads shares that XCD's L2).
__device__ __forceinline__ int xcd_remap(int id, int total) {
    if ((total & 7) != 0) return id;
    return (id & 7) * (total >> 3) + (id >> 3);
}

// Work item w (after xcd_remap) of total = rows x nblk items, as (row, block index).
// group == 1: row-major (one row's blocks together). Otherwise each XCD's contiguous range of
// rows is walked in groups of `group` rows (all of the range if group <= 0 or if it does not
// divide the range), each group by block index first: for causal problems the costliest
// blocks of the group's rows are dispatched before any lighter one (longest first), and only
// the group's rows share the XCD's L2 at a time.
__device__ __forceinline__ void work_item(int w, int total, int nblk, int group, int& row, int& blk) {
    row = w / nblk;
    blk = w - row * nblk;
    if (group != 1 && (total & 7) == 0) {
        const int per = total >> 3;
        const int nh = per / nblk;
        if (nh * nblk == per) {
            const int G = (group > 0 && group < nh && nh % group == 0) ? group : nh;
            const int xcd = w / per;
            const int k = w - xcd * per;
            const int g = k / (G * nblk);
            const int kk = k - g * G * nblk;
            blk = kk / G;
            row = xcd * nh + g * G + (kk - blk * G);
        }
    }
}

}  // namespace fa
