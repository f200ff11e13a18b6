// bf16 attention forward: instances of the shared fused kernel (fa_fwd_kernel.h) for
// bfloat16 Q, K, V and O, with the conditional-rescale threshold 2^8.
//
// Tile choices per head dimension (keys per block BC, 32-query tiles per wave NQ,
// workgroups per CU MINB, score pipeline PIPE):
//   d =  64: BC 64, NQ 1, 2 workgroups per CU, pipelined
//   d = 128: BC 32, NQ 1, pipelined; 8 waves per workgroup (one per CU) for
//            N >= 2048, else 4 waves and 2 workgroups per CU (BC 64 needs more registers than
//            two workgroups per CU leave, and the spill reloads stall on the tile loads in
//            flight, since vector-memory counters retire in order). (NQ 2 halves the LDS operand
//            traffic per FLOP but needs one wave per SIMD with 512 registers; the compiler
//            then spills and copies between register files, and it measured ~40% slower.)
//   N <= 128 (d = 64, 128): the short-sequence kernel (fa_fwd_short.hip)
//   d = 256: BC 32, NQ 1, pipelined; 8 waves in pairs that split the head dimension (each
//            wave holds Q and O for 128 columns: the d = 128 register footprint), one
//            workgroup of 128 queries per CU. A wave holding all 256 columns needs more than
//            the 256 VGPRs; the compiler then keeps O in AGPRs and copies all 128 accumulator
//            registers every key block.
#include "fa_fwd_kernel.h"
#include "fa_internal.h"


namespace fa {
namespace {

template <int D, int BC, int NQ, int MINB, bool PIPE, int WAVES = 4, int DSPLIT = 1>
hipError_t dispatch(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, float scale,
                    bool causal, hipStream_t stream) {
    constexpr InKind K = InKind::BF16;
    return causal ? launch_fwd_kernel<K, D, BC, NQ, true, 8, MINB, PIPE, WAVES, false, DSPLIT>(
                        q, k, v, nullptr, nullptr, nullptr, o, lse, BH, N, scale, stream)
                  : launch_fwd_kernel<K, D, BC, NQ, false, 8, MINB, PIPE, WAVES, false, DSPLIT>(
                        q, k, v, nullptr, nullptr, nullptr, o, lse, BH, N, scale, stream);
}

template <int D, int BC, int NQ, int MINB, int WAVES = 4>
hipError_t dispatch_ext(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int Ngrid,
                        float scale, bool causal, const FwdExt& ext, hipStream_t stream) {
    constexpr InKind K = InKind::BF16;
    return causal ? launch_fwd_kernel<K, D, BC, NQ, true, 8, MINB, true, WAVES, true>(q, k, v, nullptr, nullptr, nullptr,
                                                                                     o, lse, BH, Ngrid, scale, stream, ext)
                  : launch_fwd_kernel<K, D, BC, NQ, false, 8, MINB, true, WAVES, true>(q, k, v, nullptr, nullptr, nullptr,
                                                                                      o, lse, BH, Ngrid, scale, stream, ext);
}

}  // namespace

// grouped heads / sliding window / packed sequences: the 4-wave tiles of the plain kernel
hipError_t launch_fwd_ext_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                               int Hkv, int N, int max_seqlen, int d, float scale, bool causal, int left, int right,
                               const int* cu_seqlens, hipStream_t stream) {
    // a bound of N or more (positions differ by at most N - 1, also within a packed sequence) is
    // no limit: mapped to -1, so that the kernel's edge arithmetic (query + right, query - left)
    // stays far inside the int range
    const auto bound = [N](int x) { return (x < 0 || x >= N) ? -1 : x; };
    const FwdExt ext{Hq, Hq / Hkv, bound(left), bound(right), N, cu_seqlens, B};
    const int BH = B * Hq;
    const int Ngrid = cu_seqlens != nullptr ? max_seqlen : N;
    switch (d) {
        case 64: return dispatch_ext<64, 64, 1, 2>(q, k, v, o, lse, BH, Ngrid, scale, causal, ext, stream);
        case 128:
            // long rows without packing: 8 waves (256 queries) share each K/V tile (grouped-head
            // causal at 8k +3.4%); packed documents keep the smaller workgroups (8 waves: -8%)
            if (cu_seqlens == nullptr && N >= 4096)
                return dispatch_ext<128, 32, 1, 1, 8>(q, k, v, o, lse, BH, Ngrid, scale, causal, ext, stream);
            return dispatch_ext<128, 32, 1, 2>(q, k, v, o, lse, BH, Ngrid, scale, causal, ext, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                           float scale, bool causal, hipStream_t stream) {
    // a whole head in one workgroup's LDS (fa_fwd_short.hip)
    if (short_fwd_applies(N, d)) return launch_fwd_short_bf16(q, k, v, o, lse, BH, N, d, scale, causal, stream);
    switch (d) {
        case 64: return dispatch<64, 64, 1, 2, true>(q, k, v, o, lse, BH, N, scale, causal, stream);
        case 128:
            // rows of 2048 or more: 8 waves (256 queries) per workgroup share each K/V tile,
            // which halves the tile traffic per FLOP (+3% at N = 8k non-causal, +1-4% causal);
            // shorter rows keep 4 waves, whose smaller workgroups balance better
            if (N >= 2048)
                return dispatch<128, 32, 1, 1, true, 8>(q, k, v, o, lse, BH, N, scale, causal, stream);
            return dispatch<128, 32, 1, 2, true, 4>(q, k, v, o, lse, BH, N, scale, causal, stream);
        case 256:
            return dispatch<256, 32, 1, 1, true, 8, 2>(q, k, v, o, lse, BH, N, scale, causal, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fa
