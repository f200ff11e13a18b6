// bf16 attention forward: instances of the shared fused kernel (fa_fwd_kernel.h) for
// bfloat16 Q, K, V and O, with the conditional-rescale threshold 2^8.
#include "fa_fwd_kernel.h"
#include "fa_internal.h"

namespace fa {

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                           float scale, bool causal, hipStream_t stream) {
    constexpr InKind K = InKind::BF16;
    switch (d) {
        case 64:
            return causal ? launch_fwd_kernel<K, 64, 64, true, 8, 2>(q, k, v, nullptr, nullptr, nullptr, o, lse, BH, N,
                                                                     scale, stream)
                          : launch_fwd_kernel<K, 64, 64, false, 8, 2>(q, k, v, nullptr, nullptr, nullptr, o, lse, BH,
                                                                      N, scale, stream);
        case 128:
            return causal ? launch_fwd_kernel<K, 128, 64, true, 8, 2>(q, k, v, nullptr, nullptr, nullptr, o, lse, BH,
                                                                      N, scale, stream)
                          : launch_fwd_kernel<K, 128, 64, false, 8, 2>(q, k, v, nullptr, nullptr, nullptr, o, lse, BH,
                                                                       N, scale, stream);
        case 256:
            return causal ? launch_fwd_kernel<K, 256, 32, true, 8, 1>(q, k, v, nullptr, nullptr, nullptr, o, lse, BH,
                                                                      N, scale, stream)
                          : launch_fwd_kernel<K, 256, 32, false, 8, 1>(q, k, v, nullptr, nullptr, nullptr, o, lse, BH,
                                                                       N, scale, stream);
        default:
            return hipErrorInvalidValue;
    }
}

}  // namespace fa
