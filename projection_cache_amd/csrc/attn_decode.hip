// Type dispatch of the decode-time attention calls. The kernels and their
// launch templates live in attn_kernels.h; each element type is instantiated
// in a translation unit of its own (attn_f32.hip, attn_bf16.hip,
// attn_fp8.hip).
#include "attn_kernels.h"

namespace cke {

int cross_keys_per_pass(int D, int elem_bytes) {
    const int lpk = D * elem_bytes / 16;
    return (64 / lpk) * kCrossWaves;
}

hipError_t launch_xattn_decode(const XattnLaunch& a, hipStream_t st) {
    switch (a.dtype) {
        case CKE_F32: return launch_cross_f32(a, st);
        case CKE_BF16: return launch_cross_bf16(a, st);
        case CKE_FP8: return launch_cross_fp8(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_selfattn_append(const SelfLaunch& a, hipStream_t st) {
    return a.bf16 ? launch_self_bf16(a, st) : launch_self_f32(a, st);
}

hipError_t launch_xattn_weights(const WeightsLaunch& a, hipStream_t st) {
    switch (a.dtype) {
        case CKE_F32: return launch_weights_f32(a, st);
        case CKE_BF16: return launch_weights_bf16(a, st);
        case CKE_FP8: return launch_weights_fp8(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_selfattn_prefill(const PrefillLaunch& a, hipStream_t st) {
    return a.bf16 ? launch_prefill_bf16(a, st) : launch_prefill_f32(a, st);
}

}  // namespace cke
