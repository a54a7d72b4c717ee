// Decode-time attention kernels instantiated for fp32 caches (see
// attn_kernels.h; one translation unit per element type so they build in
// parallel).
#include "attn_kernels.h"

namespace cke {

hipError_t launch_cross_f32(const XattnLaunch& a, hipStream_t st) { return launch_cross_t<float>(a, st); }
hipError_t launch_weights_f32(const WeightsLaunch& a, hipStream_t st) { return launch_weights_t<float>(a, st); }
hipError_t launch_self_f32(const SelfLaunch& a, hipStream_t st) { return launch_self_t<float>(a, st); }
hipError_t launch_prefill_f32(const PrefillLaunch& a, hipStream_t st) { return launch_prefill_t<float>(a, st); }

}  // namespace cke
