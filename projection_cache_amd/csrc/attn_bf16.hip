// Decode-time attention kernels instantiated for bf16 caches (see
// attn_kernels.h; one translation unit per element type so they build in
// parallel).
#include "attn_kernels.h"

namespace cke {

hipError_t launch_cross_bf16(const XattnLaunch& a, hipStream_t st) { return launch_cross_t<uint16_t>(a, st); }
hipError_t launch_weights_bf16(const WeightsLaunch& a, hipStream_t st) { return launch_weights_t<uint16_t>(a, st); }
hipError_t launch_self_bf16(const SelfLaunch& a, hipStream_t st) { return launch_self_t<uint16_t>(a, st); }
hipError_t launch_prefill_bf16(const PrefillLaunch& a, hipStream_t st) { return launch_prefill_t<uint16_t>(a, st); }

}  // namespace cke
