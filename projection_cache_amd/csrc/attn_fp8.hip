// Decode-time attention kernels instantiated for fp8 (E4M3) caches (see
// attn_kernels.h; one translation unit per element type so they build in
// parallel).
#include "attn_kernels.h"

namespace cke {

hipError_t launch_cross_fp8(const XattnLaunch& a, hipStream_t st) { return launch_cross_t<uint8_t>(a, st); }
hipError_t launch_weights_fp8(const WeightsLaunch& a, hipStream_t st) { return launch_weights_t<uint8_t>(a, st); }

}  // namespace cke
