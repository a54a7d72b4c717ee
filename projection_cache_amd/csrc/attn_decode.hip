// Type dispatch of the decode-time attention calls. The kernels and their
// launch templates live in attn_kernels.h; each element type is instantiated
// in a translation unit of its own (attn_f32.hip, attn_bf16.hip,
// attn_fp8.hip).
#include "attn_kernels.h"

#include <vector>

namespace cke {

namespace {

__global__ void zero_words_kernel(unsigned* __restrict__ p, size_t n) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Probe of the workgroup-to-XCD placement: workgroup i records the XCD
// (XCC_ID hardware register) it ran on.
constexpr int kProbeGroups = 2048;
__device__ unsigned xcd_probe_ids[kProbeGroups];

__global__ void xcd_probe_kernel(unsigned* __restrict__ ids) {
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    if (threadIdx.x == 0) ids[blockIdx.x] = x;
}

}  // namespace

hipError_t launch_zero_words(unsigned* p, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

bool probe_xcd_placement() {
    void* dev = nullptr;
    if (hipGetSymbolAddress(&dev, HIP_SYMBOL(xcd_probe_ids)) != hipSuccess || !dev) {
        (void)hipGetLastError();
        return false;
    }
    hipStream_t s = nullptr;
    if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    std::vector<unsigned> ids(kProbeGroups, ~0u);
    hipLaunchKernelGGL(xcd_probe_kernel, dim3(kProbeGroups), dim3(64), 0, s, static_cast<unsigned*>(dev));
    bool ok = hipGetLastError() == hipSuccess &&
              hipMemcpyAsync(ids.data(), dev, kProbeGroups * sizeof(unsigned), hipMemcpyDeviceToHost, s) ==
                  hipSuccess &&
              hipStreamSynchronize(s) == hipSuccess;
    (void)hipStreamDestroy(s);
    (void)hipGetLastError();
    for (int i = 0; ok && i < kProbeGroups; ++i) ok = ids[i] != ~0u && ids[i] == ids[i % 8];
    return ok;
}

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
