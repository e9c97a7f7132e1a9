// Plain streaming copy, a measurement aid beside the layer: its rate is the
// device's practical streaming ceiling, and since it reads and writes a known
// number of bytes once each, its hardware byte counters give the scale factor
// for the counters of the layer's kernels.
//
// Each lane moves kCopyV 16-byte vectors: all loads first (nontemporal: the
// data is not reused), then all stores (nontemporal).  Workgroups walk the
// buffer in grid-stride steps; at most kMaxBlocks are launched, which keeps
// the grid's work-item count well inside 32 bits.
#include "fastvim_internal.h"

namespace fastvim {
namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyV = 4;
constexpr int64_t kMaxBlocks = int64_t(1) << 20;

__global__ void __launch_bounds__(kCopyThreads)
calib_copy_kernel(const f32x4* __restrict__ src, f32x4* __restrict__ dst, int64_t n) {
    constexpr int64_t kPerBlock = (int64_t)kCopyThreads * kCopyV;
    for (int64_t base = (int64_t)blockIdx.x * kPerBlock + threadIdx.x; base < n; base += (int64_t)gridDim.x * kPerBlock) {
        f32x4 r[kCopyV];
#pragma unroll
        for (int k = 0; k < kCopyV; ++k) {
            const int64_t i = base + (int64_t)k * kCopyThreads;
            if (i < n) r[k] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int k = 0; k < kCopyV; ++k) {
            const int64_t i = base + (int64_t)k * kCopyThreads;
            if (i < n) __builtin_nontemporal_store(r[k], dst + i);
        }
    }
}

}  // namespace

hipError_t launch_calib_copy(void* dst, const void* src, size_t bytes, hipStream_t st) {
    const int64_t n = (int64_t)(bytes / sizeof(f32x4));
    const int64_t per_block = (int64_t)kCopyThreads * kCopyV;
    int64_t blocks = (n + per_block - 1) / per_block;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    hipLaunchKernelGGL(calib_copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, st,
                       static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), n);
    return hipGetLastError();
}

}  // namespace fastvim
