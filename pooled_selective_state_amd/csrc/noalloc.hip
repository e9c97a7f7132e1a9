// fastvim_ssm_fwd_noalloc: the layer on a scratch buffer that lives in the
// library itself, for callers that cannot allocate (graph capture, serving
// loops, harnesses that forbid allocation).
//
// The buffer is a file-scope device array.  Each GPU holds its own copy at
// its own address, and in host code the array's name is only a host-side
// stand-in, never a device address: the address a kernel may use comes from
// hipGetSymbolAddress, looked up once per GPU with that GPU current (on the
// entry point's first call there) and kept per device.  Kernels then receive
// that address as their workspace, as they receive a caller's workspace in
// fastvim_ssm_fwd.
#include <mutex>

#include "fastvim_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[FASTVIM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each GPU, once looked up

// The current GPU's scratch address into *p.
int current_scratch(void** p) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FASTVIM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FASTVIM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
            (void)hipGetLastError();
            return FASTVIM_ERR_HIP;
        }
        g_scratch[dev] = q;
    }
    *p = g_scratch[dev];
    return FASTVIM_OK;
}

}  // namespace

extern "C" int fastvim_ssm_fwd_noalloc(const void* x, const void* z, const fastvim_params* params,
                                       const fastvim_dims* dims, int pool_axis, const int32_t* mask_idx, void* out,
                                       void* stream) {
    // the GPU's buffer is looked up only after every argument has been checked
    return fastvim::fwd_on_scratch(x, z, params, dims, pool_axis, mask_idx, out, static_cast<hipStream_t>(stream),
                                   current_scratch, FASTVIM_NOALLOC_SCRATCH_BYTES);
}
