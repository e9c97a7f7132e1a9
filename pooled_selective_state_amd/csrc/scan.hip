// Standalone scan stage: one 512-thread workgroup per (image, 64-channel
// group) runs both scan directions over the whole sequence (see scan_core.h
// for the recurrence, its sources and the lane layout).  With LBMamba's
// local backward scan (LBMamba article, 论文创新点 1-2: run inside the forward
// scan, in the thread's registers, on its own chunk) every lane scans
// forward and follows each chunk with the chunk's local backward scan, so a
// workgroup needs half the lanes.  Used by the staged
// path (masked and unpooled layers, stage-by-stage calls); the fused layer
// kernel runs the same core as one of its work items.
#include "scan_core.h"

namespace fastvim {
namespace {

// A workgroup scans kScanCh channels: in both directions (kScanThreads
// lanes), or (LOCAL, kScanThreads / 2 lanes) forward, each lane adding the
// local backward scan of its chunks.  Half-size workgroups keep the grid as
// large as in the bidirectional case (long unpooled scans balance over the
// CUs only with several workgroups per CU).
// MFMA: the step sizes' pre-activations come from the matrix cores
// (scan_core.h, scan_step_preact_mfma), each wave's through 1 KB of LDS.
// Measured at 2048^2, B = 32: the unpooled scan (T = 16384) takes 2.87 ms with
// them against 3.04 ms on the VALU (the local scan 2.97 against 3.30 ms); a
// single-chunk scan (T = 14, dt rank 48) is slower with them (89 against
// 81 us: its 12 dependent MFMAs and the LDS hand-off do not amortise over one
// chunk, and the kernel holds 9 more VGPRs), so they serve sequences longer
// than one chunk.
template <int RMAX, class USrc, bool LOCAL, bool MFMA>
__global__ void __launch_bounds__(kScanThreads) scan_kernel(ScanArgs a, USrc usrc, int nEg) {
    __shared__ __attribute__((aligned(16))) float xs[chunk_lds_floats<RMAX>()];
    __shared__ __attribute__((aligned(16))) float qs[MFMA ? kScanThreads / 64 * 256 : 4];
    const int64_t b = blockIdx.x / nEg;
    const int64_t e0 = (int64_t)(blockIdx.x % nEg) * kScanCh;
    scan_tile<RMAX, false, USrc, LOCAL, MFMA>(a, usrc, b, e0, xs, qs);
}

template <int RMAX, class USrc, bool MFMA>
hipError_t scan_launch_m(const USrc& usrc, const Geom& g, const fastvim_params& p, const Workspace& ws,
                         hipStream_t st) {
    ScanArgs a{ws.xdbl, p.fwd, p.bwd, ws.s_f, ws.s_b, g.T, g.E, (int)g.R, (int)g.NX};
    const int nEg = (int)((g.E + kScanCh - 1) / kScanCh);
    if (p.flags & FASTVIM_FLAG_LOCAL_BWD)
        hipLaunchKernelGGL((scan_kernel<RMAX, USrc, true, MFMA>), dim3((unsigned)(g.B * nEg)),
                           dim3(kScanThreads / 2), 0, st, a, usrc, nEg);
    else
        hipLaunchKernelGGL((scan_kernel<RMAX, USrc, false, MFMA>), dim3((unsigned)(g.B * nEg)), dim3(kScanThreads),
                           0, st, a, usrc, nEg);
    return hipGetLastError();
}

template <int RMAX, class USrc>
hipError_t scan_launch(const USrc& usrc, const Geom& g, const fastvim_params& p, const Workspace& ws,
                       hipStream_t st) {
    return g.T > kChunk ? scan_launch_m<RMAX, USrc, true>(usrc, g, p, ws, st)
                        : scan_launch_m<RMAX, USrc, false>(usrc, g, p, ws, st);
}

template <class USrc>
hipError_t scan_dispatch(const USrc& usrc, const Geom& g, const fastvim_params& p, const Workspace& ws,
                         hipStream_t st) {
    if (g.R <= 16) return scan_launch<16>(usrc, g, p, ws, st);
    if (g.R <= 32) return scan_launch<32>(usrc, g, p, ws, st);
    if (g.R <= 48) return scan_launch<48>(usrc, g, p, ws, st);
    return scan_launch<64>(usrc, g, p, ws, st);
}

}  // namespace

hipError_t launch_scan(const Geom& g, const void* x, const fastvim_params& p, const Workspace& ws,
                       hipStream_t st) {
    if (g.pooled) return scan_dispatch(USrcPooled{ws.u, g.T, g.E}, g, p, ws, st);
    const bool colmajor = g.axis == FASTVIM_POOL_NONE_COLMAJOR;
    if (g.io == FASTVIM_BF16) {
        const uint16_t* xb = static_cast<const uint16_t*>(x);
        return colmajor ? scan_dispatch(USrcGrid<uint16_t, true>{xb, g.h, g.w, g.E}, g, p, ws, st)
                        : scan_dispatch(USrcGrid<uint16_t, false>{xb, g.h, g.w, g.E}, g, p, ws, st);
    }
    const float* xf = static_cast<const float*>(x);
    return colmajor ? scan_dispatch(USrcGrid<float, true>{xf, g.h, g.w, g.E}, g, p, ws, st)
                    : scan_dispatch(USrcGrid<float, false>{xf, g.h, g.w, g.E}, g, p, ws, st);
}

}  // namespace fastvim
