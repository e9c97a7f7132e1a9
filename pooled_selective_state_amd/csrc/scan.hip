// Step size, zero-order-hold decay and the forward / backward selective scans.
//
// FastVim summary page (gptget.net, arXiv 2502.00594): section 方法详解,
// bullet 3 -- Delta = softplus(Parameter + s_Delta(x)) from the pooled token,
// A discretised by zero-order hold; bullet 4 -- forward and backward Mamba
// selective scans over the pooled sequence; section 术语表, "State Space
// Model" -- h_t = A h_{t-1} + B x_t, y_t = C h_t.  Per channel e, with
// A[e, n] = -exp(A_log[e, n]) and H = 0 at the start of each direction:
//   H[n] <- exp(Delta_t A[e, n]) H[n] + Delta_t B_t[n] u_t,   s_t = sum_n C_t[n] H[n]
//
// Mapping to gfx950: one lane owns one (image, channel, direction) sequence
// and keeps all N = 16 state entries, its A row (pre-scaled by log2 e for the
// hardware exp2) and its dt_proj row in registers.  A wave covers 64
// consecutive channels of one image and one direction, so the token's x_proj
// output (low-rank step input, B_t, C_t) is wave-uniform and comes through
// scalar loads; u_t is one coalesced load per lane.  Many short sequences
// pack into a wave side by side (no state reset is needed: each lane is its
// own sequence), and the 16 state entries give every lane 16 independent
// multiply-add chains per step.  The step size is computed once per (t, e)
// and never written to memory.  The scan itself writes only s.
#include "fastvim_internal.h"

namespace fastvim {
namespace {

constexpr int kN = 16;

template <class Elem, int RMAX>
__global__ void __launch_bounds__(64)
scan_kernel(const Elem* __restrict__ usrc, int pooled, int axis, int64_t h, int64_t w,
            const float* __restrict__ xdbl, fastvim_dir_params pf, fastvim_dir_params pb,
            float* __restrict__ sf, float* __restrict__ sb, int64_t T, int E, int R, int NX, int nEg) {
    const int eg = blockIdx.x % nEg;
    const int bd = blockIdx.x / nEg;
    const int dir = bd & 1;
    const int64_t b = bd >> 1;
    const int e = eg * 64 + (int)threadIdx.x;
    const bool valid = e < E;
    const int ec = valid ? e : E - 1;  // inactive lanes shadow the last channel, store nothing

    const fastvim_dir_params p = dir ? pb : pf;
    float A2[kN], hs[kN], wdt[RMAX];
    const float kLog2e = 1.4426950408889634f;
#pragma unroll
    for (int n = 0; n < kN; ++n) {
        A2[n] = -expf(p.A_log[(int64_t)ec * kN + n]) * kLog2e;
        hs[n] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < RMAX; ++r) wdt[r] = r < R ? p.dt_proj_w[(int64_t)ec * R + r] : 0.f;
    const float bias = p.dt_proj_b[ec];

    const int64_t row_stride = 2 * (int64_t)NX;
    const float* xrow = xdbl + b * T * row_stride + (int64_t)dir * NX;
    float* s = (dir ? sb : sf) + b * T * E + ec;
    const int64_t hw = h * w;

    for (int64_t step = 0; step < T; ++step) {
        const int64_t t = dir ? T - 1 - step : step;
        const float* xd = xrow + t * row_stride;
        float q = bias;
#pragma unroll
        for (int r = 0; r < RMAX; ++r)
            if (r < R) q = fmaf(wdt[r], xd[r], q);
        const float delta = q > 20.f ? q : log1pf(expf(q));
        const int64_t ui = pooled ? (b * T + t) * E + ec : (b * hw + unpooled_token(axis, t, h, w)) * E + ec;
        const float du = delta * load_elem(usrc + ui);
        const float* Bt = xd + R;
        const float* Ct = xd + R + kN;
        float acc = 0.f;
#pragma unroll
        for (int n = 0; n < kN; ++n) {
            const float a = __builtin_amdgcn_exp2f(delta * A2[n]);
            hs[n] = fmaf(a, hs[n], du * Bt[n]);
            acc = fmaf(Ct[n], hs[n], acc);
        }
        if (valid) s[t * E] = acc;
    }
}

template <class Elem, int RMAX>
hipError_t scan_launch(const Elem* usrc, const Geom& g, const fastvim_params& p, const Workspace& ws,
                       hipStream_t st) {
    const int nEg = (int)((g.E + 63) / 64);
    const unsigned blocks = (unsigned)(g.B * 2 * nEg);
    hipLaunchKernelGGL((scan_kernel<Elem, RMAX>), dim3(blocks), dim3(64), 0, st, usrc, g.pooled ? 1 : 0, g.axis,
                       g.h, g.w, ws.xdbl, p.fwd, p.bwd, ws.s_f, ws.s_b, g.T, (int)g.E, (int)g.R, (int)g.NX, nEg);
    return hipGetLastError();
}

template <class Elem>
hipError_t scan_dispatch(const Elem* usrc, const Geom& g, const fastvim_params& p, const Workspace& ws,
                         hipStream_t st) {
    if (g.R <= 16) return scan_launch<Elem, 16>(usrc, g, p, ws, st);
    if (g.R <= 32) return scan_launch<Elem, 32>(usrc, g, p, ws, st);
    return scan_launch<Elem, 64>(usrc, g, p, ws, st);
}

}  // namespace

hipError_t launch_scan(const Geom& g, const void* x, const fastvim_params& p, const Workspace& ws,
                       hipStream_t st) {
    if (g.pooled) return scan_dispatch<float>(ws.u, g, p, ws, st);
    if (g.io == FASTVIM_BF16) return scan_dispatch<uint16_t>(static_cast<const uint16_t*>(x), g, p, ws, st);
    return scan_dispatch<float>(static_cast<const float*>(x), g, p, ws, st);
}

}  // namespace fastvim
