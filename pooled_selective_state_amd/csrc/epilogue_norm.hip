// Stage kernel of the epilogue with the post-SSM LayerNorm (the per-token
// arithmetic, its sources and the team layout are in epilogue_norm.h): one
// team of TL lanes per output token, t the scan position of the cell (its
// row, its column, its raster position, or a kept token's row).
#include "epilogue_norm.h"

namespace fastvim {
namespace {

enum { kModeCols = 0, kModeRows = 1, kModeNoneRow = 2, kModeNoneCol = 3, kModeMasked = 4 };
constexpr int kNormThreads = 256;

// x and out may be one buffer (a layer with the producer Conv1D written out
// passes x_conv in out): each token's x is read before its out is written, so
// those two pointers carry no restrict.
template <class IO, int TL, int NV>
__global__ void __launch_bounds__(kNormThreads)
epilogue_norm_kernel(const typename IO::elem* x, const typename IO::elem* __restrict__ z,
                     const float* __restrict__ sf, const float* __restrict__ sb, const float* __restrict__ Df,
                     const float* __restrict__ Db, const float* __restrict__ lnw, const float* __restrict__ lnb,
                     float eps, typename IO::elem* out, const int32_t* __restrict__ rows, int mode,
                     int64_t ntok, int64_t T, int64_t h, int64_t w, int64_t K, int E) {
    using raw = typename IO::raw;
    constexpr int kTeams = kNormThreads / TL;
    const int lane = threadIdx.x % TL;
    const int64_t tok = (int64_t)blockIdx.x * kTeams + threadIdx.x / TL;  // team-uniform
    if (tok >= ntok) return;  // whole teams leave together; no barriers below
    // scan row of the token
    int64_t b, t;
    if (mode == kModeMasked) {
        b = tok / K;
        t = rows[tok];
    } else {
        const int64_t hw = h * w;
        b = tok / hw;
        const int64_t cell = tok - b * hw, i = cell / w, j = cell - i * w;
        t = mode == kModeCols ? i : mode == kModeRows ? j : mode == kModeNoneRow ? cell : j * h + i;
    }
    typename IO::elem* ob = out + tok * E;
    if (t < 0) {  // masked token with an invalid index
        norm_nan<IO, TL, NV>(ob, E, lane);
        return;
    }
    raw xr[NV], zr[NV];
    norm_load<IO, TL, NV>(x + tok * E, z + tok * E, E, lane, xr, zr);
    norm_finish<IO, TL, NV>(xr, zr, sf + (b * T + t) * E, sb + (b * T + t) * E, Df, Db, lnw, lnb, eps, ob, E, lane);
}

template <class IO, int TL, int NV>
hipError_t norm_launch(const Geom& g, const void* x, const void* z, const fastvim_params& p, const Workspace& ws,
                       void* out, hipStream_t st) {
    using elem = typename IO::elem;
    int mode;
    if (g.masked) mode = kModeMasked;
    else if (g.axis == FASTVIM_POOL_COLS) mode = kModeCols;
    else if (g.axis == FASTVIM_POOL_ROWS) mode = kModeRows;
    else if (g.axis == FASTVIM_POOL_NONE_ROWMAJOR) mode = kModeNoneRow;
    else mode = kModeNoneCol;
    const int64_t ntok = g.B * (g.masked ? g.K : g.h * g.w);
    constexpr int kTeams = kNormThreads / TL;
    hipLaunchKernelGGL((epilogue_norm_kernel<IO, TL, NV>), dim3((unsigned)((ntok + kTeams - 1) / kTeams)),
                       dim3(kNormThreads), 0, st, static_cast<const elem*>(x), static_cast<const elem*>(z), ws.s_f,
                       ws.s_b, p.fwd.D, p.bwd.D, p.ln_weight, p.ln_bias, p.ln_eps, static_cast<elem*>(out), ws.rows,
                       mode, ntok, g.T, g.h, g.w, g.K, (int)g.E);
    return hipGetLastError();
}

// The smallest team whose lanes hold a token in at most 8 vectors each (16
// for fp32 E > 2048): fewer idle lanes for narrow layers, fewer registers for
// wide ones.
template <class IO>
hipError_t norm_dispatch(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                         const Workspace& ws, void* out, hipStream_t st) {
    const int64_t vecs = g.E / IO::V;
    if (vecs <= 16 * 8) return norm_launch<IO, 16, 8>(g, x, z, p, ws, out, st);
    if (vecs <= 32 * 8) return norm_launch<IO, 32, 8>(g, x, z, p, ws, out, st);
    if (vecs <= 64 * 8) return norm_launch<IO, 64, 8>(g, x, z, p, ws, out, st);
    return norm_launch<IO, 64, 16>(g, x, z, p, ws, out, st);  // fp32, E <= 4096
}

}  // namespace

hipError_t launch_epilogue_norm(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                                const Workspace& ws, void* out, hipStream_t st) {
    return g.io == FASTVIM_BF16 ? norm_dispatch<IoBf16>(g, x, z, p, ws, out, st)
                                : norm_dispatch<IoF32>(g, x, z, p, ws, out, st);
}

}  // namespace fastvim
