// Scan and output stage in one launch, for short pooled layers without the
// post-SSM LayerNorm: a workgroup scans kScanCh = 64 channels of one image
// (both directions, or forward with LBMamba's local backward scan; scan_core.h)
// and then writes every output token of the image for those channels,
//   out[b, cell, e] = (s_fwd[b, t, e] + s_bwd[b, t, e] + (D_fwd[e] + D_bwd[e]) x[b, cell, e]) * silu(z[b, cell, e])
// with t the cell's row (COLS), its column (ROWS) or its kept token's row
// (masked; an invalid index gives NaN).
//
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解,
// bullets 3-5: the scans over the pooled tokens, then the repeat along the
// pooled axis and the skip connection; bullet 6: the masked variant writes
// only the kept tokens; Vim article (ijyty.com), section 2.1: the two
// directions are summed and gated by silu(z).
//
// Why one launch: on a short layer (a 14 x 14 grid, or 49 kept tokens) the
// scan is bound by VALU issue and the output stage by HBM.  As two kernels
// they run one after the other; here a workgroup streams its outputs while
// the other workgroups on its CU still scan, so the two overlap, and the
// scan outputs go from the scanning lanes to the output lanes through LDS
// (each lane stores its outputs there as well, scan_core.h SLDS) instead of a
// second kernel's reads.  The scan outputs are still stored to the workspace
// (s_fwd, s_bwd), where the stage exports and the stage-by-stage path find
// them.
//
// A workgroup's output tokens are 64 channels wide: 256 bytes (fp32) or 128
// bytes (bf16) per token, one 16-byte column per lane, 32 or 64 tokens per
// pass of 512 lanes, kOutU tokens per lane in flight; for single-chunk scans
// each lane's first output token's x and z are loaded before the scan.  x and
// z are read for the last time and out written once (non-temporal); x and
// out may be one buffer (x_conv written out into out), each element being
// read by the lane that then writes it.
#include "scan_core.h"

namespace fastvim {
namespace {

constexpr int kOutTmax = 64;  // longest scan whose outputs the workgroup stages in LDS
constexpr int kOutU = 4;      // output tokens per lane per pass
enum { kOutCols = 0, kOutRows = 1, kOutMasked = 2 };

__device__ __forceinline__ float out_silu(float q) { return q * __builtin_amdgcn_rcpf(1.f + __expf(-q)); }

struct OutArgs {
    const void* x;
    const void* z;
    void* out;
    const float* Df;
    const float* Db;
    const int32_t* rows;  // (B, K) masked: scan row of each kept token, -1 if invalid
    int h, w, K;
};

template <int RMAX, class IO, int MODE, bool LOCAL, bool MFMA>
__global__ void __launch_bounds__(kScanThreads) scan_out_kernel(ScanArgs a, USrcPooled usrc, int nEg, OutArgs o) {
    __shared__ __attribute__((aligned(16))) float xs[chunk_lds_floats<RMAX>()];
    __shared__ __attribute__((aligned(16))) float qs[MFMA ? kScanThreads / 64 * 256 : 4];
    __shared__ __attribute__((aligned(16))) float so[2 * kOutTmax * kScanCh];  // scan outputs [dir][t][channel]
    using elem = typename IO::elem;
    using raw = typename IO::raw;
    constexpr int V = IO::V;
    constexpr int kCols = kScanCh / V;  // 16-byte columns of the channel group
    // single-chunk scans: the lane's first output token's x and z load before
    // the scan, so their latency hides under it (one token: more registers
    // would cost the kernel a workgroup per CU; longer scans leave the
    // registers to the matrix-core step sizes)
    constexpr int kPre = MFMA ? 0 : 1;
    const int64_t b = blockIdx.x / nEg;
    const int64_t e0 = (int64_t)(blockIdx.x % nEg) * kScanCh;
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int T = (int)a.T, E = (int)a.E;
    const int nch = E - (int)e0 < kScanCh ? E - (int)e0 : kScanCh;
    const int c = tid % kCols, g = tid / kCols, G = nthr / kCols;
    const int cc = c * V;         // the lane's first channel within the group
    const bool on = cc < nch;     // E is a multiple of V: a column is wholly inside E or wholly past it
    const int64_t col = e0 + (on ? cc : 0);
    const int ntok = MODE == kOutMasked ? o.K : o.h * o.w;
    const int64_t img = b * (int64_t)ntok * E;
    const elem* xb = static_cast<const elem*>(o.x) + img + col;
    const elem* zb = static_cast<const elem*>(o.z) + img + col;
    elem* ob = static_cast<elem*>(o.out) + img + col;
    raw xr[kOutU], zr[kOutU];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const int p = g + G * u;
        if (on && p < ntok) {
            xr[u] = load_raw<true>(xb + (int64_t)p * E);
            zr[u] = load_raw<true>(zb + (int64_t)p * E);
        }
    }
    scan_tile<RMAX, false, USrcPooled, LOCAL, MFMA, true, true>(a, usrc, b, e0, xs, qs, so);
    __syncthreads();  // every scan output of the group is in so
    if (!on) return;
    float dsum[V];
#pragma unroll
    for (int v = 0; v < V; ++v) dsum[v] = o.Df[col + v] + o.Db[col + v];
    const int32_t* rb = MODE == kOutMasked ? o.rows + b * o.K : nullptr;
    for (int p0 = g; p0 < ntok; p0 += G * kOutU) {
        // tokens not loaded yet: all of them, except the first pass's first kPre
#pragma unroll
        for (int u = 0; u < kOutU; ++u) {
            const int p = p0 + G * u;
            if ((u >= kPre || p0 != g) && p < ntok) {
                xr[u] = load_raw<true>(xb + (int64_t)p * E);
                zr[u] = load_raw<true>(zb + (int64_t)p * E);
            }
        }
#pragma unroll
        for (int u = 0; u < kOutU; ++u) {
            const int p = p0 + G * u;
            if (p >= ntok) continue;
            const int t = MODE == kOutCols ? p / o.w : MODE == kOutRows ? p % o.w : rb[p];
            const bool valid = MODE != kOutMasked || t >= 0;
            float sv[V];
            if (valid) {
                // s_fwd + s_bwd, added in that order (as the two-launch output stage does)
                const float* sf = so + t * kScanCh + cc;
                const float* sb = so + (T + t) * kScanCh + cc;
#pragma unroll
                for (int v = 0; v < V; v += 4) {
                    const f32x4 f4 = *reinterpret_cast<const f32x4*>(sf + v);
                    const f32x4 b4 = *reinterpret_cast<const f32x4*>(sb + v);
                    sv[v] = f4.x + b4.x;
                    sv[v + 1] = f4.y + b4.y;
                    sv[v + 2] = f4.z + b4.z;
                    sv[v + 3] = f4.w + b4.w;
                }
            }
            float ov[V];
#pragma unroll
            for (int v = 0; v < V; ++v)
                ov[v] = valid ? (sv[v] + dsum[v] * raw_at(xr[u], v)) * out_silu(raw_at(zr[u], v))
                              : __builtin_nanf("");
            store_vec<true>(ob + (int64_t)p * E, ov);
        }
    }
}

template <int RMAX, class IO, int MODE, bool MFMA>
hipError_t scan_out_launch_m(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                             const Workspace& ws, void* out, hipStream_t st) {
    ScanArgs a{ws.xdbl, p.fwd, p.bwd, ws.s_f, ws.s_b, g.T, g.E, (int)g.R, (int)g.NX};
    OutArgs o{x, z, out, p.fwd.D, p.bwd.D, ws.rows, (int)g.h, (int)g.w, (int)g.K};
    const USrcPooled usrc{ws.u, g.T, g.E};
    const int nEg = (int)((g.E + kScanCh - 1) / kScanCh);
    const dim3 grid((unsigned)(g.B * nEg));
    if (p.flags & FASTVIM_FLAG_LOCAL_BWD)
        hipLaunchKernelGGL((scan_out_kernel<RMAX, IO, MODE, true, MFMA>), grid, dim3(kScanThreads / 2), 0, st, a,
                           usrc, nEg, o);
    else
        hipLaunchKernelGGL((scan_out_kernel<RMAX, IO, MODE, false, MFMA>), grid, dim3(kScanThreads), 0, st, a,
                           usrc, nEg, o);
    return hipGetLastError();
}

// matrix-core step sizes for scans longer than one chunk, as the stage scan kernel
template <int RMAX, class IO, int MODE>
hipError_t scan_out_launch(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                           const Workspace& ws, void* out, hipStream_t st) {
    return g.T > kChunk ? scan_out_launch_m<RMAX, IO, MODE, true>(g, x, z, p, ws, out, st)
                        : scan_out_launch_m<RMAX, IO, MODE, false>(g, x, z, p, ws, out, st);
}

template <class IO, int MODE>
hipError_t scan_out_rank(const Geom& g, const void* x, const void* z, const fastvim_params& p, const Workspace& ws,
                         void* out, hipStream_t st) {
    if (g.R <= 16) return scan_out_launch<16, IO, MODE>(g, x, z, p, ws, out, st);
    if (g.R <= 32) return scan_out_launch<32, IO, MODE>(g, x, z, p, ws, out, st);
    if (g.R <= 48) return scan_out_launch<48, IO, MODE>(g, x, z, p, ws, out, st);
    return scan_out_launch<64, IO, MODE>(g, x, z, p, ws, out, st);
}

template <class IO>
hipError_t scan_out_mode(const Geom& g, const void* x, const void* z, const fastvim_params& p, const Workspace& ws,
                         void* out, hipStream_t st) {
    if (g.masked) return scan_out_rank<IO, kOutMasked>(g, x, z, p, ws, out, st);
    if (g.axis == FASTVIM_POOL_COLS) return scan_out_rank<IO, kOutCols>(g, x, z, p, ws, out, st);
    return scan_out_rank<IO, kOutRows>(g, x, z, p, ws, out, st);
}

}  // namespace

bool scan_out_supported(const Geom& g, uint32_t flags) {
    return g.pooled && g.T <= kOutTmax && !(flags & (FASTVIM_FLAG_POST_NORM | FASTVIM_FLAG_CONV));
}

hipError_t launch_scan_out(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                           const Workspace& ws, void* out, hipStream_t st) {
    return g.io == FASTVIM_BF16 ? scan_out_mode<IoBf16>(g, x, z, p, ws, out, st)
                                : scan_out_mode<IoF32>(g, x, z, p, ws, out, st);
}

}  // namespace fastvim
