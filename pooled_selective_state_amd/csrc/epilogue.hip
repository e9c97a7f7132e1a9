// Repeat + skip + gate: every output token is written exactly once,
//   out[b, cell, e] = (s_fwd[b, t, e] + s_bwd[b, t, e] + (D_fwd[e] + D_bwd[e]) x[b, cell, e]) * silu(z[b, cell, e])
// with t the scan position of the cell: its row (COLS), its column (ROWS),
// its raster position (unpooled), or its kept token's row (masked).
//
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解,
// bullet 5: the scan output is repeated along the pooled axis, then the skip
// connection; Pith review of 2502.00594, "key_machinery": the repeat restores
// the token count before the D x skip; Vim article (ijyty.com), section 2.1:
// the forward and backward outputs are summed and gated by z.
//
// A workgroup takes a run of G * kU tokens that are contiguous in memory (part
// of one grid row, or of one image's kept tokens).  Its threads form G groups
// of VE lanes; lane c owns the 16-byte column [c*V, c*V + V) of E and thread
// (c, g) handles tokens g, g + G, ..., issuing all of its x and z loads before
// any arithmetic, so each lane keeps 2 * kU 16-byte loads in flight.  x and z
// are read for the last time (non-temporal), out is written once
// (non-temporal); the scan outputs (B, T, E) -- small, shared by the tokens of
// a row -- come through the caches.
#include "fastvim_internal.h"

namespace fastvim {
namespace {

enum { kModeCols = 0, kModeRows = 1, kModeNoneRow = 2, kModeNoneCol = 3, kModeMasked = 4 };
constexpr int kU = 4;  // tokens per thread

__device__ __forceinline__ float silu(float q) { return q * __builtin_amdgcn_rcpf(1.f + __expf(-q)); }

template <int V>
__device__ __forceinline__ void scan_sum(const float* sf, const float* sb, int64_t off, float (&sv)[V]) {
#pragma unroll
    for (int v = 0; v < V; v += 4) {
        const f32x4 p1 = load_raw<false>(sf + off + v), p2 = load_raw<false>(sb + off + v);
        sv[v] = p1.x + p2.x;
        sv[v + 1] = p1.y + p2.y;
        sv[v + 2] = p1.z + p2.z;
        sv[v + 3] = p1.w + p2.w;
    }
}

// x and out may be one buffer (a layer with the producer Conv1D written out
// passes x_conv in out): each token's x is read before its out is written, so
// those two pointers carry no restrict.
template <class IO, int MODE>
__global__ void __launch_bounds__(1024)
epilogue_kernel(const typename IO::elem* x, const typename IO::elem* __restrict__ z,
                const float* __restrict__ sf, const float* __restrict__ sb, const float* __restrict__ Df,
                const float* __restrict__ Db, typename IO::elem* out,
                const int32_t* __restrict__ rows, int64_t T, int64_t h, int64_t w, int64_t K, int64_t E, int VE,
                int G, int64_t seg_len, int64_t blocks_per_seg, int64_t segs_per_img) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    const int tid = threadIdx.x, c = tid % VE, g = tid / VE;
    if (g >= G) return;
    const int64_t blk = blockIdx.x;
    const int64_t seg = blk / blocks_per_seg;
    const int64_t p0 = (blk - seg * blocks_per_seg) * (int64_t)G * kU;  // first token of the block in its segment
    const int64_t b = seg / segs_per_img, sgi = seg - b * segs_per_img;
    const int64_t col = (int64_t)c * V;
    // token u of this thread: position p0 + g + G*u of the segment
    int64_t tok[kU];
    bool ok[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int64_t p = p0 + g + (int64_t)G * u;
        ok[u] = p < seg_len;
        tok[u] = MODE == kModeMasked ? b * K + p : (b * h + sgi) * w + p;
    }
    raw xr[kU], zr[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        if (ok[u]) {
            xr[u] = load_raw<true>(x + tok[u] * E + col);
            zr[u] = load_raw<true>(z + tok[u] * E + col);
        }
    }
    float dsum[V];
#pragma unroll
    for (int v = 0; v < V; ++v) dsum[v] = Df[col + v] + Db[col + v];
    float srow[V];
    if (MODE == kModeCols) scan_sum<V>(sf, sb, (b * T + sgi) * E + col, srow);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        if (!ok[u]) continue;
        const int64_t p = p0 + g + (int64_t)G * u;
        float sv[V];
        bool valid = true;
        if (MODE == kModeCols) {
#pragma unroll
            for (int v = 0; v < V; ++v) sv[v] = srow[v];
        } else {
            int64_t t;
            if (MODE == kModeRows) t = p;
            else if (MODE == kModeNoneRow) t = sgi * w + p;
            else if (MODE == kModeNoneCol) t = p * h + sgi;
            else t = rows[tok[u]];
            valid = t >= 0;
            if (valid) scan_sum<V>(sf, sb, (b * T + t) * E + col, sv);
        }
        float o[V];
#pragma unroll
        for (int v = 0; v < V; ++v)
            o[v] = valid ? (sv[v] + dsum[v] * raw_at(xr[u], v)) * silu(raw_at(zr[u], v)) : __builtin_nanf("");
        store_vec<true>(out + tok[u] * E + col, o);
    }
}

template <class IO, int MODE>
hipError_t epi_launch(const Geom& g, const void* x, const void* z, const fastvim_params& p, const Workspace& ws,
                      void* out, hipStream_t st) {
    const int64_t VE = g.E / IO::V;
    int64_t G = 512 / VE;
    if (G < 1) G = 1;
    const int64_t seg_len = MODE == kModeMasked ? g.K : g.w;
    const int64_t segs_per_img = MODE == kModeMasked ? 1 : g.h;
    if (G * kU > seg_len) G = (seg_len + kU - 1) / kU;
    if (G < 1) G = 1;
    const int64_t blocks_per_seg = (seg_len + G * kU - 1) / (G * kU);
    const int threads = (int)((VE * G + 63) / 64 * 64);
    using elem = typename IO::elem;
    const int64_t blocks = g.B * segs_per_img * blocks_per_seg;
    hipLaunchKernelGGL((epilogue_kernel<IO, MODE>), dim3((unsigned)blocks), dim3(threads), 0, st,
                       static_cast<const elem*>(x), static_cast<const elem*>(z), ws.s_f, ws.s_b, p.fwd.D, p.bwd.D,
                       static_cast<elem*>(out), ws.rows, g.T, g.h, g.w, g.K, g.E, (int)VE, (int)G, seg_len,
                       blocks_per_seg, segs_per_img);
    return hipGetLastError();
}

template <class IO>
hipError_t epi_dispatch(const Geom& g, const void* x, const void* z, const fastvim_params& p, const Workspace& ws,
                        void* out, hipStream_t st) {
    if (g.masked) return epi_launch<IO, kModeMasked>(g, x, z, p, ws, out, st);
    switch (g.axis) {
        case FASTVIM_POOL_COLS: return epi_launch<IO, kModeCols>(g, x, z, p, ws, out, st);
        case FASTVIM_POOL_ROWS: return epi_launch<IO, kModeRows>(g, x, z, p, ws, out, st);
        case FASTVIM_POOL_NONE_ROWMAJOR: return epi_launch<IO, kModeNoneRow>(g, x, z, p, ws, out, st);
        default: return epi_launch<IO, kModeNoneCol>(g, x, z, p, ws, out, st);
    }
}

}  // namespace

hipError_t launch_epilogue(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                           const Workspace& ws, void* out, hipStream_t st) {
    return g.io == FASTVIM_BF16 ? epi_dispatch<IoBf16>(g, x, z, p, ws, out, st)
                                : epi_dispatch<IoF32>(g, x, z, p, ws, out, st);
}

}  // namespace fastvim
