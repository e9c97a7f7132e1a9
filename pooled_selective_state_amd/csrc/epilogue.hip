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
// The grid is cut into segments of tokens that are contiguous in memory (one
// grid row of w tokens; a run of kept tokens when masked).  A workgroup walks
// one segment with G groups of VE 16-byte lanes; x and z stream through once
// (non-temporal: this is their last use), out is written with non-temporal
// stores, and the scan outputs s (B, T, E) -- small, shared by every token of
// a row -- come through the caches.
#include "fastvim_internal.h"

namespace fastvim {
namespace {

enum { kModeCols = 0, kModeRows = 1, kModeNoneRow = 2, kModeNoneCol = 3, kModeMasked = 4 };

__device__ __forceinline__ float silu(float q) {
    return q * __builtin_amdgcn_rcpf(1.f + __expf(-q));
}

template <class IO, int MODE>
__global__ void __launch_bounds__(1024)
epilogue_kernel(const typename IO::elem* __restrict__ x, const typename IO::elem* __restrict__ z,
                const float* __restrict__ sf, const float* __restrict__ sb, const float* __restrict__ Df,
                const float* __restrict__ Db, typename IO::elem* __restrict__ out,
                const int32_t* __restrict__ rows, int64_t T, int64_t h, int64_t w, int64_t K, int64_t E, int VE,
                int G, int seg_len, int segs_per_img) {
    constexpr int V = IO::V;
    const int tid = threadIdx.x, c = tid % VE, g = tid / VE;
    if (g >= G) return;
    const int64_t seg = blockIdx.x;
    const int64_t b = seg / segs_per_img, sgi = seg - b * segs_per_img;
    const int64_t col = (int64_t)c * V;
    float dsum[V];
#pragma unroll
    for (int k = 0; k < V; ++k) dsum[k] = Df[col + k] + Db[col + k];

    for (int p = g; p < seg_len; p += G) {
        int64_t tok, t;
        if (MODE == kModeMasked) {
            const int64_t k = sgi * seg_len + p;
            if (k >= K) break;
            tok = b * K + k;
            t = rows[tok];
        } else {
            const int64_t i = sgi, j = p;
            tok = (b * h + i) * w + j;
            t = MODE == kModeCols ? i : MODE == kModeRows ? j : MODE == kModeNoneRow ? i * w + j : j * h + i;
        }
        float xv[V], zv[V], o[V];
        load_vec<true>(x + tok * E + col, xv);
        load_vec<true>(z + tok * E + col, zv);
        if (MODE == kModeMasked && t < 0) {
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = __builtin_nanf("");
        } else {
            const float* s1 = sf + (b * T + t) * E + col;
            const float* s2 = sb + (b * T + t) * E + col;
            float a[V], bb[V];
#pragma unroll
            for (int k = 0; k < V; k += 4) {
                float t1[4], t2[4];
                load_vec<false>(s1 + k, t1);
                load_vec<false>(s2 + k, t2);
#pragma unroll
                for (int q = 0; q < 4; ++q) { a[k + q] = t1[q]; bb[k + q] = t2[q]; }
            }
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = (a[k] + bb[k] + dsum[k] * xv[k]) * silu(zv[k]);
        }
        store_vec<true>(out + tok * E + col, o);
    }
}

template <class IO, int MODE>
hipError_t epi_launch(const Geom& g, const void* x, const void* z, const fastvim_params& p, const Workspace& ws,
                      void* out, hipStream_t st) {
    const int64_t VE = g.E / IO::V;
    int64_t seg_len, segs;
    if (MODE == kModeMasked) {
        seg_len = g.K < 8 ? g.K : 8;
        segs = (g.K + seg_len - 1) / seg_len;
    } else {
        seg_len = g.w;
        segs = g.h;
    }
    int64_t G = 1024 / VE;
    if (G > 4) G = 4;
    if (G > seg_len) G = seg_len;
    if (G < 1) G = 1;
    const int threads = (int)((VE * G + 63) / 64 * 64);
    using elem = typename IO::elem;
    hipLaunchKernelGGL((epilogue_kernel<IO, MODE>), dim3((unsigned)(g.B * segs)), dim3(threads), 0, st,
                       static_cast<const elem*>(x), static_cast<const elem*>(z), ws.s_f, ws.s_b, p.fwd.D, p.bwd.D,
                       static_cast<elem*>(out), ws.rows, g.T, g.h, g.w, g.K, g.E, (int)VE, (int)G, (int)seg_len,
                       (int)segs);
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
