// Producer side fused into the layer: the depthwise causal Conv1D + SiLU that
// makes the layer's x is computed where x is read -- in the pool and again in
// the epilogue's skip term -- so x_conv never goes to memory.
//
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解,
// bullets 1-2: the token grid is pooled after the Conv1D; Vim article
// (ijyty.com) 2.1: conv1d, then the SSM.  With x the conv's input (B, h, w, E)
// and the oriented grid's sequence r (row-major r = i*w + j for COLS,
// column-major r = j*h + i for ROWS, the transposed grid),
//   x_conv[r, e] = silu(conv_b[e] + sum_{k<4} conv_w[e, k] x[r - 3 + k, e])
// with zeros before the start of the sequence (oldest tap first).
//
// Each token's value needs its three predecessors in the sequence: for COLS
// they are the three previous tokens in memory (crossing into the previous
// grid row at its start); for ROWS the same column of the three previous grid
// rows (crossing into earlier columns at the top).  Lanes walk runs of cells
// that follow one another in the sequence and slide a window of three raw
// vectors, so each cell is loaded once plus a halo of three per run; the halo
// is the neighbouring lane's cells, loaded at about the same time, and comes
// from the caches.  The kernels follow the pool and epilogue kernels
// (pool.hip, epilogue.hip) otherwise.
#include "bwd_internal.h"
#include "conv_common.h"

namespace fastvim {
namespace {

// ------------------------------------------------------------------ pool
// One workgroup per pooled token (b, t), G groups of VE vector lanes.  Group g
// takes a run of consecutive pooled positions [g L, g L + L): along the pooled
// axis each cell's predecessor in the sequence is the previous cell of the
// run (COLS: (t, j - 1); ROWS: (i - 1, t)), so a lane slides a window of
// three raw vectors and loads the run's cells once, plus a halo of three at
// its start.  Fixed-order LDS reduction of the G partial sums.
constexpr int kPU = 4;  // cells loaded at once per lane
template <class IO, bool COLS>
__global__ void __launch_bounds__(1024)
conv_pool_kernel(const typename IO::elem* __restrict__ x, const float* __restrict__ cw, const float* __restrict__ cb,
                 float* __restrict__ u, int T, int P, int h, int w, int VE, int G, int E, float inv_p) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    extern __shared__ float red[];  // [G][VE * V]
    const int64_t bt = blockIdx.x;
    const int64_t b = bt / T;
    const int t = (int)(bt - b * T);
    const int tid = threadIdx.x;
    const int c = tid % VE, g = tid / VE;
    const int coff = c * V;
    if (g < G) {
        ConvW<V> W;
        load_conv_w<V>(cw, cb, coff, W);
        const typename IO::elem* xb = x + b * (int64_t)h * w * E;
        const int pstr = (COLS ? 1 : w) * E;  // tokens along the pooled axis
        const int L = (P + G - 1) / G;
        const int p0 = g * L, p1 = p0 + L < P ? p0 + L : P;
        float acc[V];
#pragma unroll
        for (int v = 0; v < V; ++v) acc[v] = 0.f;
        if (p0 < p1) {
            const int i0 = COLS ? t : p0, j0 = COLS ? p0 : t;
            raw w3, w2, w1;
            load_halo<IO, COLS>(xb, coff, E, i0, j0, h, w, w3, w2, w1);
            const typename IO::elem* cell = xb + (coff + (i0 * w + j0) * E);
            for (int p = p0; p < p1; p += kPU) {
                raw cur[kPU];
#pragma unroll
                for (int q = 0; q < kPU; ++q)
                    if (p + q < p1) cur[q] = load_raw<false>(cell + (p - p0 + q) * pstr);
#pragma unroll
                for (int q = 0; q < kPU; ++q) {
                    if (p + q < p1) {
                        float xc[V];
                        conv_window<IO>(w3, w2, w1, cur[q], W, xc);
#pragma unroll
                        for (int v = 0; v < V; ++v) acc[v] += xc[v];
                        w3 = w2;
                        w2 = w1;
                        w1 = cur[q];
                    }
                }
            }
        }
#pragma unroll
        for (int v = 0; v < V; ++v) red[(g * VE + c) * V + v] = acc[v];
    }
    __syncthreads();
    const int width = VE * V;
    for (int q = tid; q < width; q += blockDim.x) {
        float s = red[q];
        for (int gg = 1; gg < G; ++gg) s += red[gg * width + q];
        u[bt * E + q] = s * inv_p;
    }
}

// -------------------------------------------------------------- epilogue
// out = (s_fwd + s_bwd + (D_fwd + D_bwd) x_conv) silu(z), each output written
// once.  Lane (c, g) takes kU cells that follow one another in the sequence
// and slides the conv window over them, with a halo of three at their start:
//   COLS: a workgroup covers G * kU consecutive cells of grid row i, lane
//         group g the cells j0 + g kU + m (the scan row i is shared);
//   ROWS: a workgroup covers kU grid rows x G columns, lane group g walks
//         column j0 + g down the rows i0 + m (its scan row j is fixed).
// All x and z loads of a lane are issued before its arithmetic.
constexpr int kU = 4;

template <class IO, bool COLS>
__global__ void __launch_bounds__(1024)
conv_epilogue_kernel(const typename IO::elem* __restrict__ x, const typename IO::elem* __restrict__ z,
                     const float* __restrict__ cw, const float* __restrict__ cb, const float* __restrict__ sf,
                     const float* __restrict__ sb, const float* __restrict__ Df, const float* __restrict__ Db,
                     typename IO::elem* __restrict__ out, int T, int h, int w, int E, int VE, int G, int nbi,
                     int nbj) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    const int tid = threadIdx.x, c = tid % VE, g = tid / VE;
    if (g >= G) return;
    // block (b, bi, bj): COLS bi = grid row, bj = run of G kU cells; ROWS bi =
    // run of kU rows, bj = run of G columns
    const int64_t blk = blockIdx.x;
    const int64_t b = blk / ((int64_t)nbi * nbj);
    const int rem = (int)(blk - b * nbi * nbj);
    const int bi = rem / nbj, bj = rem - (rem / nbj) * nbj;
    const int i0 = COLS ? bi : bi * kU;
    const int j0 = COLS ? bj * G * kU + g * kU : bj * G + g;
    const int n = COLS ? (w - j0 < kU ? w - j0 : kU) : (h - i0 < kU ? h - i0 : kU);  // cells of this lane
    if (n <= 0 || j0 >= w) return;
    const int coff = c * V;
    const int cstr = (COLS ? 1 : w) * E;  // token stride between the lane's cells
    const int64_t img = b * (int64_t)h * w * E;
    const typename IO::elem* xb = x + img;
    const int off0 = coff + (i0 * w + j0) * E;
    raw xr[kU], zr[kU];
#pragma unroll
    for (int m = 0; m < kU; ++m) {
        if (m < n) {
            xr[m] = load_raw<false>(xb + (off0 + m * cstr));
            zr[m] = load_raw<true>(z + img + (off0 + m * cstr));
        }
    }
    raw w3, w2, w1;
    load_halo<IO, COLS>(xb, coff, E, i0, j0, h, w, w3, w2, w1);
    ConvW<V> W;
    load_conv_w<V>(cw, cb, coff, W);
    float dsum[V], sv[V];
#pragma unroll
    for (int v = 0; v < V; ++v) dsum[v] = Df[coff + v] + Db[coff + v];
    const int64_t srow = (b * T + (COLS ? i0 : j0)) * E + coff;
#pragma unroll
    for (int v = 0; v < V; v += 4) {
        const f32x4 q1 = load_raw<false>(sf + srow + v), q2 = load_raw<false>(sb + srow + v);
        sv[v] = q1.x + q2.x;
        sv[v + 1] = q1.y + q2.y;
        sv[v + 2] = q1.z + q2.z;
        sv[v + 3] = q1.w + q2.w;
    }
    typename IO::elem* ob = out + img;
#pragma unroll
    for (int m = 0; m < kU; ++m) {
        if (m < n) {
            float xc[V], o[V];
            conv_window<IO>(w3, w2, w1, xr[m], W, xc);
            w3 = w2;
            w2 = w1;
            w1 = xr[m];
#pragma unroll
            for (int v = 0; v < V; ++v) o[v] = (sv[v] + dsum[v] * xc[v]) * conv_silu_f(raw_at(zr[m], v));
            store_vec<true>(ob + (off0 + m * cstr), o);
        }
    }
}

template <class IO>
hipError_t conv_pool_t(const Geom& g, const void* x, const fastvim_params& p, const Workspace& ws, hipStream_t st) {
    const int64_t VE = g.E / IO::V;
    int64_t G = 512 / VE;
    if (G > g.P) G = g.P;
    if (G < 1) G = 1;
    const int threads = (int)((VE * G + 63) / 64 * 64);
    const size_t lds = (size_t)G * VE * IO::V * sizeof(float);
    const auto* xe = static_cast<const typename IO::elem*>(x);
    if (g.axis == FASTVIM_POOL_COLS)
        hipLaunchKernelGGL((conv_pool_kernel<IO, true>), dim3((unsigned)(g.B * g.T)), dim3(threads), lds, st, xe,
                           p.conv_w, p.conv_b, ws.u, (int)g.T, (int)g.P, (int)g.h, (int)g.w, (int)VE, (int)G,
                           (int)g.E, pool_norm(g));
    else
        hipLaunchKernelGGL((conv_pool_kernel<IO, false>), dim3((unsigned)(g.B * g.T)), dim3(threads), lds, st, xe,
                           p.conv_w, p.conv_b, ws.u, (int)g.T, (int)g.P, (int)g.h, (int)g.w, (int)VE, (int)G,
                           (int)g.E, pool_norm(g));
    return hipGetLastError();
}

template <class IO>
hipError_t conv_epi_t(const Geom& g, const void* x, const void* z, const fastvim_params& p, const Workspace& ws,
                      void* out, hipStream_t st) {
    using elem = typename IO::elem;
    const int64_t VE = g.E / IO::V;
    int64_t G = 512 / VE;
    if (G < 1) G = 1;
    const bool cols = g.axis == FASTVIM_POOL_COLS;
    if (cols && G * kU > g.w) G = (g.w + kU - 1) / kU;
    if (!cols && G > g.w) G = g.w;
    if (G < 1) G = 1;
    const int64_t nbi = cols ? g.h : (g.h + kU - 1) / kU;
    const int64_t nbj = cols ? (g.w + G * kU - 1) / (G * kU) : (g.w + G - 1) / G;
    const int threads = (int)((VE * G + 63) / 64 * 64);
    const dim3 grid((unsigned)(g.B * nbi * nbj));
    const auto* xe = static_cast<const elem*>(x);
    const auto* ze = static_cast<const elem*>(z);
    auto* oe = static_cast<elem*>(out);
    if (cols)
        hipLaunchKernelGGL((conv_epilogue_kernel<IO, true>), grid, dim3(threads), 0, st, xe, ze, p.conv_w, p.conv_b,
                           ws.s_f, ws.s_b, p.fwd.D, p.bwd.D, oe, (int)g.T, (int)g.h, (int)g.w, (int)g.E, (int)VE,
                           (int)G, (int)nbi, (int)nbj);
    else
        hipLaunchKernelGGL((conv_epilogue_kernel<IO, false>), grid, dim3(threads), 0, st, xe, ze, p.conv_w, p.conv_b,
                           ws.s_f, ws.s_b, p.fwd.D, p.bwd.D, oe, (int)g.T, (int)g.h, (int)g.w, (int)g.E, (int)VE,
                           (int)G, (int)nbi, (int)nbj);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_conv_pool(const Geom& g, const void* x, const fastvim_params& p, const Workspace& ws,
                            hipStream_t st) {
    return g.io == FASTVIM_BF16 ? conv_pool_t<IoBf16>(g, x, p, ws, st) : conv_pool_t<IoF32>(g, x, p, ws, st);
}

hipError_t launch_conv_epilogue(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                                const Workspace& ws, void* out, hipStream_t st) {
    return g.io == FASTVIM_BF16 ? conv_epi_t<IoBf16>(g, x, z, p, ws, out, st)
                                : conv_epi_t<IoF32>(g, x, z, p, ws, out, st);
}

namespace {

// ------------------------------------------------------- backward, pass 2
// The second pass of the backward pass of a layer whose x is the Conv1D's
// input.  The layer's own adjoint gives, per sequence position q (cell of
// scan position t(q) = q / P),
//   g[q]   = dout silu(z),  dxc[q] = g (D_fwd + D_bwd) + du[b, t(q)] / P
//   dz[q]  = dout (s_fwd + s_bwd + (D_fwd + D_bwd) x_conv) silu'(z)
// and the conv's adjoint, with a[q] the pre-activation and da = dxc silu'(a),
//   dx[r]  = sum_k conv_w[k] da[r + 3 - k],  d conv_w[k] += da[r] x[r - 3 + k],
//   d conv_b += da[r],  dD += g[r] x_conv[r].
// A lane walks a run of the sequence positions of one scan position, kBatchCb
// positions' loads at a time.  At each position q it loads x, z and dout,
// forms x_conv, dz and da[q] (x[q - 3 .. q] in a window) and adds its terms to
// the sums, and it finishes dx[q - 3] from da[q - 3 .. q] (a ring of three).
// Past the run it forms da for three more positions (the next run's first
// cells) to finish its last dx.  Positions before the sequence have x = 0,
// positions after it da = 0.  Workgroups loop over the (image,
// scan position) items and keep per-lane sums; at the end each workgroup
// writes one row of partials [dD | d conv_b | d conv_w] (6 E floats, its
// channel slice), summed over the rows by a later kernel.
constexpr int kCbThreads = 256;  // at most; a workgroup holds G groups of VEs lanes
constexpr int kCbSlice = 128;    // most vector lanes in a workgroup's channel slice (even slices)

template <class IO, bool COLS>
__global__ void __launch_bounds__(kCbThreads)
bwd_conv_epilogue_kernel(const typename IO::elem* __restrict__ x, const typename IO::elem* __restrict__ z,
                         const typename IO::elem* __restrict__ dout, const float* __restrict__ cw,
                         const float* __restrict__ cb, const float* __restrict__ sf, const float* __restrict__ sb,
                         const float* __restrict__ du, const float* __restrict__ Df, const float* __restrict__ Db,
                         typename IO::elem* __restrict__ dx, typename IO::elem* __restrict__ dz,
                         float* __restrict__ parts, int B, int T, int P, int h, int w, int E, int VE, int VEs, int G,
                         float inv_p) {
    constexpr int V = IO::V;
    constexpr int kBatchCb = V == 4 ? 4 : 1;  // positions whose loads are issued together (bf16: registers)
    using raw = typename IO::raw;
    extern __shared__ float red[];  // [G][6][VEs V]
    const int tid = threadIdx.x, c = tid % VEs, g = tid / VEs;
    const int vc = blockIdx.y * VEs + c;  // vector lane of the channel dimension
    const bool act = g < G && vc < VE;
    const int coff = vc * V;
    const int n = h * w;
    const int run = (P + G - 1) / G;
    float aD[V], aB[V], aW[V][kTaps];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        aD[v] = aB[v] = 0.f;
#pragma unroll
        for (int k = 0; k < kTaps; ++k) aW[v][k] = 0.f;
    }
    if (act) {
        ConvW<V> W;
        load_conv_w<V>(cw, cb, coff, W);
        float dsum[V];
#pragma unroll
        for (int v = 0; v < V; ++v) dsum[v] = Df[coff + v] + Db[coff + v];
        // token (within the image) of sequence position q
        auto tok_of = [&](int q) { return COLS ? q : (q % h) * w + q / h; };
        for (int64_t item = blockIdx.x; item < (int64_t)B * T; item += gridDim.x) {
            const int64_t b = item / T;
            const int t = (int)(item - b * T);
            const int ra = t * P + g * run;
            const int rb = ra + run < (t + 1) * P ? ra + run : (t + 1) * P;
            if (ra >= rb) continue;
            const int64_t img = b * (int64_t)n * E;
            float sv[V];
#pragma unroll
            for (int v = 0; v < V; v += 4) {
                const f32x4 q1 = load_raw<false>(sf + (b * T + t) * E + coff + v);
                const f32x4 q2 = load_raw<false>(sb + (b * T + t) * E + coff + v);
                sv[v] = q1.x + q2.x;
                sv[v + 1] = q1.y + q2.y;
                sv[v + 2] = q1.z + q2.z;
                sv[v + 3] = q1.w + q2.w;
            }
            const float* ur = du + (b * T + t) * E + coff;
            float uv[V];  // du / P at scan position t (the run's cells)
#pragma unroll
            for (int v = 0; v < V; ++v) uv[v] = ur[v] * inv_p;
            auto pos = [&](int q) { return img + (int64_t)tok_of(q) * E + coff; };
            raw x3{}, x2{}, x1{};  // x[q - 3 .. q - 1]
            if (ra >= 3) x3 = load_raw<false>(x + pos(ra - 3));
            if (ra >= 2) x2 = load_raw<false>(x + pos(ra - 2));
            if (ra >= 1) x1 = load_raw<false>(x + pos(ra - 1));
            float d3[V], d2[V], d1[V];  // da[q - 3 .. q - 1]
#pragma unroll
            for (int v = 0; v < V; ++v) d3[v] = d2[v] = d1[v] = 0.f;
            // dx[q - 3] from da[q - 3 .. q] (q - 3 in the run), then the rings move on
            auto finish = [&](const raw& xv, const float (&da)[V], int q) {
                if (q - 3 >= ra) {
                    float ox[V];
#pragma unroll
                    for (int v = 0; v < V; ++v)
                        ox[v] = fmaf(W.w[v][0], da[v], fmaf(W.w[v][1], d1[v], fmaf(W.w[v][2], d2[v], W.w[v][3] * d3[v])));
                    store_vec<true>(dx + pos(q - 3), ox);
                }
                x3 = x2;
                x2 = x1;
                x1 = xv;
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    d3[v] = d2[v];
                    d2[v] = d1[v];
                    d1[v] = da[v];
                }
            };
            // position q at the front: da[q]; for the run's own positions also
            // dz[q] and the sums (those past the run only feed dx behind them)
            auto step = [&](const raw& xv, const raw& zr, const raw& orw, const float (&uq)[V], int q, bool own) {
                float da[V], oz[V];
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    float a = fmaf(W.w[v][3], raw_at(xv, v), W.b[v]);
                    a = fmaf(W.w[v][2], raw_at(x1, v), a);
                    a = fmaf(W.w[v][1], raw_at(x2, v), a);
                    a = fmaf(W.w[v][0], raw_at(x3, v), a);
                    const float sga = __builtin_amdgcn_rcpf(1.f + __expf(-a));
                    const float zv = raw_at(zr, v), dv = raw_at(orw, v);
                    const float sgz = __builtin_amdgcn_rcpf(1.f + __expf(-zv));
                    const float gv = dv * zv * sgz;
                    const float dxc = fmaf(gv, dsum[v], uq[v]);
                    da[v] = dxc * sga * fmaf(a, 1.f - sga, 1.f);
                    if (own) {
                        const float xc = a * sga;
                        oz[v] = dv * fmaf(dsum[v], xc, sv[v]) * sgz * fmaf(zv, 1.f - sgz, 1.f);
                        aD[v] = fmaf(gv, xc, aD[v]);
                        aB[v] += da[v];
                        aW[v][0] = fmaf(da[v], raw_at(x3, v), aW[v][0]);
                        aW[v][1] = fmaf(da[v], raw_at(x2, v), aW[v][1]);
                        aW[v][2] = fmaf(da[v], raw_at(x1, v), aW[v][2]);
                        aW[v][3] = fmaf(da[v], raw_at(xv, v), aW[v][3]);
                    }
                }
                if (own) store_vec<true>(dz + pos(q), oz);
                finish(xv, da, q);
            };
            // the run's positions, kBatchCb at a time with all their loads first
            int q = ra;
            for (; q + kBatchCb <= rb; q += kBatchCb) {
                raw xf[kBatchCb], zf[kBatchCb], of[kBatchCb];
#pragma unroll
                for (int i = 0; i < kBatchCb; ++i) {
                    const int64_t o = pos(q + i);
                    xf[i] = load_raw<false>(x + o);
                    zf[i] = load_raw<false>(z + o);
                    of[i] = load_raw<false>(dout + o);
                }
#pragma unroll
                for (int i = 0; i < kBatchCb; ++i) step(xf[i], zf[i], of[i], uv, q + i, true);
            }
            for (; q < rb; ++q) {
                const int64_t o = pos(q);
                const raw xv = load_raw<false>(x + o), zv = load_raw<false>(z + o), ov = load_raw<false>(dout + o);
                step(xv, zv, ov, uv, q, true);
            }
            // three positions past the run (da = 0 past the sequence); the last
            // run of a scan position reaches into the next one
            for (; q < rb + 3; ++q) {
                if (q < n) {
                    const int64_t o = pos(q);
                    const raw xv = load_raw<false>(x + o), zv = load_raw<false>(z + o),
                              ov = load_raw<false>(dout + o);
                    const float* uq = du + (b * T + q / P) * E + coff;
                    float un[V];
#pragma unroll
                    for (int v = 0; v < V; ++v) un[v] = uq[v] * inv_p;
                    step(xv, zv, ov, un, q, false);
                } else {
                    float da[V];
#pragma unroll
                    for (int v = 0; v < V; ++v) da[v] = 0.f;
                    finish(raw{}, da, q);
                }
            }
        }
    }
    // the workgroup's partial row: groups added through LDS in a fixed order
    const int width = VEs * V;
    if (g < G) {
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float* rg = red + (int64_t)g * 6 * width + c * V + v;
            rg[0] = aD[v];
            rg[width] = aB[v];
#pragma unroll
            for (int k = 0; k < kTaps; ++k) rg[(2 + k) * width] = aW[v][k];
        }
    }
    __syncthreads();
    float* prow = parts + (int64_t)blockIdx.x * 6 * E;
    const int col0 = blockIdx.y * VEs * V;
    for (int o = tid; o < 6 * width; o += blockDim.x) {
        const int k = o / width, cc = o - k * width;
        if (col0 + cc >= E) continue;
        float s = red[o];
        for (int gg = 1; gg < G; ++gg) s += red[(int64_t)gg * 6 * width + o];
        if (k < 2) prow[k * E + col0 + cc] = s;
        else prow[2 * E + (col0 + cc) * kTaps + (k - 2)] = s;
    }
}

template <class IO>
hipError_t bwd_conv_epi_t(const Geom& g, const void* x, const void* z, const void* dout, const fastvim_params& p,
                          const float* sf, const float* sb, const float* du, float* parts, int64_t nparts, void* dx,
                          void* dz, hipStream_t st) {
    using elem = typename IO::elem;
    const int VE = (int)(g.E / IO::V);
    const int nsl = (VE + kCbSlice - 1) / kCbSlice;  // channel slices of equal width
    const int VEs = (VE + nsl - 1) / nsl;
    int G = kCbThreads / VEs;
    if (G > g.P) G = (int)g.P;
    if (G < 1) G = 1;
    const int threads = (VEs * G + 63) / 64 * 64;
    const dim3 grid((unsigned)nparts, (unsigned)nsl);
    const size_t lds = (size_t)G * 6 * VEs * IO::V * sizeof(float);
    const auto* xe = static_cast<const elem*>(x);
    const auto* ze = static_cast<const elem*>(z);
    const auto* de = static_cast<const elem*>(dout);
    auto* dxe = static_cast<elem*>(dx);
    auto* dze = static_cast<elem*>(dz);
    if (g.axis == FASTVIM_POOL_COLS)
        hipLaunchKernelGGL((bwd_conv_epilogue_kernel<IO, true>), grid, dim3(threads), lds, st, xe, ze, de, p.conv_w,
                           p.conv_b, sf, sb, du, p.fwd.D, p.bwd.D, dxe, dze, parts, (int)g.B, (int)g.T, (int)g.P,
                           (int)g.h, (int)g.w, (int)g.E, VE, VEs, G, pool_norm(g));
    else
        hipLaunchKernelGGL((bwd_conv_epilogue_kernel<IO, false>), grid, dim3(threads), lds, st, xe, ze, de,
                           p.conv_w, p.conv_b, sf, sb, du, p.fwd.D, p.bwd.D, dxe, dze, parts, (int)g.B, (int)g.T,
                           (int)g.P, (int)g.h, (int)g.w, (int)g.E, VE, VEs, G, pool_norm(g));
    return hipGetLastError();
}

}  // namespace

int64_t bwd_conv_parts(const Geom& g) {
    const int64_t items = g.B * g.T, cap = 32 * g.B;
    return items < cap ? items : cap;
}

hipError_t launch_bwd_conv_epilogue(const Geom& g, const void* x, const void* z, const void* dout,
                                    const fastvim_params& p, const float* sf, const float* sb, const float* du,
                                    float* parts, void* dx, void* dz, hipStream_t st) {
    const int64_t np = bwd_conv_parts(g);
    return g.io == FASTVIM_BF16 ? bwd_conv_epi_t<IoBf16>(g, x, z, dout, p, sf, sb, du, parts, np, dx, dz, st)
                                : bwd_conv_epi_t<IoF32>(g, x, z, dout, p, sf, sb, du, parts, np, dx, dz, st);
}

}  // namespace fastvim
