// The producer Conv1D + SiLU written out once, and its adjoint, for the
// layers whose stages cannot slide the conv window where they read x: masked
// layers (the conv runs along the kept tokens as given), layers with the
// post-SSM LayerNorm (whose output stage takes whole tokens) and unpooled
// layers.  The layer then runs unchanged on x_conv.
//
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解,
// bullets 1-2 (the grid is pooled after the Conv1D) and 6 (FastMaskVim on the
// kept tokens); Vim article (ijyty.com) 2.1 (conv1d, then the SSM).  With r
// the position in the sequence -- the oriented grid's row-major (COLS,
// NONE_ROWMAJOR) or column-major (ROWS, NONE_COLMAJOR) order, or the kept
// tokens k = 0 .. K-1 of a masked layer -- and zeros before its start:
//   x_conv[r, e] = silu(conv_b[e] + sum_{k<4} conv_w[e, k] x[r - 3 + k, e])
// and, with dxc = dL/dx_conv, a[r] the pre-activation and da = dxc silu'(a):
//   dx[r] = sum_k conv_w[k] da[r + 3 - k],  d conv_w[k] = sum_r da[r] x[r - 3 + k],
//   d conv_b = sum_r da[r].
//
// Work unit: a run of L consecutive sequence positions of one image for one
// 16-byte channel vector; a lane slides a window of three raw vectors along
// its run (so each token is loaded once, plus a halo of three at the start).
// The adjoint works in place: dxc arrives in the dx buffer and dx[r] replaces
// it three positions behind the front that reads dxc.  Its reads past the
// end of a run (the next run's first three positions) would race with the
// next run's writes, so a pre-pass stores da at the first three positions of
// every run into a halo buffer and the adjoint takes them from there.
#include "bwd_internal.h"
#include "conv_common.h"

namespace fastvim {
namespace {

constexpr int kSeqThreads = 256;
constexpr int kAdjRunsPerSlot = 4;  // runs per adjoint workgroup slot

__device__ __forceinline__ int seq_token(int r, int h, int w, bool colmajor) {
    return colmajor ? (r % h) * w + r / h : r;
}

// x_conv of the runs of L positions, one (image, run, vector) per thread.
template <class IO>
__global__ void __launch_bounds__(kSeqThreads)
conv_seq_kernel(const typename IO::elem* x, typename IO::elem* xc, const float* __restrict__ cw,
                const float* __restrict__ cb, int n, int h, int w, int colmajor, int E, int VE, int L, int nruns,
                int64_t items) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    const int64_t gi = (int64_t)blockIdx.x * kSeqThreads + threadIdx.x;
    if (gi >= items) return;
    const int c = (int)(gi % VE);
    const int64_t br = gi / VE;
    const int64_t b = br / nruns;
    const int run = (int)(br - b * nruns);
    const int r0 = run * L, r1 = r0 + L < n ? r0 + L : n;
    const bool cm = colmajor != 0;
    const int coff = c * V;
    const typename IO::elem* xb = x + b * (int64_t)n * E;
    typename IO::elem* ob = xc + b * (int64_t)n * E;
    ConvW<V> W;
    load_conv_w<V>(cw, cb, coff, W);
    raw p3{}, p2{}, p1{};
    if (r0 >= 3) p3 = load_raw<false>(xb + (seq_token(r0 - 3, h, w, cm) * E + coff));
    if (r0 >= 2) p2 = load_raw<false>(xb + (seq_token(r0 - 2, h, w, cm) * E + coff));
    if (r0 >= 1) p1 = load_raw<false>(xb + (seq_token(r0 - 1, h, w, cm) * E + coff));
    for (int r = r0; r < r1; r += 4) {
        raw cur[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (r + q < r1) cur[q] = load_raw<false>(xb + (seq_token(r + q, h, w, cm) * E + coff));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (r + q < r1) {
                float o[V];
                conv_window<IO>(p3, p2, p1, cur[q], W, o);
                store_vec<false>(ob + (seq_token(r + q, h, w, cm) * E + coff), o);
                p3 = p2;
                p2 = p1;
                p1 = cur[q];
            }
        }
    }
}

// da = dxc silu'(a) at the first three positions of every run after the
// first of its image, into halo[(b nruns + run) 3 + p][E] (fp32).
template <class IO>
__global__ void __launch_bounds__(kSeqThreads)
conv_adjoint_halo_kernel(const typename IO::elem* x, const typename IO::elem* dxc, const float* __restrict__ cw,
                         const float* __restrict__ cb, float* __restrict__ halo, int n, int h, int w, int colmajor,
                         int E, int VE, int L, int nruns, int64_t items) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    const int64_t gi = (int64_t)blockIdx.x * kSeqThreads + threadIdx.x;
    if (gi >= items) return;
    const int c = (int)(gi % VE);
    const int64_t br = gi / VE;
    const int64_t b = br / nruns;
    const int run = (int)(br - b * nruns);
    if (run == 0) return;
    const bool cm = colmajor != 0;
    const int coff = c * V;
    const typename IO::elem* xb = x + b * (int64_t)n * E;
    const typename IO::elem* gb = dxc + b * (int64_t)n * E;
    ConvW<V> W;
    load_conv_w<V>(cw, cb, coff, W);
    const int r0 = run * L;  // >= L >= 4: every window position lies inside the sequence
    raw win[6];
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        win[k] = raw{};
        if (r0 - 3 + k < n) win[k] = load_raw<false>(xb + (seq_token(r0 - 3 + k, h, w, cm) * E + coff));
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const int r = r0 + p;
        if (r >= n) break;
        const raw gr = load_raw<false>(gb + (seq_token(r, h, w, cm) * E + coff));
        float* dst = halo + ((br * 3 + p) * E + coff);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float a = fmaf(W.w[v][3], raw_at(win[p + 3], v), W.b[v]);
            a = fmaf(W.w[v][2], raw_at(win[p + 2], v), a);
            a = fmaf(W.w[v][1], raw_at(win[p + 1], v), a);
            a = fmaf(W.w[v][0], raw_at(win[p], v), a);
            dst[v] = raw_at(gr, v) * conv_silu_grad(a);
        }
    }
}

// The adjoint, in place.  Workgroup (group g, channel block cb) of k slots of
// VB lanes (VB = min(VE, 256) vectors of a token, k = 256 / VB): lane l of
// slot q takes vector cb VB + l and the runs g k R + q + k i (R =
// kAdjRunsPerSlot), so every lane has work whatever E is.  A lane walks its run with a front f: at f it
// loads x and dxc and forms da[f] (past the run, da comes from the halo
// buffer, past the sequence it is 0), adds the conv's weight and bias
// gradient terms, and writes dx[f - 3] from da[f - 3 .. f].  dxc is read only
// at positions whose dx is written later by the same lane.  At the end the k
// slots' sums are added in LDS in a fixed order and the workgroup writes its
// slice of partial row g: [d conv_b (E) | d conv_w (E, 4)].
template <class IO>
__global__ void __launch_bounds__(kSeqThreads)
conv_adjoint_kernel(const typename IO::elem* x, typename IO::elem* dx, const float* __restrict__ cw,
                    const float* __restrict__ cb, const float* __restrict__ halo, float* __restrict__ parts, int n,
                    int h, int w, int colmajor, int E, int VE, int VB, int L, int nruns, int64_t total_runs) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    extern __shared__ float red[];  // [k][VB][5 V]
    const int k = (int)blockDim.x / VB;
    const int slot = (int)threadIdx.x / VB, lane = (int)threadIdx.x - slot * VB;
    const int c = (int)blockIdx.y * VB + lane;
    const bool valid = c < VE;
    const int coff = (valid ? c : VE - 1) * V;
    const bool cm = colmajor != 0;
    ConvW<V> W;
    load_conv_w<V>(cw, cb, coff, W);
    float sdb[V], sdw[4][V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        sdb[v] = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) sdw[k][v] = 0.f;
    }
    const int64_t rpg = (int64_t)k * kAdjRunsPerSlot;  // runs per workgroup
    const int64_t run_end = ((int64_t)blockIdx.x + 1) * rpg < total_runs ? ((int64_t)blockIdx.x + 1) * rpg
                                                                         : total_runs;
    for (int64_t run = (int64_t)blockIdx.x * rpg + slot; run < run_end; run += k) {
        const int64_t b = run / nruns;
        const int j = (int)(run - b * nruns);
        const int r0 = j * L, r1 = r0 + L < n ? r0 + L : n;
        const typename IO::elem* xb = x + b * (int64_t)n * E;
        typename IO::elem* gb = dx + b * (int64_t)n * E;
        const float* hb = halo + ((run + 1) * 3 * E + coff);  // the next run's first three positions
        raw p3{}, p2{}, p1{};
        if (r0 >= 3) p3 = load_raw<false>(xb + (seq_token(r0 - 3, h, w, cm) * E + coff));
        if (r0 >= 2) p2 = load_raw<false>(xb + (seq_token(r0 - 2, h, w, cm) * E + coff));
        if (r0 >= 1) p1 = load_raw<false>(xb + (seq_token(r0 - 1, h, w, cm) * E + coff));
        float d3[V], d2[V], d1[V];
#pragma unroll
        for (int v = 0; v < V; ++v) d3[v] = d2[v] = d1[v] = 0.f;
        for (int f0 = r0; f0 < r1 + 3; f0 += 4) {
            // this batch's loads first: dxc at f0 .. f0 + 3 precedes every store
            // of the batch (they reach at most position f0)
            raw xf[4], gf[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (f0 + q < r1) {
                    const int off = seq_token(f0 + q, h, w, cm) * E + coff;
                    xf[q] = load_raw<false>(xb + off);
                    gf[q] = load_raw<false>(gb + off);
                }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int f = f0 + q;
                if (f >= r1 + 3) break;
                float da[V];
                if (f < r1) {
#pragma unroll
                    for (int v = 0; v < V; ++v) {
                        const float x0 = raw_at(p3, v), x1 = raw_at(p2, v), x2 = raw_at(p1, v),
                                    x3 = raw_at(xf[q], v);
                        float a = fmaf(W.w[v][3], x3, W.b[v]);
                        a = fmaf(W.w[v][2], x2, a);
                        a = fmaf(W.w[v][1], x1, a);
                        a = fmaf(W.w[v][0], x0, a);
                        da[v] = raw_at(gf[q], v) * conv_silu_grad(a);
                        sdb[v] += da[v];
                        sdw[0][v] = fmaf(da[v], x0, sdw[0][v]);
                        sdw[1][v] = fmaf(da[v], x1, sdw[1][v]);
                        sdw[2][v] = fmaf(da[v], x2, sdw[2][v]);
                        sdw[3][v] = fmaf(da[v], x3, sdw[3][v]);
                    }
                    p3 = p2;
                    p2 = p1;
                    p1 = xf[q];
                } else {
#pragma unroll
                    for (int v = 0; v < V; ++v) da[v] = f < n ? hb[(f - r1) * E + v] : 0.f;
                }
                const int back = f - 3;
                if (back >= r0 && valid) {
                    float o[V];
#pragma unroll
                    for (int v = 0; v < V; ++v)
                        o[v] = fmaf(W.w[v][0], da[v], fmaf(W.w[v][1], d1[v], fmaf(W.w[v][2], d2[v], W.w[v][3] * d3[v])));
                    store_vec<false>(gb + (seq_token(back, h, w, cm) * E + coff), o);
                }
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    d3[v] = d2[v];
                    d2[v] = d1[v];
                    d1[v] = da[v];
                }
            }
        }
    }
    if (slot > 0) {
        float* mine = red + ((slot - 1) * VB + lane) * 5 * V;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            mine[v] = sdb[v];
#pragma unroll
            for (int t = 0; t < 4; ++t) mine[V + 4 * v + t] = sdw[t][v];
        }
    }
    __syncthreads();
    if (slot == 0 && valid) {
        float* row = parts + (int64_t)blockIdx.x * 5 * E;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float s = sdb[v];
            for (int u = 1; u < k; ++u) s += red[((u - 1) * VB + lane) * 5 * V + v];
            row[coff + v] = s;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float q = sdw[t][v];
                for (int u = 1; u < k; ++u) q += red[((u - 1) * VB + lane) * 5 * V + V + 4 * v + t];
                row[E + (coff + v) * 4 + t] = q;
            }
        }
    }
}

struct SeqGeom {
    int n, colmajor;
};

SeqGeom seq_geom(const Geom& g) {
    if (g.masked) return SeqGeom{(int)g.K, 0};
    const bool cm = g.axis == FASTVIM_POOL_ROWS || g.axis == FASTVIM_POOL_NONE_COLMAJOR;
    return SeqGeom{(int)(g.h * g.w), cm ? 1 : 0};
}

constexpr int kSeqRun = 64;  // positions per run of the forward conv

template <class IO>
hipError_t conv_seq_t(const Geom& g, const void* x, const fastvim_params& p, void* xc, hipStream_t st) {
    const SeqGeom s = seq_geom(g);
    const int VE = (int)(g.E / IO::V);
    const int nruns = (s.n + kSeqRun - 1) / kSeqRun;
    const int64_t items = g.B * nruns * (int64_t)VE;
    hipLaunchKernelGGL((conv_seq_kernel<IO>), dim3((unsigned)((items + kSeqThreads - 1) / kSeqThreads)),
                       dim3(kSeqThreads), 0, st, static_cast<const typename IO::elem*>(x),
                       static_cast<typename IO::elem*>(xc), p.conv_w, p.conv_b, s.n, (int)g.h, (int)g.w, s.colmajor,
                       (int)g.E, VE, kSeqRun, nruns, items);
    return hipGetLastError();
}

// Vectors per slot of an adjoint workgroup, and its slots.
int adjoint_vb(const Geom& g) {
    const int VE = (int)(g.E / (g.io == FASTVIM_BF16 ? IoBf16::V : IoF32::V));
    return VE < kSeqThreads ? VE : kSeqThreads;
}
int adjoint_slots(const Geom& g) { return kSeqThreads / adjoint_vb(g); }

// Run length of the adjoint whose halo, partial rows and column-sum scratch
// fit in `floats`: the shortest of 64, 128, ... (a whole sequence as one run
// needs no halo).  *groups: partial rows.
int adjoint_run(const Geom& g, int64_t floats, int64_t* groups) {
    const SeqGeom s = seq_geom(g);
    const int64_t rpg = (int64_t)adjoint_slots(g) * kAdjRunsPerSlot;
    for (int L = 64;; L *= 2) {
        if (L > s.n) L = s.n;
        const int64_t nruns = (s.n + L - 1) / L;
        const int64_t gr = (g.B * nruns + rpg - 1) / rpg;
        const int64_t need = (nruns > 1 ? g.B * nruns * 3 * g.E : 0) + gr * 5 * g.E +
                             ((gr + kColRowsPerBlock - 1) / kColRowsPerBlock) * 4 * g.E + 64;
        if (need <= floats || L >= s.n) {
            *groups = gr;
            return need <= floats ? L : 0;
        }
    }
}

template <class IO>
hipError_t conv_adjoint_t(const Geom& g, const void* x, void* dx, const fastvim_params& p, float* scratch,
                          int64_t floats, float* dcw, float* dcb, hipStream_t st) {
    using elem = typename IO::elem;
    const SeqGeom s = seq_geom(g);
    int64_t groups = 0;
    const int L = adjoint_run(g, floats, &groups);
    if (L == 0) return hipErrorInvalidValue;  // cannot happen: the backward workspace holds a partial row per image
    const int VE = (int)(g.E / IO::V);
    const int nruns = (s.n + L - 1) / L;
    const int64_t total_runs = g.B * nruns;
    float* halo = scratch;
    float* parts = halo + (nruns > 1 ? total_runs * 3 * g.E : 0);
    float* tmp = parts + groups * 5 * g.E;
    const elem* xe = static_cast<const elem*>(x);
    elem* de = static_cast<elem*>(dx);
    if (nruns > 1) {
        const int64_t items = total_runs * VE;
        hipLaunchKernelGGL((conv_adjoint_halo_kernel<IO>), dim3((unsigned)((items + kSeqThreads - 1) / kSeqThreads)),
                           dim3(kSeqThreads), 0, st, xe, static_cast<const elem*>(dx), p.conv_w, p.conv_b, halo, s.n,
                           (int)g.h, (int)g.w, s.colmajor, (int)g.E, VE, L, nruns, items);
    }
    const int VB = adjoint_vb(g), slots = adjoint_slots(g);
    const size_t lds = (size_t)((slots - 1) * VB * 5 * IO::V) * sizeof(float);
    hipLaunchKernelGGL((conv_adjoint_kernel<IO>), dim3((unsigned)groups, (unsigned)((VE + VB - 1) / VB)),
                       dim3((unsigned)(slots * VB)), lds, st, xe, de, p.conv_w, p.conv_b, halo, parts, s.n, (int)g.h,
                       (int)g.w, s.colmajor, (int)g.E, VE, VB, L, nruns, total_runs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((e = launch_colsum(parts, groups, g.E, 5 * g.E, dcb, nullptr, tmp, st)) != hipSuccess) return e;
    return launch_colsum(parts + g.E, groups, 4 * g.E, 5 * g.E, dcw, nullptr, tmp, st);
}

}  // namespace

hipError_t launch_conv_seq(const Geom& g, const void* x, const fastvim_params& p, void* xc, hipStream_t st) {
    return g.io == FASTVIM_BF16 ? conv_seq_t<IoBf16>(g, x, p, xc, st) : conv_seq_t<IoF32>(g, x, p, xc, st);
}

hipError_t launch_conv_adjoint(const Geom& g, const void* x, void* dx, const fastvim_params& p, float* scratch,
                               int64_t floats, float* dcw, float* dcb, hipStream_t st) {
    return g.io == FASTVIM_BF16 ? conv_adjoint_t<IoBf16>(g, x, dx, p, scratch, floats, dcw, dcb, st)
                                : conv_adjoint_t<IoF32>(g, x, dx, p, scratch, floats, dcw, dcb, st);
}

bool conv_adjoint_fits(const Geom& g, int64_t floats) {
    int64_t groups = 0;
    return adjoint_run(g, floats, &groups) > 0;
}

}  // namespace fastvim
