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
// The sequence of an image is cut into lines -- the grid rows of a row-major
// sequence, the grid columns of a column-major one (a masked sequence is one
// line) -- so that a pooled layer's scan position is the line, and each line
// into runs of at most L positions.  Work unit: a run of one image for one
// 16-byte channel vector; a lane slides a window of three raw vectors along
// its run with a fixed stride between positions (so each token is loaded
// once, plus a halo of three at the start).  Lanes next to each other take
// the channel vectors of one token; runs next to each other in the launch are
// next to each other in memory (the runs of a grid row, or the same run of
// neighbouring columns).
// The adjoint works in place: dxc arrives in the dx buffer and dx[r] replaces
// it three positions behind the front that reads dxc.  A lane walks a chunk
// of consecutive runs as one; its reads past the chunk's end (the next
// chunk's first three positions) would race with that chunk's writes, so a
// pre-pass stores da at the first three positions of every chunk into a halo
// buffer and the adjoint takes them from there.
#include "bwd_internal.h"
#include "conv_common.h"

namespace fastvim {
namespace {

constexpr int kSeqThreads = 256;
constexpr int kAdjRunsPerSlot = 4;  // runs per adjoint workgroup slot (one chunk)
constexpr int kBatch = 4;           // positions whose loads are issued together

// An image's sequence as lines of runs (element offsets within the image).
struct SeqShape {
    int n;           // positions
    int len;         // positions per line (the last line may be shorter only when lines == 1)
    int lines;
    int L;           // positions per run
    int nk;          // runs per line
    int colmajor;    // conv_seq_kernel: runs of neighbouring lines are neighbours in the launch
    int64_t pstride; // elements from one position of a line to the next
    int64_t lstride; // elements from one line's first position to the next line's

    __host__ __device__ int64_t runs() const { return (int64_t)lines * nk; }
    // element offset of sequence position r (0 <= r < n)
    __device__ int64_t off(int r) const { return (int64_t)(r / len) * lstride + (int64_t)(r % len) * pstride; }
    // sequence-order index (line nk + k) of the launch's run u within an image
    __device__ void run_of(int64_t u, int* line, int* k) const {
        if (colmajor) {
            *line = (int)(u % lines);
            *k = (int)(u / lines);
        } else {
            *line = (int)(u / nk);
            *k = (int)(u % nk);
        }
    }
};

SeqShape seq_shape(const Geom& g, int L) {
    SeqShape s{};
    const int64_t E = g.E;
    if (g.masked) {
        s.n = s.len = (int)g.K;
        s.lines = 1;
        s.pstride = E;
        s.lstride = s.n * E;
    } else if (g.axis == FASTVIM_POOL_ROWS || g.axis == FASTVIM_POOL_NONE_COLMAJOR) {
        s.n = (int)(g.h * g.w);
        s.len = (int)g.h;
        s.lines = (int)g.w;
        s.colmajor = 1;
        s.pstride = g.w * E;
        s.lstride = E;
    } else {
        s.n = (int)(g.h * g.w);
        s.len = (int)g.w;
        s.lines = (int)g.h;
        s.pstride = E;
        s.lstride = g.w * E;
    }
    s.L = L < s.len ? L : s.len;
    s.nk = (s.len + s.L - 1) / s.L;
    return s;
}

// The conv's output gradient dxc at one cell from the vector the dx buffer
// holds there: dxc itself, or (FROM_G, a dense pooled layer with the
// post-SSM LayerNorm whose second pass was left to the adjoint) the norm's
// g, from which dxc = g (D_fwd + D_bwd) + du[b, t] inv_p, t the scan
// position (the cell's line).  ds = D_fwd + D_bwd and u = du[b, t] of the
// lane's channels.
template <int V, bool FROM_G>
__device__ __forceinline__ void du_row(const DxcFromG& fg, int64_t b, int t, int E, int coff, float (&u)[V]) {
#pragma unroll
    for (int v = 0; v < V; ++v) u[v] = 0.f;
    if (FROM_G) {
        const float* ur = fg.du + (b * fg.T + t) * E + coff;
#pragma unroll
        for (int v = 0; v < V; ++v) u[v] = ur[v];
    }
}
template <int V, bool FROM_G>
__device__ __forceinline__ void dsum_of(const DxcFromG& fg, int coff, float (&ds)[V]) {
#pragma unroll
    for (int v = 0; v < V; ++v) ds[v] = FROM_G ? fg.Df[coff + v] + fg.Db[coff + v] : 0.f;
}
template <class IO, bool FROM_G>
__device__ __forceinline__ float dxc_at(const typename IO::raw& r, int v, const float (&u)[IO::V],
                                        const float (&ds)[IO::V], float inv_p) {
    return FROM_G ? fmaf(raw_at(r, v), ds[v], u[v] * inv_p) : raw_at(r, v);
}

// x_conv, one (image, run, vector) per thread.
template <class IO>
__global__ void __launch_bounds__(kSeqThreads)
conv_seq_kernel(const typename IO::elem* x, typename IO::elem* xc, const float* __restrict__ cw,
                const float* __restrict__ cb, SeqShape sq, int E, int VE, int64_t items) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    const int64_t gi = (int64_t)blockIdx.x * kSeqThreads + threadIdx.x;
    if (gi >= items) return;
    const int c = (int)(gi % VE);
    const int64_t br = gi / VE;
    const int64_t b = br / sq.runs();
    int line, k;
    sq.run_of(br - b * sq.runs(), &line, &k);
    const int r0 = line * sq.len + k * sq.L;
    const int cnt = min(sq.L, sq.len - k * sq.L);
    const int coff = c * V;
    const typename IO::elem* xb = x + b * (int64_t)sq.n * E + coff;
    typename IO::elem* ob = xc + b * (int64_t)sq.n * E + coff;
    ConvW<V> W;
    load_conv_w<V>(cw, cb, coff, W);
    raw p3{}, p2{}, p1{};
    if (r0 >= 3) p3 = load_raw<false>(xb + sq.off(r0 - 3));
    if (r0 >= 2) p2 = load_raw<false>(xb + sq.off(r0 - 2));
    if (r0 >= 1) p1 = load_raw<false>(xb + sq.off(r0 - 1));
    const int64_t ps = sq.pstride;
    const typename IO::elem* xp = xb + sq.off(r0);
    typename IO::elem* op = ob + sq.off(r0);
    auto step = [&](const raw& cur, int f) {
        float o[V];
        conv_window<IO>(p3, p2, p1, cur, W, o);
        store_vec<false>(op + f * ps, o);
        p3 = p2;
        p2 = p1;
        p1 = cur;
    };
    int f0 = 0;
    for (; f0 + kBatch <= cnt; f0 += kBatch) {
        raw cur[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) cur[q] = load_raw<false>(xp + (f0 + q) * ps);
#pragma unroll
        for (int q = 0; q < kBatch; ++q) step(cur[q], f0 + q);
    }
    for (int f = f0; f < cnt; ++f) step(load_raw<false>(xp + f * ps), f);
}

// da = dxc silu'(a) at the first three positions of every run that starts an
// adjoint slot's chunk (global run index U = c kAdjRunsPerSlot) but an
// image's first, into halo[c 3 + p][E] (fp32).
template <class IO, bool FROM_G>
__global__ void __launch_bounds__(kSeqThreads)
conv_adjoint_halo_kernel(const typename IO::elem* x, const typename IO::elem* dxc, const float* __restrict__ cw,
                         const float* __restrict__ cb, float* __restrict__ halo, SeqShape sq, int E, int VE,
                         int64_t items, int64_t total_runs, DxcFromG fg) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    const int64_t gi = (int64_t)blockIdx.x * kSeqThreads + threadIdx.x;
    if (gi >= items) return;
    const int c = (int)(gi % VE);
    const int64_t ci = gi / VE;  // chunk
    const int64_t U = ci * kAdjRunsPerSlot;
    if (U >= total_runs) return;
    const int64_t b = U / sq.runs();
    const int64_t sr = U - b * sq.runs();  // sequence-order run within the image
    if (sr == 0) return;
    const int line = (int)(sr / sq.nk), k = (int)(sr - (int64_t)line * sq.nk);
    const int r0 = line * sq.len + k * sq.L;  // >= 1
    const int coff = c * V;
    const typename IO::elem* xb = x + b * (int64_t)sq.n * E + coff;
    const typename IO::elem* gb = dxc + b * (int64_t)sq.n * E + coff;
    ConvW<V> W;
    load_conv_w<V>(cw, cb, coff, W);
    float ds[V];
    dsum_of<V, FROM_G>(fg, coff, ds);
    raw win[6];
#pragma unroll
    for (int q = 0; q < 6; ++q) {
        win[q] = raw{};
        const int r = r0 - 3 + q;
        if (r >= 0 && r < sq.n) win[q] = load_raw<false>(xb + sq.off(r));
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        const int r = r0 + p;
        if (r >= sq.n) break;
        const raw gr = load_raw<false>(gb + sq.off(r));
        float u[V];
        du_row<V, FROM_G>(fg, b, r / sq.len, E, coff, u);
        float* dst = halo + ((ci * 3 + p) * E + coff);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float a = fmaf(W.w[v][3], raw_at(win[p + 3], v), W.b[v]);
            a = fmaf(W.w[v][2], raw_at(win[p + 2], v), a);
            a = fmaf(W.w[v][1], raw_at(win[p + 1], v), a);
            a = fmaf(W.w[v][0], raw_at(win[p], v), a);
            dst[v] = dxc_at<IO, FROM_G>(gr, v, u, ds, fg.inv_p) * conv_silu_grad(a);
        }
    }
}

// The adjoint, in place.  Workgroup (group g, channel block cb) of k slots of
// VB lanes (VB = min(VE, 256) vectors of a token, k = 256 / VB): lane l of
// slot q takes vector cb VB + l and the chunk of R = kAdjRunsPerSlot runs
// g k R + q R + i, i < R, which are consecutive in sequence order, so every
// lane has work whatever E is.  A lane walks its chunk with a front f: at f it
// loads x and dxc and forms da[f], adds the conv's weight and bias gradient
// terms, and writes dx[f - 3] from da[f - 3 .. f].  The walk goes on from one
// run of the chunk into the next (the windows carry over); past the chunk's
// last run da comes from the halo buffer (0 past the sequence).  dxc is read
// only at positions whose dx is written later by the same lane.  At the end
// the k slots' sums are added in LDS in a fixed order and the workgroup writes
// its slice of partial row g: [d conv_b (E) | d conv_w (E, 4)].
template <class IO, bool FROM_G>
__global__ void __launch_bounds__(kSeqThreads)
conv_adjoint_kernel(const typename IO::elem* x, typename IO::elem* dx, const float* __restrict__ cw,
                    const float* __restrict__ cb, const float* __restrict__ halo, float* __restrict__ parts,
                    SeqShape sq, int E, int VE, int VB, int64_t total_runs, DxcFromG fg) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    constexpr int kB = V == 4 ? kBatch : 1;  // positions per batch (bf16: registers)
    extern __shared__ float red[];  // [k][VB][5 V]
    const int k = (int)blockDim.x / VB;
    const int slot = (int)threadIdx.x / VB, lane = (int)threadIdx.x - slot * VB;
    const int c = (int)blockIdx.y * VB + lane;
    const bool valid = c < VE;
    const int coff = (valid ? c : VE - 1) * V;
    ConvW<V> W;
    load_conv_w<V>(cw, cb, coff, W);
    float ds[V];
    dsum_of<V, FROM_G>(fg, coff, ds);
    float sdb[V], sdw[4][V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        sdb[v] = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) sdw[t][v] = 0.f;
    }
    const int64_t rpi = sq.runs();  // runs per image
    const int64_t ps = sq.pstride;
    const int64_t c0 = ((int64_t)blockIdx.x * k + slot) * kAdjRunsPerSlot;  // the slot's first run
    raw p3{}, p2{}, p1{};
    float d3[V], d2[V], d1[V];
    int rc0 = 0;  // first position of the walk (in its image)
    for (int i = 0; i < kAdjRunsPerSlot; ++i) {
        const int64_t U = c0 + i;
        if (U >= total_runs) break;
        const int64_t b = U / rpi;
        const int sr = (int)(U - b * rpi);  // sequence order within the image
        const int line = sr / sq.nk, kk = sr - line * sq.nk;
        const int r0 = line * sq.len + kk * sq.L;
        const int cnt = min(sq.L, sq.len - kk * sq.L);
        const bool cont = i > 0 && sr > 0;  // the walk goes on from the previous run
        const bool last = i + 1 == kAdjRunsPerSlot || U + 1 == total_runs || sr + 1 == rpi;
        const typename IO::elem* xb = x + b * (int64_t)sq.n * E + coff;
        typename IO::elem* gbase = dx + b * (int64_t)sq.n * E + coff;
        const typename IO::elem* xp = xb + sq.off(r0);
        typename IO::elem* gp = gbase + sq.off(r0);
        float u[V];
        du_row<V, FROM_G>(fg, b, line, E, coff, u);  // one scan position per run
        if (!cont) {
            rc0 = r0;
            p3 = p2 = p1 = raw{};
            if (r0 >= 3) p3 = load_raw<false>(xb + sq.off(r0 - 3));
            if (r0 >= 2) p2 = load_raw<false>(xb + sq.off(r0 - 2));
            if (r0 >= 1) p1 = load_raw<false>(xb + sq.off(r0 - 1));
#pragma unroll
            for (int v = 0; v < V; ++v) d3[v] = d2[v] = d1[v] = 0.f;
        }
        // dx[f - 3] from da[f - 3 .. f], for the positions of the walk: in this
        // run, or (f < 3, a continued walk) at the end of the previous runs
        auto emit = [&](const float (&da)[V], int f) {
            if (r0 + f - 3 >= rc0 && valid) {
                float o[V];
#pragma unroll
                for (int v = 0; v < V; ++v)
                    o[v] = fmaf(W.w[v][0], da[v], fmaf(W.w[v][1], d1[v], fmaf(W.w[v][2], d2[v], W.w[v][3] * d3[v])));
                store_vec<false>(f >= 3 ? gp + (f - 3) * ps : gbase + sq.off(r0 + f - 3), o);
            }
#pragma unroll
            for (int v = 0; v < V; ++v) {
                d3[v] = d2[v];
                d2[v] = d1[v];
                d1[v] = da[v];
            }
        };
        // position f < cnt of the run: da from the cell's x and dxc
        auto step = [&](const raw& xv, const raw& gv, int f) {
            float da[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float x0 = raw_at(p3, v), x1 = raw_at(p2, v), x2 = raw_at(p1, v), x3 = raw_at(xv, v);
                float a = fmaf(W.w[v][3], x3, W.b[v]);
                a = fmaf(W.w[v][2], x2, a);
                a = fmaf(W.w[v][1], x1, a);
                a = fmaf(W.w[v][0], x0, a);
                da[v] = dxc_at<IO, FROM_G>(gv, v, u, ds, fg.inv_p) * conv_silu_grad(a);
                sdb[v] += da[v];
                sdw[0][v] = fmaf(da[v], x0, sdw[0][v]);
                sdw[1][v] = fmaf(da[v], x1, sdw[1][v]);
                sdw[2][v] = fmaf(da[v], x2, sdw[2][v]);
                sdw[3][v] = fmaf(da[v], x3, sdw[3][v]);
            }
            p3 = p2;
            p2 = p1;
            p1 = xv;
            emit(da, f);
        };
        // whole batches, two in flight: the next batch's loads are issued
        // before the current batch computes and stores (a load of dxc at
        // position p always precedes the store of dx at p, and the stores of a
        // batch reach at most its first position)
        auto load_batch = [&](raw (&xo)[kB], raw (&go)[kB], int fb) {
#pragma unroll
            for (int q = 0; q < kB; ++q) {
                xo[q] = load_raw<false>(xp + (fb + q) * ps);
                go[q] = load_raw<false>(gp + (fb + q) * ps);
            }
        };
        auto run_batch = [&](const raw (&xi)[kB], const raw (&gi)[kB], int fb) {
#pragma unroll
            for (int q = 0; q < kB; ++q) step(xi[q], gi[q], fb + q);
        };
        const int nb = cnt / kB;
        raw xa[kB], ga[kB], xb2[kB], gb2[kB];
        if (nb > 0) load_batch(xa, ga, 0);
        int ib = 0;
        for (; ib + 2 < nb; ib += 2) {  // batches ib + 1 and ib + 2 exist
            load_batch(xb2, gb2, (ib + 1) * kB);
            run_batch(xa, ga, ib * kB);
            load_batch(xa, ga, (ib + 2) * kB);
            run_batch(xb2, gb2, (ib + 1) * kB);
        }
        if (ib + 2 == nb) {
            load_batch(xb2, gb2, (ib + 1) * kB);
            run_batch(xa, ga, ib * kB);
            run_batch(xb2, gb2, (ib + 1) * kB);
        } else if (ib + 1 == nb) {
            run_batch(xa, ga, ib * kB);
        }
        for (int f = nb * kB; f < cnt; ++f) {
            const raw xv = load_raw<false>(xp + f * ps), gv = load_raw<false>(gp + f * ps);
            step(xv, gv, f);
        }
        if (last) {
            // the three positions past the chunk: da from the halo of the next
            // chunk's first run (0 past the sequence)
            const float* hb = halo + ((U + 1) / kAdjRunsPerSlot * 3 * E + coff);
            for (int f = cnt; f < cnt + 3; ++f) {
                float da[V];
#pragma unroll
                for (int v = 0; v < V; ++v) da[v] = r0 + f < sq.n ? hb[(f - cnt) * E + v] : 0.f;
                emit(da, f);
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
            for (int u2 = 1; u2 < k; ++u2) s += red[((u2 - 1) * VB + lane) * 5 * V + v];
            row[coff + v] = s;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                float q = sdw[t][v];
                for (int u2 = 1; u2 < k; ++u2) q += red[((u2 - 1) * VB + lane) * 5 * V + V + 4 * v + t];
                row[E + (coff + v) * 4 + t] = q;
            }
        }
    }
}

constexpr int kSeqRun = 64;  // positions per run of the forward conv

template <class IO>
hipError_t conv_seq_t(const Geom& g, const void* x, const fastvim_params& p, void* xc, hipStream_t st) {
    const SeqShape s = seq_shape(g, kSeqRun);
    const int VE = (int)(g.E / IO::V);
    const int64_t items = g.B * s.runs() * VE;
    hipLaunchKernelGGL((conv_seq_kernel<IO>), dim3((unsigned)((items + kSeqThreads - 1) / kSeqThreads)),
                       dim3(kSeqThreads), 0, st, static_cast<const typename IO::elem*>(x),
                       static_cast<typename IO::elem*>(xc), p.conv_w, p.conv_b, s, (int)g.E, VE, items);
    return hipGetLastError();
}

// Vectors per slot of an adjoint workgroup, and its slots.
int adjoint_vb(const Geom& g) {
    const int VE = (int)(g.E / (g.io == FASTVIM_BF16 ? IoBf16::V : IoF32::V));
    return VE < kSeqThreads ? VE : kSeqThreads;
}
int adjoint_slots(const Geom& g) { return kSeqThreads / adjoint_vb(g); }

// Run length of the adjoint whose halo, partial rows and column-sum scratch
// fit in `floats`: the shortest of 64, 128, ... (runs never cross lines; a
// whole sequence as one run needs no halo).  *groups: partial rows.
int adjoint_run(const Geom& g, int64_t floats, int64_t* groups) {
    const int64_t rpg = (int64_t)adjoint_slots(g) * kAdjRunsPerSlot;
    for (int L = 64;; L *= 2) {
        const SeqShape s = seq_shape(g, L);
        const int64_t runs = g.B * s.runs();
        const int64_t gr = (runs + rpg - 1) / rpg;
        const int64_t chunks = (runs + kAdjRunsPerSlot - 1) / kAdjRunsPerSlot;
        const int64_t need = (s.runs() > 1 ? (chunks + 1) * 3 * g.E : 0) + gr * 5 * g.E +
                             ((gr + kColRowsPerBlock - 1) / kColRowsPerBlock) * 4 * g.E + 64;
        if (need <= floats || s.runs() == 1) {
            *groups = gr;
            return need <= floats ? s.L : 0;
        }
        if (s.L == s.len && L >= s.n) {  // runs of whole lines; cannot shrink the halo further
            *groups = gr;
            return 0;
        }
    }
}

template <class IO, bool FROM_G>
hipError_t conv_adjoint_t(const Geom& g, const void* x, void* dx, const fastvim_params& p, float* scratch,
                          int64_t floats, float* dcw, float* dcb, const DxcFromG& fg, hipStream_t st) {
    using elem = typename IO::elem;
    int64_t groups = 0;
    const int L = adjoint_run(g, floats, &groups);
    if (L == 0) return hipErrorInvalidValue;  // callers check conv_adjoint_fits first
    const SeqShape s = seq_shape(g, L);
    const int VE = (int)(g.E / IO::V);
    const int64_t total_runs = g.B * s.runs();
    float* halo = scratch;
    const int64_t chunks = (total_runs + kAdjRunsPerSlot - 1) / kAdjRunsPerSlot;
    float* parts = halo + (s.runs() > 1 ? (chunks + 1) * 3 * g.E : 0);
    float* tmp = parts + groups * 5 * g.E;
    const elem* xe = static_cast<const elem*>(x);
    elem* de = static_cast<elem*>(dx);
    if (s.runs() > 1) {
        const int64_t items = chunks * VE;
        hipLaunchKernelGGL((conv_adjoint_halo_kernel<IO, FROM_G>),
                           dim3((unsigned)((items + kSeqThreads - 1) / kSeqThreads)), dim3(kSeqThreads), 0, st, xe,
                           static_cast<const elem*>(dx), p.conv_w, p.conv_b, halo, s, (int)g.E, VE, items,
                           total_runs, fg);
    }
    const int VB = adjoint_vb(g), slots = adjoint_slots(g);
    const size_t lds = (size_t)((slots - 1) * VB * 5 * IO::V) * sizeof(float);
    hipLaunchKernelGGL((conv_adjoint_kernel<IO, FROM_G>), dim3((unsigned)groups, (unsigned)((VE + VB - 1) / VB)),
                       dim3((unsigned)(slots * VB)), lds, st, xe, de, p.conv_w, p.conv_b, halo, parts, s, (int)g.E,
                       VE, VB, total_runs, fg);
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
                               int64_t floats, float* dcw, float* dcb, hipStream_t st, const DxcFromG* fg) {
    if (fg)
        return g.io == FASTVIM_BF16 ? conv_adjoint_t<IoBf16, true>(g, x, dx, p, scratch, floats, dcw, dcb, *fg, st)
                                    : conv_adjoint_t<IoF32, true>(g, x, dx, p, scratch, floats, dcw, dcb, *fg, st);
    const DxcFromG none{};
    return g.io == FASTVIM_BF16 ? conv_adjoint_t<IoBf16, false>(g, x, dx, p, scratch, floats, dcw, dcb, none, st)
                                : conv_adjoint_t<IoF32, false>(g, x, dx, p, scratch, floats, dcw, dcb, none, st);
}

bool conv_adjoint_fits(const Geom& g, int64_t floats) {
    int64_t groups = 0;
    return adjoint_run(g, floats, &groups) > 0;
}

}  // namespace fastvim
