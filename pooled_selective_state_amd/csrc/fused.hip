// The whole dense pooled layer in one pipelined launch.
//
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解,
// bullets 2-5 (pool one axis, input-dependent projections and step size,
// forward and backward scans, repeat + skip); Pith review, "key_machinery"
// (repeat before the D x skip); Vim article (ijyty.com) 2.1 (sum of both
// directions gated by z).  Each stage computes what the staged kernels
// compute (pool.hip, proj.hip, scan_core.h, epilogue.hip).
//
// Why one launch: the output needs x twice (its own skip term) and the scan
// needs every token of the image, so the layer reads x, then z and x again.
// Run image by image as a software pipeline, the second read of x comes a few
// images after the first, while the image is still in the 256 MB Infinity
// Cache (the first read uses ordinary, allocating loads; z and out use
// non-allocating ones), so HBM sees close to one read of x, one of z and one
// write of out.  The projection and scan work of one image overlaps the
// streaming of others.
//
// Work items, one per 512-thread workgroup:
//   A(b, k)  pool scan positions [k*RG, k*RG + RG) of image b and project the
//            pooled tokens (both directions); count it in rowsDone[b];
//   S(b, k)  once rowsDone[b] == nA, scan channels [64k, 64k + 64) of image b
//            in both directions (scan_core.h), or with LBMamba's local
//            backward scan, channels [128k, 128k + 128) forward with each
//            chunk's local backward scan; count it in scanDone[b];
//   E(b, k)  once scanDone[b] == nS, repeat + skip + gate a block of image
//            b: grid rows [k*RE, k*RE + RE) (COLS), or RE rows x CJ columns
//            with the block's scan rows staged in LDS (ROWS); with the
//            post-SSM LayerNorm, grid rows [k*RE, k*RE + RE) in teams of
//            lanes per token (epilogue_norm.h), both orientations.
// Items are numbered slot by slot, slot s = [A(s, *)] [S(s - LS, *)]
// [E(s - LE, *)] with 1 <= LS <= LE (items outside [0, B) are left out), and
// handed out through one atomic ticket counter.  A workgroup takes its ticket
// when it starts and waits only for items with smaller tickets, which were
// taken by workgroups that had already started, so every wait ends whatever
// the grid size or residency.  As a guard against a broken invariant a wait
// also gives up after a bounded number of polls and raises a status bit.
//
// Publication without L2 write-backs: a producer stores its results with
// agent-scope atomic stores (written through to the device-coherent level),
// waits for them to complete, then bumps the counter; a consumer polls the
// counter, then executes an agent-scope acquire (invalidating its CU's L1 and
// its XCD's L2) before reading with ordinary loads.
#include <cstdlib>

#include "epilogue_norm.h"
#include "scan_core.h"

namespace fastvim {
namespace {

constexpr int kFT = 512;                                     // threads per workgroup
// LDS of one workgroup: the scan's rows of a whole sequence, or the pooling
// item's [G][E] partial sums + [RG][E] pooled tokens + [RG][KS][2 NX] partial
// projections.  48 KB lets three workgroups share a CU.
constexpr int kLdsFloats = kScanLdsFloats;
static_assert(sizeof(ScanSmem) == kLdsFloats * sizeof(float), "one buffer");
constexpr unsigned kSpinLimit = 1u << 20;                   // about a second of polling
constexpr int kEU = 4;                                       // tokens per lane per batch (E items)
constexpr int kMaxIv = 6;
constexpr int kNormTL = 64;  // norm E items: lanes per token (a wave) ...
constexpr int kNormNV = 2;   // ... and vectors per lane: E / V <= 128

struct FusedArgs {
    const void* x;
    const void* z;
    void* out;
    fastvim_dir_params pf, pb;
    float* u;
    float* xdbl;
    float* s_f;
    float* s_b;
    const float* ln_w;  // post-SSM LayerNorm (NORM instances)
    const float* ln_b;
    float ln_eps;
    float pool_norm;  // pool_scale / P
    unsigned* sync;  // [0] ticket, [1] status, [2, 2+B) rowsDone, [2+B, 2+2B) scanDone
    int64_t B, h, w, E, T, P;
    int R, NX, axis;
    int nA, nS, nE, RG, RE, CJ, G, VE, KS;
    int LS, LE;
    int niv;                  // slot intervals with a constant number of items per slot
    int64_t iv_s0[kMaxIv];    // first slot of the interval
    int64_t iv_t0[kMaxIv];    // first ticket of the interval
    int64_t iv_sz[kMaxIv];    // items per slot in the interval
    int64_t total;
};

union alignas(16) FusedSmem {
    ScanSmem scan;
    float buf[kLdsFloats];
};

// Thread 0 only: poll until *cnt >= target, then acquire at agent scope.
__device__ __forceinline__ void wait_at_least(unsigned* cnt, unsigned target, unsigned* status) {
    unsigned spins = 0;
    while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
        __builtin_amdgcn_s_sleep(2);
        if (++spins > kSpinLimit) {
            __hip_atomic_fetch_or(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// All threads: wait for this thread's write-through stores to complete, then
// (after the barrier) thread 0 counts the item done.
__device__ __forceinline__ void publish(unsigned* cnt) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_through(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float silu(float q) { return q * __builtin_amdgcn_rcpf(1.f + __expf(-q)); }

// ---------------------------------------------------------------- A items
template <class IO>
__device__ void item_pool_proj(const FusedArgs& a, int64_t b, int k, float* lds) {
    constexpr int V = IO::V;
    using elem = typename IO::elem;
    using raw = typename IO::raw;
    const elem* x = static_cast<const elem*>(a.x);
    const int tid = threadIdx.x;
    const int VE = a.VE, G = a.G;
    const int c = tid % VE, g = tid / VE;
    const int64_t E = a.E, T = a.T, P = a.P;
    const int64_t t0 = (int64_t)k * a.RG;
    const int npos = (int)(T - t0 < a.RG ? T - t0 : a.RG);
    const bool cols = a.axis == FASTVIM_POOL_COLS;
    const int64_t p_stride = cols ? E : a.w * E;
    const float inv_p = a.pool_norm;
    const int NO = 2 * a.NX;
    float* red = lds;                        // [G][E]
    float* urow = lds + (int64_t)G * E;      // [RG][E]
    float* part = urow + (int64_t)a.RG * E;  // [RG][NO][KS]

    const int pstr = (int)p_stride;
    for (int pos = 0; pos < npos; ++pos) {
        const int64_t t = t0 + pos;
        if (g < G) {
            // wave-uniform base, 32-bit lane offsets (an image holds < 2^31 elements)
            const elem* base = x + b * a.h * a.w * E + (cols ? t * a.w * E : t * E);
            const int coff = c * V;
            float acc[V];
#pragma unroll
            for (int v = 0; v < V; ++v) acc[v] = 0.f;
            int p = g;
            // 8 allocating loads in flight per lane (x is read again by E items)
            for (; p + 7 * G < P; p += 8 * G) {
                raw r[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) r[q] = load_raw<false>(base + (coff + (p + q * G) * pstr));
#pragma unroll
                for (int v = 0; v < V; ++v)
                    acc[v] += ((raw_at(r[0], v) + raw_at(r[1], v)) + (raw_at(r[2], v) + raw_at(r[3], v))) +
                              ((raw_at(r[4], v) + raw_at(r[5], v)) + (raw_at(r[6], v) + raw_at(r[7], v)));
            }
            for (; p < P; p += G) {
                const raw r0 = load_raw<false>(base + (coff + p * pstr));
#pragma unroll
                for (int v = 0; v < V; ++v) acc[v] += raw_at(r0, v);
            }
#pragma unroll
            for (int v = 0; v < V; ++v) red[g * (int)E + coff + v] = acc[v];
        }
        __syncthreads();
        for (int q = tid; q < E; q += kFT) {
            float s = red[q];
            for (int gg = 1; gg < G; ++gg) s += red[(int64_t)gg * E + q];
            s *= inv_p;
            urow[(int64_t)pos * E + q] = s;
            store_through(a.u + (b * T + t) * E + q, s);
        }
        __syncthreads();
    }

    // x_proj of the pooled tokens: pair (o, kk) dots the kk-th interleaved
    // part of E with weight row o, for every position (weights through the cache).
    const int npairs = NO * a.KS;
    const int E4 = (int)(E / 4);
    for (int pr = tid; pr < npairs; pr += kFT) {
        const int o = pr / a.KS, kk = pr - o * a.KS;
        const float* W = o < a.NX ? a.pf.x_proj_w + (int64_t)o * E : a.pb.x_proj_w + (int64_t)(o - a.NX) * E;
        for (int q = 0; q < npos; ++q) {  // the weight row is re-read from the cache per position
            const float* ur = urow + q * (int)E;
            float acc = 0.f;
#pragma unroll 4
            for (int c4 = kk; c4 < E4; c4 += a.KS) {
                const f32x4 wv = *reinterpret_cast<const f32x4*>(W + 4 * c4);
                const f32x4 uv = *reinterpret_cast<const f32x4*>(ur + 4 * c4);
                acc = fmaf(wv.x, uv.x, fmaf(wv.y, uv.y, fmaf(wv.z, uv.z, fmaf(wv.w, uv.w, acc))));
            }
            part[(q * NO + o) * a.KS + kk] = acc;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < npos * NO; idx += kFT) {
        const int q = idx / NO, o = idx - q * NO;
        float v = 0.f;
        for (int kk = 0; kk < a.KS; ++kk) v += part[((int64_t)q * NO + o) * a.KS + kk];
        store_through(a.xdbl + (b * T + t0 + q) * NO + o, v);
    }
    publish(&a.sync[2 + b]);
}

// ---------------------------------------------------------------- E items
template <int V>
__device__ __forceinline__ void scan_sum(const FusedArgs& a, int64_t b, int64_t t, int64_t col, float (&sv)[V]) {
    const float* s1 = a.s_f + (b * a.T + t) * a.E + col;
    const float* s2 = a.s_b + (b * a.T + t) * a.E + col;
#pragma unroll
    for (int v = 0; v < V; v += 4) {
        const f32x4 p1 = load_raw<false>(s1 + v), p2 = load_raw<false>(s2 + v);
        sv[v] = p1.x + p2.x;
        sv[v + 1] = p1.y + p2.y;
        sv[v + 2] = p1.z + p2.z;
        sv[v + 3] = p1.w + p2.w;
    }
}

// Grid rows [k*RE, k*RE + RE) of image b.  x and z are read for the last time
// (non-temporal), out is written once (non-temporal).  Lane (c, g) handles the
// row's tokens g + G*m in batches of kEU, all loads of a batch issued first.
template <class IO, bool COLS>
__device__ void item_epilogue(const FusedArgs& a, int64_t b, int k) {
    constexpr int V = IO::V;
    using elem = typename IO::elem;
    using raw = typename IO::raw;
    const int tid = threadIdx.x;
    if (tid == 0) wait_at_least(&a.sync[2 + a.B + b], (unsigned)a.nS, &a.sync[1]);
    __syncthreads();
    const int VE = a.VE, G = a.G;
    const int c = tid % VE, g = tid / VE;
    if (g >= G) return;
    const int64_t E = a.E, w = a.w;
    const int64_t col = (int64_t)c * V;
    float dsum[V];
#pragma unroll
    for (int v = 0; v < V; ++v) dsum[v] = a.pf.D[col + v] + a.pb.D[col + v];

    const int64_t i0 = (int64_t)k * a.RE;
    const int64_t i1 = i0 + a.RE < a.h ? i0 + a.RE : a.h;
    const int iw = (int)w, iE = (int)E, coff = (int)col;
    for (int64_t i = i0; i < i1; ++i) {
        // wave-uniform row bases, 32-bit lane offsets
        const int64_t rowoff = (b * a.h + i) * w * E;
        const elem* xr = static_cast<const elem*>(a.x) + rowoff;
        const elem* zr = static_cast<const elem*>(a.z) + rowoff;
        elem* orow = static_cast<elem*>(a.out) + rowoff;
        float srow[V];
        if (COLS) scan_sum<V>(a, b, i, col, srow);
        for (int j0 = g; j0 < iw; j0 += G * kEU) {
            raw xv[kEU], zv[kEU];
#pragma unroll
            for (int m = 0; m < kEU; ++m) {
                const int j = j0 + G * m;
                if (j < iw) {
                    xv[m] = load_raw<true>(xr + (coff + j * iE));
                    zv[m] = load_raw<true>(zr + (coff + j * iE));
                }
            }
#pragma unroll
            for (int m = 0; m < kEU; ++m) {
                const int j = j0 + G * m;
                if (j >= iw) continue;
                float sv[V];
                if (COLS) {
#pragma unroll
                    for (int v = 0; v < V; ++v) sv[v] = srow[v];
                } else {
                    scan_sum<V>(a, b, j, col, sv);
                }
                float o[V];
#pragma unroll
                for (int v = 0; v < V; ++v) o[v] = (sv[v] + dsum[v] * raw_at(xv[m], v)) * silu(raw_at(zv[m], v));
                store_vec<true>(orow + (coff + j * iE), o);
            }
        }
    }
}

// ROWS: token (i, j) belongs to scan position j, so neighbouring tokens of a
// grid row need different scan rows.  An item covers grid rows
// [i0, i0 + RE) x columns [j0, j0 + CJ) of image b: it stages
// s_fwd + s_bwd of its CJ columns in LDS once (CJ * E floats), then streams
// the block's tokens (each row segment of the block is contiguous in memory)
// in batches of kEU per lane, all loads of a batch issued first, walking the
// block row by row without divisions.
template <class IO>
__device__ void item_epilogue_rows(const FusedArgs& a, int64_t b, int k, float* lds) {
    constexpr int V = IO::V;
    using elem = typename IO::elem;
    using raw = typename IO::raw;
    const int tid = threadIdx.x;
    if (tid == 0) wait_at_least(&a.sync[2 + a.B + b], (unsigned)a.nS, &a.sync[1]);
    __syncthreads();
    const int64_t E = a.E, w = a.w;
    const int nJB = (int)((w + a.CJ - 1) / a.CJ);
    const int ib = k / nJB, jb = k - ib * nJB;
    const int64_t i0 = (int64_t)ib * a.RE, j0 = (int64_t)jb * a.CJ;
    const int ni = (int)(i0 + a.RE < a.h ? a.RE : a.h - i0);
    const int nj = (int)(j0 + a.CJ < w ? a.CJ : w - j0);
    const int iE = (int)E, iw = (int)w;
    {
        // all loads in flight at once: the rows come from beyond this XCD's L2
        constexpr int kIt = kLdsFloats / (4 * kFT);
        const float* s1 = a.s_f + (b * a.T + j0) * E;  // columns j0 .. are consecutive scan rows
        const float* s2 = a.s_b + (b * a.T + j0) * E;
        const int n = nj * iE;
        f32x4 p1[kIt], p2[kIt];
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int q = 4 * tid + 4 * kFT * it;
            if (q < n) {
                p1[it] = load_raw<false>(s1 + q);
                p2[it] = load_raw<false>(s2 + q);
            }
        }
#pragma unroll
        for (int it = 0; it < kIt; ++it) {
            const int q = 4 * tid + 4 * kFT * it;
            if (q < n) *reinterpret_cast<f32x4*>(lds + q) = p1[it] + p2[it];
        }
    }
    __syncthreads();
    const int VE = a.VE, G = a.G;
    const int c = tid % VE, g = tid / VE;
    if (g >= G) return;
    const int coff = c * V;
    float dsum[V];
#pragma unroll
    for (int v = 0; v < V; ++v) dsum[v] = a.pf.D[coff + v] + a.pb.D[coff + v];
    // wave-uniform block base, 32-bit token offsets (an image holds < 2^31 elements)
    const int64_t base = (b * a.h + i0) * w * E + j0 * E;
    const elem* xb = static_cast<const elem*>(a.x) + base;
    const elem* zb = static_cast<const elem*>(a.z) + base;
    elem* ob = static_cast<elem*>(a.out) + base;
    int ii = g / nj, jj = g - (g / nj) * nj;  // this lane's next token of the block
    while (ii < ni) {
        int off[kEU], sj[kEU];
        bool ok[kEU];
        raw xv[kEU], zv[kEU];
#pragma unroll
        for (int m = 0; m < kEU; ++m) {
            ok[m] = ii < ni;
            off[m] = (ii * iw + jj) * iE + coff;
            sj[m] = jj * iE + coff;
            jj += G;
            while (jj >= nj) {
                jj -= nj;
                ++ii;
            }
        }
#pragma unroll
        for (int m = 0; m < kEU; ++m)
            if (ok[m]) {
                xv[m] = load_raw<true>(xb + off[m]);
                zv[m] = load_raw<true>(zb + off[m]);
            }
#pragma unroll
        for (int m = 0; m < kEU; ++m) {
            if (!ok[m]) continue;
            float o[V];
#pragma unroll
            for (int v = 0; v < V; v += 4) {
                const f32x4 sv = *reinterpret_cast<const f32x4*>(lds + sj[m] + v);
                o[v] = (sv.x + dsum[v] * raw_at(xv[m], v)) * silu(raw_at(zv[m], v));
                o[v + 1] = (sv.y + dsum[v + 1] * raw_at(xv[m], v + 1)) * silu(raw_at(zv[m], v + 1));
                o[v + 2] = (sv.z + dsum[v + 2] * raw_at(xv[m], v + 2)) * silu(raw_at(zv[m], v + 2));
                o[v + 3] = (sv.w + dsum[v + 3] * raw_at(xv[m], v + 3)) * silu(raw_at(zv[m], v + 3));
            }
            store_vec<true>(ob + off[m], o);
        }
    }
}

// Norm E items: grid rows [k*RE, k*RE + RE) of image b.  The per-channel
// vectors (D_fwd + D_bwd, the norm's weight and bias) are staged in LDS once
// per item and, for COLS, the summed scan row once per grid row; each team of
// kNormTL lanes (a wave) then takes two tokens at a time and runs the
// per-token norm epilogue, the next two tokens' x and z loads issued before
// the current two are computed.  ROWS tokens read their scan rows through
// the caches.
template <class IO, bool COLS>
__device__ void item_epilogue_norm(const FusedArgs& a, int64_t b, int k, float* lds) {
    using raw = typename IO::raw;
    using elem = typename IO::elem;
    constexpr int kTeams = kFT / kNormTL;
    const int tid = threadIdx.x;
    if (tid == 0) wait_at_least(&a.sync[2 + a.B + b], (unsigned)a.nS, &a.sync[1]);
    const int w = (int)a.w, E = (int)a.E;
    float* ds = lds;              // [E] D_fwd + D_bwd
    float* gw = lds + E;          // [E] norm weight
    float* gb = lds + 2 * E;      // [E] norm bias
    float* srow = lds + 3 * E;    // [E] COLS: s_fwd + s_bwd of the current grid row
    for (int e = tid; e < E; e += kFT) {
        ds[e] = a.pf.D[e] + a.pb.D[e];
        gw[e] = a.ln_w[e];
        gb[e] = a.ln_b[e];
    }
    __syncthreads();
    const int lane = tid % kNormTL, team = tid / kNormTL;
    const int64_t i0 = (int64_t)k * a.RE;
    const int64_t i1 = i0 + a.RE < a.h ? i0 + a.RE : a.h;
    const int64_t img = b * a.h * a.w;
    const elem* x = static_cast<const elem*>(a.x);
    const elem* z = static_cast<const elem*>(a.z);
    elem* out = static_cast<elem*>(a.out);
    for (int64_t i = i0; i < i1; ++i) {
        if (COLS) {
            __syncthreads();  // the previous row's tokens are done with srow
            const float* s1 = a.s_f + (b * a.T + i) * E;
            const float* s2 = a.s_b + (b * a.T + i) * E;
            for (int e = tid; e < E; e += kFT) srow[e] = s1[e] + s2[e];
            __syncthreads();
        }
        // the next pair's x and z are loaded before the current pair is computed
        raw nx1[kNormNV], nz1[kNormNV], nx2[kNormNV], nz2[kNormNV];
        auto load_pair = [&](int j) {
            const int j2 = j + kTeams;
            const int64_t c1 = img + i * w + j, c2 = img + i * w + (j2 < w ? j2 : j);
            norm_load<IO, kNormTL, kNormNV>(x + c1 * E, z + c1 * E, E, lane, nx1, nz1);
            if (j2 < w) norm_load<IO, kNormTL, kNormNV>(x + c2 * E, z + c2 * E, E, lane, nx2, nz2);
        };
        if (team < w) load_pair(team);
        for (int j = team; j < w; j += 2 * kTeams) {
            const int j2 = j + kTeams;
            const bool two = j2 < w;
            const int64_t c1 = img + i * w + j, c2 = img + i * w + (two ? j2 : j);
            raw x1[kNormNV], z1[kNormNV], x2[kNormNV], z2[kNormNV];
#pragma unroll
            for (int v = 0; v < kNormNV; ++v) {
                x1[v] = nx1[v];
                z1[v] = nz1[v];
                x2[v] = nx2[v];
                z2[v] = nz2[v];
            }
            if (j + 2 * kTeams < w) load_pair(j + 2 * kTeams);
            if (COLS) {
                norm_finish<IO, kNormTL, kNormNV, true>(x1, z1, srow, nullptr, ds, nullptr, gw, gb, a.ln_eps,
                                                        out + c1 * E, E, lane);
                if (two)
                    norm_finish<IO, kNormTL, kNormNV, true>(x2, z2, srow, nullptr, ds, nullptr, gw, gb, a.ln_eps,
                                                            out + c2 * E, E, lane);
            } else {
                norm_finish<IO, kNormTL, kNormNV>(x1, z1, a.s_f + (b * a.T + j) * E, a.s_b + (b * a.T + j) * E,
                                                  a.pf.D, a.pb.D, gw, gb, a.ln_eps, out + c1 * E, E, lane);
                if (two)
                    norm_finish<IO, kNormTL, kNormNV>(x2, z2, a.s_f + (b * a.T + j2) * E,
                                                      a.s_b + (b * a.T + j2) * E, a.pf.D, a.pb.D, gw, gb, a.ln_eps,
                                                      out + c2 * E, E, lane);
            }
        }
    }
}

// ---------------------------------------------------------------- kernel
template <class IO, bool COLS, int RMAX, bool NORM, bool LOCAL>
__global__ void __launch_bounds__(kFT) fused_layer_kernel(FusedArgs a) {
    __shared__ FusedSmem sm;
    __shared__ unsigned s_ticket;
    if (threadIdx.x == 0)
        s_ticket = __hip_atomic_fetch_add(&a.sync[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int64_t ticket = s_ticket;
    if (ticket >= a.total) return;
    // ticket -> (slot, index within the slot)
    int iv = 0;
    while (iv + 1 < a.niv && ticket >= a.iv_t0[iv + 1]) ++iv;
    const int64_t off = ticket - a.iv_t0[iv];
    const int64_t slot = a.iv_s0[iv] + off / a.iv_sz[iv];
    int64_t r = off % a.iv_sz[iv];
    if (slot < a.B) {
        if (r < a.nA) {
            item_pool_proj<IO>(a, slot, (int)r, sm.buf);
            return;
        }
        r -= a.nA;
    }
    const int64_t bs = slot - a.LS;
    if (bs >= 0 && bs < a.B) {
        if (r < a.nS) {
            if (threadIdx.x == 0) wait_at_least(&a.sync[2 + bs], (unsigned)a.nA, &a.sync[1]);
            __syncthreads();
            __builtin_amdgcn_s_setprio(2);  // the scan is on the critical path of its image
            ScanArgs sa{a.xdbl, a.pf, a.pb, a.s_f, a.s_b, a.T, a.E, a.R, a.NX};
            scan_tile_resident<RMAX, true, USrcPooled, LOCAL>(sa, USrcPooled{a.u, a.T, a.E}, bs,
                                                              (int64_t)r * (LOCAL ? 2 : 1) * kScanCh, sm.scan);
            __builtin_amdgcn_s_setprio(0);
            publish(&a.sync[2 + a.B + bs]);
            return;
        }
        r -= a.nS;
    }
    if (NORM) item_epilogue_norm<IO, COLS>(a, slot - a.LE, (int)r, sm.buf);
    else if (COLS) item_epilogue<IO, true>(a, slot - a.LE, (int)r);
    else item_epilogue_rows<IO>(a, slot - a.LE, (int)r, sm.buf);
}

__global__ void zero_sync_kernel(unsigned* sync, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        sync[i] = 0u;
}

int env_int(const char* name, int dflt) {
    const char* s = getenv(name);
    return s ? atoi(s) : dflt;
}

// Item sizes and ticket layout for a geometry; false if not covered.  norm:
// with the post-SSM LayerNorm (E items of whole grid rows, E / V <= 128);
// local: with LBMamba's local backward scan (not with the norm).
bool plan(const Geom& g, FusedArgs* a, bool norm, bool local) {
    if (!g.pooled || g.masked || g.B < 1 || (norm && local)) return false;
    // the scan items hold a whole sequence's x_proj rows in LDS
    const int64_t tmax = g.R <= 16 ? resident_tmax<16>() : g.R <= 32 ? resident_tmax<32>() : resident_tmax<64>();
    if (g.T > tmax) return false;
    if (g.h * g.w * g.E >= ((int64_t)1 << 31)) return false;  // 32-bit offsets within an image
    const int V = g.io == FASTVIM_BF16 ? 8 : 4;
    const int64_t esz = g.io == FASTVIM_BF16 ? 2 : 4;
    const int64_t VE = g.E / V;
    if (VE > kFT) return false;
    if (norm && VE > kNormTL * kNormNV) return false;
    const int G = (int)(kFT / VE);
    const int64_t NO = 2 * g.NX;
    int KS = (int)(kFT / NO);
    KS = KS < 1 ? 1 : (KS > 4 ? 4 : KS);
    // A items: about 200 KB of x each, at most 8 positions, within the LDS budget.
    const int64_t pos_bytes = g.P * g.E * esz;
    int64_t RG = (200 * 1024) / (pos_bytes > 0 ? pos_bytes : 1);
    RG = RG < 1 ? 1 : (RG > 8 ? 8 : RG);
    if (RG > g.T) RG = g.T;
    while (RG > 1 && G * g.E + RG * g.E + RG * NO * KS > kLdsFloats) --RG;
    if (G * g.E + RG * g.E + RG * NO * KS > kLdsFloats) return false;
    // E items: about 200 KB of each stream.  COLS: RE whole grid rows.  ROWS:
    // RE rows x CJ columns, CJ as many columns as the LDS holds scan rows of.
    int64_t RE, CJ;
    if (g.axis == FASTVIM_POOL_COLS || norm) {
        const int64_t row_bytes = g.w * g.E * esz;
        RE = (200 * 1024) / row_bytes;
        CJ = g.w;
    } else {
        CJ = kLdsFloats / g.E;
        if (CJ > 32) CJ = 32;
        if (CJ > g.w) CJ = g.w;
        if (CJ < 1) return false;
        RE = (200 * 1024) / (CJ * g.E * esz);
    }
    RE = RE < 1 ? 1 : (RE > g.h ? g.h : RE);
    a->B = g.B; a->h = g.h; a->w = g.w; a->E = g.E; a->T = g.T; a->P = g.P;
    a->pool_norm = pool_norm(g);
    a->R = (int)g.R; a->NX = (int)g.NX; a->axis = g.axis;
    a->VE = (int)VE; a->G = G; a->KS = KS; a->RG = (int)RG; a->RE = (int)RE; a->CJ = (int)CJ;
    a->nA = (int)((g.T + RG - 1) / RG);
    const int64_t sch = (local ? 2 : 1) * kScanCh;  // channels per scan item
    a->nS = (int)((g.E + sch - 1) / sch);
    a->nE = (int)(((g.h + RE - 1) / RE) * ((g.w + CJ - 1) / CJ));
    // Lags.  Between the A items of image b (slot b) and its E items (slot
    // b + LE) the pipeline reads LE other images' x with allocating loads;
    // E items find x in the 256 MB Infinity Cache only while that stays
    // within about 180 MB, so LE = 180 MB / x bytes per image (7 images at
    // 2048^2 fp32, 14 in bf16: measured best, 7-8 and 12-16).  The scans
    // start LS slots after pooling, enough for the image's A items to drain.
    // The environment variables override both (for lag sweeps).
    const int64_t x_img = g.h * g.w * g.E * esz;
    int64_t le = (180ll << 20) / x_img;
    le = le < 1 ? 1 : (le > g.B ? g.B : le);
    int64_t ls = le / 4 < 3 ? 3 : le / 4;
    if (ls > le) ls = le;
    a->LS = env_int("FASTVIM_FUSED_LS", (int)ls);
    a->LE = env_int("FASTVIM_FUSED_LE", (int)le);
    if (a->LS < 1) a->LS = 1;
    if (a->LE < a->LS) a->LE = a->LS;
    // slots [0, B + LE): piecewise-constant item counts between the breakpoints
    int64_t pts[6] = {0, a->LS, a->LE, g.B, g.B + a->LS, g.B + a->LE};
    for (int i = 1; i < 6; ++i)  // insertion sort
        for (int j = i; j > 0 && pts[j] < pts[j - 1]; --j) {
            const int64_t tmp = pts[j];
            pts[j] = pts[j - 1];
            pts[j - 1] = tmp;
        }
    int64_t tick = 0;
    a->niv = 0;
    for (int i = 0; i + 1 < 6; ++i) {
        const int64_t s0 = pts[i], s1 = pts[i + 1];
        if (s1 <= s0) continue;
        const int64_t sz = (s0 < g.B ? a->nA : 0) + (s0 >= a->LS && s0 < g.B + a->LS ? a->nS : 0) +
                           (s0 >= a->LE && s0 < g.B + a->LE ? a->nE : 0);
        if (sz == 0) continue;
        a->iv_s0[a->niv] = s0;
        a->iv_t0[a->niv] = tick;
        a->iv_sz[a->niv] = sz;
        ++a->niv;
        tick += (s1 - s0) * sz;
    }
    a->total = tick;
    return a->niv > 0 && a->total < (int64_t)UINT32_MAX;
}

template <class IO, int RMAX, bool NORM, bool LOCAL>
hipError_t fused_launch_n(const FusedArgs& a, hipStream_t st) {
    if (a.axis == FASTVIM_POOL_COLS)
        hipLaunchKernelGGL((fused_layer_kernel<IO, true, RMAX, NORM, LOCAL>), dim3((unsigned)a.total), dim3(kFT), 0,
                           st, a);
    else
        hipLaunchKernelGGL((fused_layer_kernel<IO, false, RMAX, NORM, LOCAL>), dim3((unsigned)a.total), dim3(kFT), 0,
                           st, a);
    return hipGetLastError();
}

template <class IO, int RMAX>
hipError_t fused_launch_r(const FusedArgs& a, hipStream_t st, bool local) {
    if (a.ln_w) return fused_launch_n<IO, RMAX, true, false>(a, st);
    return local ? fused_launch_n<IO, RMAX, false, true>(a, st) : fused_launch_n<IO, RMAX, false, false>(a, st);
}

template <class IO>
hipError_t fused_launch_io(const FusedArgs& a, hipStream_t st, bool local) {
    if (a.R <= 16) return fused_launch_r<IO, 16>(a, st, local);
    if (a.R <= 32) return fused_launch_r<IO, 32>(a, st, local);
    return fused_launch_r<IO, 64>(a, st, local);
}

}  // namespace

bool fused_supported(const Geom& g, bool norm, bool local) {
    FusedArgs a;
    return plan(g, &a, norm, local);
}

bool fused_preferred(const Geom& g, bool norm, bool local) {
    // The pipeline's fixed costs (scan latency per image, fill and drain)
    // pay off once an image's x is several MB: measured faster than the stage
    // kernels at 2048^2 (25 MB fp32, 12.6 MB bf16), slower at 1024^2 (6.3 MB)
    // and below.
    // With the norm, ROWS reads each token's scan rows through the caches and
    // measured slower than its stage kernels; COLS (a scan row per grid row,
    // staged in LDS) is faster.
    const int64_t esz = g.io == FASTVIM_BF16 ? 2 : 4;
    if (norm && g.axis != FASTVIM_POOL_COLS) return false;
    return g.h * g.w * g.E * esz >= (8ll << 20) && fused_supported(g, norm, local);
}

hipError_t launch_zero_sync(const Workspace& ws, int64_t n, hipStream_t st) {
    hipLaunchKernelGGL(zero_sync_kernel, dim3(1), dim3(256), 0, st, ws.sync, n);
    return hipGetLastError();
}

hipError_t launch_fused(const Geom& g, const void* x, const void* z, const fastvim_params& p, const Workspace& ws,
                        void* out, hipStream_t st) {
    FusedArgs a;
    const bool norm = (p.flags & FASTVIM_FLAG_POST_NORM) != 0;
    const bool local = (p.flags & FASTVIM_FLAG_LOCAL_BWD) != 0;
    if (!plan(g, &a, norm, local)) return hipErrorInvalidValue;
    a.x = x; a.z = z; a.out = out;
    a.pf = p.fwd; a.pb = p.bwd;
    a.ln_w = norm ? p.ln_weight : nullptr;
    a.ln_b = norm ? p.ln_bias : nullptr;
    a.ln_eps = norm ? p.ln_eps : 0.f;
    a.u = ws.u; a.xdbl = ws.xdbl; a.s_f = ws.s_f; a.s_b = ws.s_b;
    a.sync = ws.sync;
    return g.io == FASTVIM_BF16 ? fused_launch_io<IoBf16>(a, st, local) : fused_launch_io<IoF32>(a, st, local);
}

}  // namespace fastvim
