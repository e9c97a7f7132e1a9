// The whole dense pooled layer in one launch.
//
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解,
// bullets 2-5 (pool one axis, input-dependent projections and step size,
// forward and backward scans, repeat + skip); Pith review, "key_machinery"
// (repeat before the D x skip); Vim article (ijyty.com) 2.1 (sum of both
// directions gated by z).  Each stage computes exactly what the staged
// kernels compute (pool.hip, proj.hip, scan_core.h, epilogue.hip).
//
// Why one launch: the output needs x twice (its own skip term) and the scan
// needs every token of the image, so the layer reads x, then z and x again.
// Run image by image in a software pipeline, the second read of x comes a
// couple of images after the first, while the image is still in the 256 MB
// Infinity Cache (the first read uses ordinary, allocating loads), so HBM sees
// close to one read of x, one of z and one write of out.  The small
// projection and scan work of one image overlaps the streaming of others.
//
// Work items, each run by one 512-thread workgroup:
//   A(b, k)  pool scan positions [k*RG, k*RG + RG) of image b, then x_proj of
//            those pooled tokens (both directions); count it in rowsDone[b];
//   S(b, k)  wait until rowsDone[b] == nA, then scan channels [64k, 64k + 64)
//            of image b in both directions (scan_core.h); count it in scanDone[b];
//   E(b, k)  wait until scanDone[b] == nS, then repeat + skip + gate grid rows
//            [k*RE, k*RE + RE) of image b.
// Items are handed out through one atomic ticket counter, in slots:
//   slot s = [A(s, *)] [S(s - LS, *)] [E(s - LE, *)],  1 <= LS <= LE.
// A workgroup takes its ticket when it starts and only ever waits for items
// with smaller tickets, which were taken by workgroups that had already
// started; so every wait ends, whatever the grid size or residency.  As a
// guard against a broken invariant, a wait also gives up after a bounded
// number of polls and raises a status bit instead of hanging.
#include <cstdlib>

#include "scan_core.h"

namespace fastvim {
namespace {

constexpr int kFusedThreads = 512;
constexpr int kLdsFloats = (int)(sizeof(ScanSmem) / sizeof(float));
constexpr unsigned kSpinLimit = 1u << 20;  // about a second of polling; normal waits are microseconds

struct FusedArgs {
    const void* x;
    const void* z;
    void* out;
    fastvim_dir_params pf, pb;
    float* u;
    float* xdbl;
    float* s_f;
    float* s_b;
    unsigned* sync;  // [0] ticket, [1] status, [2, 2+B) rowsDone, [2+B, 2+2B) scanDone
    int64_t B, h, w, E, T, P;
    int R, NX, axis;
    int nA, nS, nE, RG, RE, G, VE, KS;
    int LS, LE;
    int64_t per_slot, total;
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

// Thread 0 only, after a workgroup barrier: publish the workgroup's stores.
__device__ __forceinline__ void count_done(unsigned* cnt) {
    __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
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
    const float inv_p = 1.0f / (float)P;
    const int NO = 2 * a.NX;
    float* red = lds;                       // [G][E]
    float* urow = lds + (int64_t)G * E;     // [RG][E]
    float* part = urow + (int64_t)a.RG * E; // [RG][NO][KS]

    for (int pos = 0; pos < npos; ++pos) {
        const int64_t t = t0 + pos;
        if (g < G) {
            const elem* base = x + b * a.h * a.w * E + (cols ? t * a.w * E : t * E) + (int64_t)c * V;
            float acc[V];
#pragma unroll
            for (int v = 0; v < V; ++v) acc[v] = 0.f;
            int64_t p = g;
            for (; p + 3 * G < P; p += 4 * G) {
                const raw r0 = load_raw<false>(base + p * p_stride);
                const raw r1 = load_raw<false>(base + (p + G) * p_stride);
                const raw r2 = load_raw<false>(base + (p + 2 * G) * p_stride);
                const raw r3 = load_raw<false>(base + (p + 3 * G) * p_stride);
#pragma unroll
                for (int v = 0; v < V; ++v)
                    acc[v] += (raw_at(r0, v) + raw_at(r1, v)) + (raw_at(r2, v) + raw_at(r3, v));
            }
            for (; p < P; p += G) {
                const raw r0 = load_raw<false>(base + p * p_stride);
#pragma unroll
                for (int v = 0; v < V; ++v) acc[v] += raw_at(r0, v);
            }
#pragma unroll
            for (int v = 0; v < V; ++v) red[(int64_t)g * E + (int64_t)c * V + v] = acc[v];
        }
        __syncthreads();
        for (int q = tid; q < E; q += kFusedThreads) {
            float s = red[q];
            for (int gg = 1; gg < G; ++gg) s += red[(int64_t)gg * E + q];
            s *= inv_p;
            urow[(int64_t)pos * E + q] = s;
            a.u[(b * T + t) * E + q] = s;
        }
        __syncthreads();
    }

    // x_proj of the npos pooled tokens: pair (o, kk) dots the kk-th interleaved
    // quarter of E with weight row o, for every position.
    const int npairs = NO * a.KS;
    for (int pr = tid; pr < npairs; pr += kFusedThreads) {
        const int o = pr / a.KS, kk = pr - o * a.KS;
        const float* W = o < a.NX ? a.pf.x_proj_w + (int64_t)o * E : a.pb.x_proj_w + (int64_t)(o - a.NX) * E;
        float accp[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) accp[q] = 0.f;
        for (int64_t c4 = kk; c4 < E / 4; c4 += a.KS) {
            const f32x4 wv = *reinterpret_cast<const f32x4*>(W + 4 * c4);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                if (q < npos) {
                    const f32x4 uv = *reinterpret_cast<const f32x4*>(urow + (int64_t)q * E + 4 * c4);
                    accp[q] = fmaf(wv.x, uv.x, fmaf(wv.y, uv.y, fmaf(wv.z, uv.z, fmaf(wv.w, uv.w, accp[q]))));
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
            if (q < npos) part[((int64_t)q * NO + o) * a.KS + kk] = accp[q];
    }
    __syncthreads();
    for (int idx = tid; idx < npos * NO; idx += kFusedThreads) {
        const int q = idx / NO, o = idx - q * NO;
        float v = 0.f;
        for (int kk = 0; kk < a.KS; ++kk) v += part[((int64_t)q * NO + o) * a.KS + kk];
        a.xdbl[(b * T + t0 + q) * NO + o] = v;
    }
    __syncthreads();
    if (tid == 0) count_done(&a.sync[2 + b]);
}

// ---------------------------------------------------------------- E items
// out of one token from its raw x and z vectors and its scan sum sv.
template <class IO>
__device__ __forceinline__ void emit_token(typename IO::elem* dst, const typename IO::raw& xr,
                                           const typename IO::raw& zr, const float* sv, const float* dsum) {
    constexpr int V = IO::V;
    float o[V];
#pragma unroll
    for (int v = 0; v < V; ++v) o[v] = (sv[v] + dsum[v] * raw_at(xr, v)) * silu(raw_at(zr, v));
    store_vec<true>(dst, o);
}

// s_fwd + s_bwd of scan position t for the lane's V channels.
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
// (non-temporal), out is written once (non-temporal).  COLS: every token of
// row i uses scan position i; ROWS: token (i, j) uses scan position j.
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
    if (g >= G) return;  // no barrier follows
    const int64_t E = a.E, w = a.w;
    const int64_t col = (int64_t)c * V;
    float dsum[V];
#pragma unroll
    for (int v = 0; v < V; ++v) dsum[v] = a.pf.D[col + v] + a.pb.D[col + v];

    const int64_t i0 = (int64_t)k * a.RE;
    const int64_t i1 = i0 + a.RE < a.h ? i0 + a.RE : a.h;
    for (int64_t i = i0; i < i1; ++i) {
        const int64_t rowoff = (b * a.h + i) * w * E + col;
        const elem* xr = static_cast<const elem*>(a.x) + rowoff;
        const elem* zr = static_cast<const elem*>(a.z) + rowoff;
        elem* orow = static_cast<elem*>(a.out) + rowoff;
        if (COLS) {
            float sv[V];
            scan_sum<V>(a, b, i, col, sv);
            int64_t j = g;
            for (; j + G < w; j += 2 * G) {
                const raw x0 = load_raw<true>(xr + j * E), z0 = load_raw<true>(zr + j * E);
                const raw x1 = load_raw<true>(xr + (j + G) * E), z1 = load_raw<true>(zr + (j + G) * E);
                emit_token<IO>(orow + j * E, x0, z0, sv, dsum);
                emit_token<IO>(orow + (j + G) * E, x1, z1, sv, dsum);
            }
            if (j < w) emit_token<IO>(orow + j * E, load_raw<true>(xr + j * E), load_raw<true>(zr + j * E), sv, dsum);
        } else {
            for (int64_t j = g; j < w; j += G) {
                const raw x0 = load_raw<true>(xr + j * E), z0 = load_raw<true>(zr + j * E);
                float sv[V];
                scan_sum<V>(a, b, j, col, sv);
                emit_token<IO>(orow + j * E, x0, z0, sv, dsum);
            }
        }
    }
}

// ---------------------------------------------------------------- kernel
template <class IO>
__device__ __forceinline__ void run_item(const FusedArgs& a, int64_t ticket, FusedSmem& sm);

// Persistent workgroups: each takes tickets in increasing order until they run
// out, so every item waits only for items taken earlier by running workgroups.
template <class IO>
__global__ void __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(8))) fused_layer_kernel(FusedArgs a) {
    __shared__ FusedSmem sm;
    __shared__ unsigned s_ticket;
    for (;;) {
        __syncthreads();  // the previous item is finished by every thread before s_ticket changes
        if (threadIdx.x == 0)
            s_ticket = __hip_atomic_fetch_add(&a.sync[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int64_t ticket = s_ticket;
        if (ticket >= a.total) return;
        run_item<IO>(a, ticket, sm);
    }
}

template <class IO>
__device__ __forceinline__ void run_item(const FusedArgs& a, int64_t ticket, FusedSmem& sm) {
    const int64_t slot = ticket / a.per_slot;
    const int r = (int)(ticket - slot * a.per_slot);
    if (r < a.nA) {
        if (slot < a.B) item_pool_proj<IO>(a, slot, r, sm.buf);
    } else if (r < a.nA + a.nS) {
        const int64_t b = slot - a.LS;
        if (b >= 0 && b < a.B) {
            if (threadIdx.x == 0) wait_at_least(&a.sync[2 + b], (unsigned)a.nA, &a.sync[1]);
            __syncthreads();
            ScanArgs sa{a.xdbl, a.pf, a.pb, a.s_f, a.s_b, a.T, a.E, a.R, a.NX};
            scan_tile(sa, USrcPooled{a.u, a.T, a.E}, b, (int64_t)(r - a.nA) * kScanCh, sm.scan);
            __syncthreads();
            if (threadIdx.x == 0) count_done(&a.sync[2 + a.B + b]);
        }
    } else {
        const int64_t b = slot - a.LE;
        if (b >= 0 && b < a.B) {
            if (a.axis == FASTVIM_POOL_COLS) item_epilogue<IO, true>(a, b, r - a.nA - a.nS);
            else item_epilogue<IO, false>(a, b, r - a.nA - a.nS);
        }
    }
}

__global__ void zero_sync_kernel(unsigned* sync, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        sync[i] = 0u;
}

int env_int(const char* name, int dflt) {
    const char* s = getenv(name);
    return s ? atoi(s) : dflt;
}

// Item sizes for a geometry; false if the fused kernel does not cover it.
bool plan(const Geom& g, FusedArgs* a) {
    if (!g.pooled || g.masked) return false;
    const int V = g.io == FASTVIM_BF16 ? 8 : 4;
    const int64_t esz = g.io == FASTVIM_BF16 ? 2 : 4;
    const int64_t VE = g.E / V;
    if (VE > kFusedThreads) return false;
    const int G = (int)(kFusedThreads / VE);
    const int64_t NO = 2 * g.NX;
    int KS = (int)(kFusedThreads / NO);
    KS = KS < 1 ? 1 : (KS > 4 ? 4 : KS);
    // A items: about 384 KB of x each, at most 8 positions, within the LDS budget.
    const int64_t pos_bytes = g.P * g.E * esz;
    int64_t RG = (384 * 1024) / (pos_bytes > 0 ? pos_bytes : 1);
    RG = RG < 1 ? 1 : (RG > 8 ? 8 : RG);
    if (RG > g.T) RG = g.T;
    while (RG > 1 && G * g.E + RG * g.E + RG * NO * KS > kLdsFloats) --RG;
    if (G * g.E + RG * g.E + RG * NO * KS > kLdsFloats) return false;
    // E items: about 256 KB of each stream.
    const int64_t row_bytes = g.w * g.E * esz;
    int64_t RE = (256 * 1024) / (row_bytes > 0 ? row_bytes : 1);
    RE = RE < 1 ? 1 : RE;
    if (RE > g.h) RE = g.h;
    a->B = g.B; a->h = g.h; a->w = g.w; a->E = g.E; a->T = g.T; a->P = g.P;
    a->R = (int)g.R; a->NX = (int)g.NX; a->axis = g.axis;
    a->VE = (int)VE; a->G = G; a->KS = KS; a->RG = (int)RG; a->RE = (int)RE;
    a->nA = (int)((g.T + RG - 1) / RG);
    a->nS = (int)((g.E + kScanCh - 1) / kScanCh);
    a->nE = (int)((g.h + RE - 1) / RE);
    a->LS = env_int("FASTVIM_FUSED_LS", 1);
    a->LE = env_int("FASTVIM_FUSED_LE", 2);
    if (a->LS < 1) a->LS = 1;
    if (a->LE < a->LS) a->LE = a->LS;
    a->per_slot = a->nA + a->nS + a->nE;
    a->total = (g.B + a->LE) * a->per_slot;
    return a->total < (int64_t)UINT32_MAX;
}

// Persistent grid: as many workgroups as can be resident at once (never more
// than there are tickets).
template <class IO>
hipError_t fused_launch_io(const FusedArgs& a, hipStream_t st) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_layer_kernel<IO>, kFusedThreads, 0);
    if (e != hipSuccess) return e;
    int64_t grid = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    if (grid > a.total) grid = a.total;
    hipLaunchKernelGGL((fused_layer_kernel<IO>), dim3((unsigned)grid), dim3(kFusedThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

bool fused_supported(const Geom& g) {
    FusedArgs a;
    return plan(g, &a);
}

hipError_t launch_zero_sync(const Workspace& ws, int64_t n, hipStream_t st) {
    hipLaunchKernelGGL(zero_sync_kernel, dim3(1), dim3(256), 0, st, ws.sync, n);
    return hipGetLastError();
}

hipError_t launch_fused(const Geom& g, const void* x, const void* z, const fastvim_params& p, const Workspace& ws,
                        void* out, hipStream_t st) {
    FusedArgs a;
    if (!plan(g, &a)) return hipErrorInvalidValue;
    a.x = x; a.z = z; a.out = out;
    a.pf = p.fwd; a.pb = p.bwd;
    a.u = ws.u; a.xdbl = ws.xdbl; a.s_f = ws.s_f; a.s_b = ws.s_b;
    a.sync = ws.sync;
    return g.io == FASTVIM_BF16 ? fused_launch_io<IoBf16>(a, st) : fused_launch_io<IoF32>(a, st);
}

}  // namespace fastvim
