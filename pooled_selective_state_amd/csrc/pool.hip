// Mean pooling of the post-Conv1D token grid along one spatial axis, and the
// masked (kept-token) variant.
//
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解:
// bullet 2 -- the (B, h, w, D) grid is averaged without parameters along one
// axis to (B, h, 1, D); bullet 5 -- the next block works on the transposed
// grid, so the other axis is pooled; bullet 6 -- FastMaskVim pools the kept
// tokens through their sparse indices and normalises by the fixed width.
//
// Layout: x (B, h, w, E) with E innermost; the pooled tokens u (B, T, E) fp32.
// One workgroup produces one pooled token u[b, t, :].  Its threads form G
// groups of VE vector lanes: lane c owns the 16-byte column [c*V, c*V + V) of
// E, group g sums the pooled positions p = g, g+G, ...; the G partial sums are
// combined through LDS in a fixed order, so results are deterministic.
#include "fastvim_internal.h"
#include "mask_list.h"

namespace fastvim {
namespace {

template <class IO>
__global__ void __launch_bounds__(1024)
pool_dense_kernel(const typename IO::elem* __restrict__ x, float* __restrict__ u, int64_t T, int64_t P,
                  int VE, int G, int64_t E, int64_t img_stride, int64_t t_stride, int64_t p_stride,
                  float inv_p) {
    constexpr int V = IO::V;
    extern __shared__ float red[];  // [G][VE * V]
    const int64_t bt = blockIdx.x;
    const int64_t b = bt / T, t = bt - b * T;
    const int tid = threadIdx.x;
    const int c = tid % VE, g = tid / VE;
    if (g < G) {
        using raw = typename IO::raw;
        float acc[V];
#pragma unroll
        for (int k = 0; k < V; ++k) acc[k] = 0.f;
        const typename IO::elem* base = x + b * img_stride + t * t_stride + (int64_t)c * V;
        int64_t p = g;
        // 8 loads in flight per lane, summed in a fixed pairwise order
        for (; p + 7 * G < P; p += 8 * G) {
            raw r[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) r[u] = load_raw<true>(base + (p + u * G) * p_stride);
#pragma unroll
            for (int k = 0; k < V; ++k)
                acc[k] += ((raw_at(r[0], k) + raw_at(r[1], k)) + (raw_at(r[2], k) + raw_at(r[3], k))) +
                          ((raw_at(r[4], k) + raw_at(r[5], k)) + (raw_at(r[6], k) + raw_at(r[7], k)));
        }
        for (; p < P; p += G) {
            const raw r0 = load_raw<true>(base + p * p_stride);
#pragma unroll
            for (int k = 0; k < V; ++k) acc[k] += raw_at(r0, k);
        }
#pragma unroll
        for (int k = 0; k < V; ++k) red[((int64_t)g * VE + c) * V + k] = acc[k];
    }
    __syncthreads();
    const int width = VE * V;
    for (int q = tid; q < width; q += blockDim.x) {
        float s = red[q];
        for (int gg = 1; gg < G; ++gg) s += red[gg * width + q];
        u[bt * E + q] = s * inv_p;
    }
}

// Row of every kept token and validation of the mask.  One workgroup per
// image counts the occurrences of each grid cell in LDS; an index outside
// [0, h*w) or one that occurs twice gets row -1 (its outputs become NaN).
__global__ void __launch_bounds__(256)
mask_rows_kernel(const int32_t* __restrict__ idx, int32_t* __restrict__ rows, int32_t* __restrict__ bad,
                 unsigned* __restrict__ status, int64_t K, int64_t hw, int64_t w, int axis) {
    extern __shared__ uint32_t cnt[];  // [hw]
    __shared__ uint32_t nbad;
    const int64_t b = blockIdx.x;
    if (threadIdx.x == 0) nbad = 0;
    for (int64_t q = threadIdx.x; q < hw; q += blockDim.x) cnt[q] = 0;
    __syncthreads();
    for (int64_t k = threadIdx.x; k < K; k += blockDim.x) {
        const int64_t v = idx[b * K + k];
        if (v >= 0 && v < hw) atomicAdd(&cnt[v], 1u);
    }
    __syncthreads();
    uint32_t mine = 0;
    for (int64_t k = threadIdx.x; k < K; k += blockDim.x) {
        const int64_t v = idx[b * K + k];
        const bool ok = v >= 0 && v < hw && cnt[v] == 1u;
        rows[b * K + k] = ok ? (int32_t)(axis == FASTVIM_POOL_COLS ? v / w : v % w) : -1;
        mine += ok ? 0u : 1u;
    }
    if (mine) atomicAdd(&nbad, mine);
    __syncthreads();
    if (threadIdx.x == 0) {
        bad[b] = (int32_t)nbad;
        if (status && nbad) atomicOr(status, kStatusBadIndex);
    }
}

// Masked pooling: workgroup (b, t) sums the kept tokens whose row is t and
// divides by the fixed row length P.  The image's kept tokens are taken in
// slices of blockDim.x: the slice's tokens of row t are listed first
// (mask_list.h), then group g loads list entries g, g + G, ... kB at a time.
template <class IO>
__global__ void __launch_bounds__(1024)
pool_masked_kernel(const typename IO::elem* __restrict__ x, const int32_t* __restrict__ rows,
                   float* __restrict__ u, int64_t T, int64_t K, int VE, int G, int64_t E, float inv_p) {
    constexpr int V = IO::V;
    constexpr int kB = 16 / V;  // list entries in flight per lane (64 bytes of each stream)
    extern __shared__ float red[];  // [G][VE * V]
    __shared__ int list[1024];
    __shared__ int wave_cnt[kMaxListWaves];
    const int64_t bt = blockIdx.x;
    const int64_t b = bt / T, t = bt - b * T;
    const int tid = threadIdx.x;
    const int c = tid % VE, g = tid / VE;
    float acc[V];
#pragma unroll
    for (int k = 0; k < V; ++k) acc[k] = 0.f;
    for (int64_t k0 = 0; k0 < K; k0 += blockDim.x) {
        const int n = row_token_list(rows + b * K, K, t, k0, list, wave_cnt);
        if (g >= G) continue;
        const typename IO::elem* xs = x + (b * K + k0) * E + (int64_t)c * V;
        for (int i0 = g; i0 < n; i0 += kB * G) {
            float a[kB][V];
#pragma unroll
            for (int j = 0; j < kB; ++j)
                if (i0 + j * G < n) load_vec<false>(xs + (int64_t)list[i0 + j * G] * E, a[j]);
#pragma unroll
            for (int j = 0; j < kB; ++j)
                if (i0 + j * G < n) {
#pragma unroll
                    for (int q = 0; q < V; ++q) acc[q] += a[j][q];
                }
        }
    }
    if (g < G) {
#pragma unroll
        for (int k = 0; k < V; ++k) red[((int64_t)g * VE + c) * V + k] = acc[k];
    }
    __syncthreads();
    const int width = VE * V;
    for (int q = tid; q < width; q += blockDim.x) {
        float s = red[q];
        for (int gg = 1; gg < G; ++gg) s += red[gg * width + q];
        u[bt * E + q] = s * inv_p;
    }
}

// Threads per workgroup: G groups of VE lanes, G <= P, about 512 threads.
void pick_groups(int64_t VE, int64_t P, int* G, int* threads) {
    int64_t g = 512 / VE;
    if (g < 1) g = 1;
    if (g > P) g = P;
    if (g < 1) g = 1;
    int64_t th = VE * g;
    th = (th + 63) / 64 * 64;
    *G = (int)g;
    *threads = (int)th;
}

template <class IO>
hipError_t pool_dense_t(const Geom& g, const void* x, const Workspace& ws, hipStream_t st) {
    const int64_t VE = g.E / IO::V;
    int G, threads;
    pick_groups(VE, g.P, &G, &threads);
    const size_t lds = (size_t)G * VE * IO::V * sizeof(float);
    const int64_t t_stride = g.axis == FASTVIM_POOL_COLS ? g.w * g.E : g.E;
    const int64_t p_stride = g.axis == FASTVIM_POOL_COLS ? g.E : g.w * g.E;
    hipLaunchKernelGGL(pool_dense_kernel<IO>, dim3((unsigned)(g.B * g.T)), dim3(threads), lds, st,
                       static_cast<const typename IO::elem*>(x), ws.u, g.T, g.P, (int)VE, G, g.E,
                       g.h * g.w * g.E, t_stride, p_stride, pool_norm(g));
    return hipGetLastError();
}

template <class IO>
hipError_t pool_masked_t(const Geom& g, const void* x, const Workspace& ws, hipStream_t st) {
    const int64_t VE = g.E / IO::V;
    int G, threads;
    pick_groups(VE, g.K, &G, &threads);
    const size_t lds = (size_t)G * VE * IO::V * sizeof(float);
    hipLaunchKernelGGL(pool_masked_kernel<IO>, dim3((unsigned)(g.B * g.T)), dim3(threads), lds, st,
                       static_cast<const typename IO::elem*>(x), ws.rows, ws.u, g.T, g.K, (int)VE, G, g.E,
                       pool_norm(g));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mask_rows(const Geom& g, const int32_t* idx, const Workspace& ws, unsigned* status,
                            hipStream_t st) {
    const size_t lds = (size_t)(g.h * g.w) * sizeof(uint32_t);
    hipLaunchKernelGGL(mask_rows_kernel, dim3((unsigned)g.B), dim3(256), lds, st, idx, ws.rows, ws.bad, status,
                       g.K, g.h * g.w, g.w, g.axis);
    return hipGetLastError();
}

hipError_t launch_pool(const Geom& g, const void* x, const Workspace& ws, hipStream_t st) {
    if (g.masked) return g.io == FASTVIM_BF16 ? pool_masked_t<IoBf16>(g, x, ws, st) : pool_masked_t<IoF32>(g, x, ws, st);
    return g.io == FASTVIM_BF16 ? pool_dense_t<IoBf16>(g, x, ws, st) : pool_dense_t<IoF32>(g, x, ws, st);
}

}  // namespace fastvim
