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

// Masked layers with at most kImgMaxK kept tokens per image: mask rows and
// pooling in one launch, one 1024-thread workgroup per image.
//   1. as mask_rows_kernel: LDS occurrence counts of the grid cells, the row
//      of every kept token (-1 if out of range or repeated), the image's
//      invalid count;
//   2. per-row token lists in LDS, in increasing k: a token's place in its
//      row's list is the number of valid tokens of that row before it;
//   3. lane group g of G = blockDim / VE takes rows g, g + G, ...: lane c
//      loads the 16-byte column c of the row's listed tokens kB at a time and
//      adds them in list order, then writes u[b, row] = sum * pool_scale / P
//      (an empty row pools to 0).
// The row sums come out in token order, deterministically; one workgroup per
// image replaces B*T small workgroups whose fixed costs (a list built with
// barriers per row, an LDS reduction) outweighed their few loads.
constexpr int kImgThreads = 1024;
constexpr int64_t kImgMaxK = kImgThreads;

template <class IO>
__global__ void __launch_bounds__(kImgThreads)
pool_masked_image_kernel(const typename IO::elem* __restrict__ x, const int32_t* __restrict__ idx,
                         int32_t* __restrict__ rows, int32_t* __restrict__ bad, unsigned* __restrict__ status,
                         float* __restrict__ u, int64_t T, int64_t K, int64_t hw, int64_t w, int axis, int VE,
                         int64_t E, float inv_p) {
    constexpr int V = IO::V;
    constexpr int kB = 8;                    // listed tokens in flight per lane
    extern __shared__ uint32_t sm[];         // cnt[hw], then rowk[K], list[K], rcnt[T], rstart[T]
    uint32_t* cnt = sm;
    int* rowk = reinterpret_cast<int*>(sm + hw);
    int* list = rowk + K;
    int* rcnt = list + K;
    int* rstart = rcnt + T;
    __shared__ uint32_t nbad;
    const int64_t b = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid == 0) nbad = 0;
    for (int64_t q = tid; q < hw; q += blockDim.x) cnt[q] = 0;
    for (int64_t q = tid; q < T; q += blockDim.x) rcnt[q] = 0;
    __syncthreads();
    // 1. validation and rows (K <= blockDim: one token per thread)
    const bool has = tid < K;
    const int64_t v = has ? idx[b * K + tid] : -1;
    if (has && v >= 0 && v < hw) atomicAdd(&cnt[v], 1u);
    __syncthreads();
    int r = -1;
    if (has) {
        const bool ok = v >= 0 && v < hw && cnt[v] == 1u;
        r = ok ? (int)(axis == FASTVIM_POOL_COLS ? v / w : v % w) : -1;
        rows[b * K + tid] = r;
        rowk[tid] = r;
        if (!ok) atomicAdd(&nbad, 1u);
        else atomicAdd(&rcnt[r], 1);
    }
    __syncthreads();
    if (tid == 0) {
        bad[b] = (int32_t)nbad;
        if (status && nbad) atomicOr(status, kStatusBadIndex);
        int acc = 0;
        for (int64_t t = 0; t < T; ++t) {
            rstart[t] = acc;
            acc += rcnt[t];
        }
    }
    __syncthreads();
    // 2. per-row lists in token order
    if (r >= 0) {
        int rank = 0;
        for (int k = 0; k < tid; ++k) rank += rowk[k] == r ? 1 : 0;
        list[rstart[r] + rank] = tid;
    }
    __syncthreads();
    // 3. row sums
    const int G = (int)(blockDim.x / VE);
    const int c = tid % VE, g = tid / VE;
    if (g >= G) return;
    const typename IO::elem* xs = x + b * K * E + (int64_t)c * V;
    float* ub = u + b * T * E + (int64_t)c * V;
    for (int64_t t = g; t < T; t += G) {
        const int n = rcnt[t], s0 = rstart[t];
        float acc[V];
#pragma unroll
        for (int q = 0; q < V; ++q) acc[q] = 0.f;
        for (int i0 = 0; i0 < n; i0 += kB) {
            float a[kB][V];
#pragma unroll
            for (int j = 0; j < kB; ++j)
                if (i0 + j < n) load_vec<false>(xs + (int64_t)list[s0 + i0 + j] * E, a[j]);
#pragma unroll
            for (int j = 0; j < kB; ++j)
                if (i0 + j < n) {
#pragma unroll
                    for (int q = 0; q < V; ++q) acc[q] += a[j][q];
                }
        }
#pragma unroll
        for (int q = 0; q < V; q += 4)
            *reinterpret_cast<f32x4*>(ub + t * E + q) =
                f32x4{acc[q] * inv_p, acc[q + 1] * inv_p, acc[q + 2] * inv_p, acc[q + 3] * inv_p};
    }
}

// Dynamic LDS bytes of pool_masked_image_kernel, or 0 when the layer does not
// fit it (more kept tokens than threads, a row's lanes wider than the
// workgroup, or more than 60 KB of cell counts and lists: with the kernel's
// static word the workgroup stays within the 64 KB it may hold).  Layers that
// do not fit take the mask-rows and per-row pooling kernels.
template <class IO>
size_t pool_masked_image_lds(const Geom& g) {
    if (g.K > kImgMaxK || g.E / IO::V > kImgThreads) return 0;
    const size_t bytes = (size_t)(g.h * g.w + 2 * g.K + 2 * g.T) * 4;
    return bytes <= 60 * 1024 ? bytes : 0;
}

template <class IO>
hipError_t pool_masked_image_t(const Geom& g, const int32_t* idx, const void* x, const Workspace& ws,
                               unsigned* status, hipStream_t st) {
    hipLaunchKernelGGL(pool_masked_image_kernel<IO>, dim3((unsigned)g.B), dim3(kImgThreads),
                       pool_masked_image_lds<IO>(g), st, static_cast<const typename IO::elem*>(x), idx, ws.rows,
                       ws.bad, status, ws.u, g.T, g.K, g.h * g.w, g.w, g.axis, (int)(g.E / IO::V), g.E,
                       pool_norm(g));
    return hipGetLastError();
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

bool mask_pool_supported(const Geom& g) {
    if (!g.masked || !g.pooled) return false;
    return g.io == FASTVIM_BF16 ? pool_masked_image_lds<IoBf16>(g) != 0 : pool_masked_image_lds<IoF32>(g) != 0;
}

hipError_t launch_mask_pool(const Geom& g, const int32_t* idx, const void* x, const Workspace& ws,
                            unsigned* status, hipStream_t st) {
    return g.io == FASTVIM_BF16 ? pool_masked_image_t<IoBf16>(g, idx, x, ws, status, st)
                                : pool_masked_image_t<IoF32>(g, idx, x, ws, status, st);
}

hipError_t launch_pool(const Geom& g, const void* x, const Workspace& ws, hipStream_t st) {
    if (g.masked) return g.io == FASTVIM_BF16 ? pool_masked_t<IoBf16>(g, x, ws, st) : pool_masked_t<IoF32>(g, x, ws, st);
    return g.io == FASTVIM_BF16 ? pool_dense_t<IoBf16>(g, x, ws, st) : pool_dense_t<IoF32>(g, x, ws, st);
}

}  // namespace fastvim
