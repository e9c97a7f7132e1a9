// Input-dependent projection of every scanned token, both directions at once:
//   xdbl[m, d, o] = sum_e x_proj_w^d[o, e] * u[m, e],   o < NX = R + 2N
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解,
// bullet 3: Linear_N produces the input-dependent B, C and the input of the
// step size.  m runs over the B*T scanned tokens: pooled tokens (fp32 u) or,
// unpooled, the grid tokens of x in scan order.
//
// A workgroup computes a 32-row x 2NX tile.  E is walked in chunks of 32; the
// row chunk and both weight chunks are staged in LDS (k-major, so the inner
// loop reads broadcasts of u and conflict-free runs of weights), and each
// thread accumulates 2 rows x CPT columns in registers.
#include "fastvim_internal.h"

namespace fastvim {
namespace {

constexpr int kMT = 32;     // rows per workgroup
constexpr int kKC = 32;     // E chunk

__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
    f32x4 t = *reinterpret_cast<const f32x4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void load4(const uint16_t* p, float (&v)[4]) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2 t = *reinterpret_cast<const u32x2*>(p);
    v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xffff0000u);
    v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xffff0000u);
}

template <class Elem, int CPT>
__global__ void __launch_bounds__(256)
proj_kernel(const Elem* __restrict__ src, int map_axis, int64_t M, int64_t T, int64_t h, int64_t w, int64_t E,
            const float* __restrict__ Wf, const float* __restrict__ Wb, int NX, float* __restrict__ xdbl) {
    __shared__ float Us[kKC][kMT + 1];
    __shared__ float Ws[kKC][16 * CPT];
    const int NO = 2 * NX;
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int64_t m0 = (int64_t)blockIdx.x * kMT;

    // Load-phase role: row lr of the tile, 4 consecutive k at kq * 4.
    const int lr = tid >> 3, kq = tid & 7;
    const int64_t lm = m0 + lr;
    const Elem* rowp = nullptr;
    if (lm < M) {
        int64_t tok = lm;  // pooled tokens and row-major order: row m is token m
        if (map_axis == FASTVIM_POOL_NONE_COLMAJOR) {
            const int64_t b = lm / T, t = lm - b * T;
            tok = b * h * w + unpooled_token(map_axis, t, h, w);
        }
        rowp = src + tok * E;
    }

    float acc[2][CPT];
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[0][c] = acc[1][c] = 0.f;

    for (int64_t k0 = 0; k0 < E; k0 += kKC) {
        {
            float a[4] = {0.f, 0.f, 0.f, 0.f};
            const int64_t kk = k0 + kq * 4;
            if (rowp && kk < E) load4(rowp + kk, a);
#pragma unroll
            for (int q = 0; q < 4; ++q) Us[kq * 4 + q][lr] = a[q];
        }
        for (int q = tid; q < 16 * CPT * (kKC / 4); q += 256) {
            const int o = q >> 3, kq2 = q & 7;
            const int64_t kk = k0 + kq2 * 4;
            float a[4] = {0.f, 0.f, 0.f, 0.f};
            if (o < NO && kk < E) load4((o < NX ? Wf + (int64_t)o * E : Wb + (int64_t)(o - NX) * E) + kk, a);
#pragma unroll
            for (int r = 0; r < 4; ++r) Ws[kq2 * 4 + r][o] = a[r];
        }
        __syncthreads();
#pragma unroll 8
        for (int k = 0; k < kKC; ++k) {
            const float a0 = Us[k][ty], a1 = Us[k][ty + 16];
#pragma unroll
            for (int c = 0; c < CPT; ++c) {
                const float wv = Ws[k][tx + 16 * c];
                acc[0][c] = fmaf(a0, wv, acc[0][c]);
                acc[1][c] = fmaf(a1, wv, acc[1][c]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int64_t m = m0 + ty + 16 * r;
        if (m >= M) continue;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
            const int o = tx + 16 * c;
            if (o < NO) xdbl[m * NO + o] = acc[r][c];
        }
    }
}

template <class Elem, int CPT>
hipError_t proj_launch(const Elem* src, int map_axis, const Geom& g, const fastvim_params& p, const Workspace& ws,
                       hipStream_t st) {
    const int64_t M = g.B * g.T;
    const unsigned blocks = (unsigned)((M + kMT - 1) / kMT);
    hipLaunchKernelGGL((proj_kernel<Elem, CPT>), dim3(blocks), dim3(256), 0, st, src, map_axis, M, g.T, g.h, g.w,
                       g.E, p.fwd.x_proj_w, p.bwd.x_proj_w, (int)g.NX, ws.xdbl);
    return hipGetLastError();
}

template <class Elem>
hipError_t proj_dispatch(const Elem* src, int map_axis, const Geom& g, const fastvim_params& p,
                         const Workspace& ws, hipStream_t st) {
    const int cpt = (int)((2 * g.NX + 15) / 16);
    switch (cpt) {
#define FASTVIM_CPT(n) \
    case n: return proj_launch<Elem, n>(src, map_axis, g, p, ws, st);
        FASTVIM_CPT(5) FASTVIM_CPT(6) FASTVIM_CPT(7) FASTVIM_CPT(8) FASTVIM_CPT(9) FASTVIM_CPT(10)
        FASTVIM_CPT(11) FASTVIM_CPT(12)
#undef FASTVIM_CPT
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_proj(const Geom& g, const void* x, const fastvim_params& p, const Workspace& ws,
                       hipStream_t st) {
    if (g.pooled) return proj_dispatch<float>(ws.u, FASTVIM_POOL_COLS, g, p, ws, st);
    if (g.io == FASTVIM_BF16) return proj_dispatch<uint16_t>(static_cast<const uint16_t*>(x), g.axis, g, p, ws, st);
    return proj_dispatch<float>(static_cast<const float*>(x), g.axis, g, p, ws, st);
}

}  // namespace fastvim
