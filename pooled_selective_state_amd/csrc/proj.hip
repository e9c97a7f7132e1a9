// Input-dependent projection of every scanned token, both directions at once:
//   xdbl[m, d, o] = sum_e x_proj_w^d[o, e] * u[m, e],   o < NX = R + 2N
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解,
// bullet 3: Linear_N produces the input-dependent B, C and the input of the
// step size.  m runs over the B*T scanned tokens: pooled tokens (fp32 u) or,
// unpooled, the grid tokens of x in scan order.
//
// A dense (M x E) . (E x 2NX) contraction on the matrix cores: fp32
// v_mfma_f32_16x16x4f32 (fp32 products and sums, so results stay within fp32
// rounding of the plain dot products).  One 256-thread workgroup owns 16 rows
// and every output column (CT tiles of 16); its four waves take interleaved
// 16-wide steps of E, and their partial tiles are summed through LDS in a
// fixed order (deterministic).  Per step a lane loads one 16-byte run of its
// row (row lane % 16, k = 4 (lane / 16) .. +3) and one of each column tile's
// weight row, and feeds them to 4 MFMAs per tile: lane l supplies
// A[l % 16][l / 16] and B[l / 16][l % 16], and MFMA i of the step covers
// k = k0 + 4 (l / 16) + i for both operands.  Accumulator register r of lane
// l holds output row 4 (l / 16) + r, column l % 16.
#include "fastvim_internal.h"

namespace fastvim {
namespace {

constexpr int kPW = 4;  // waves per workgroup

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

template <class Elem, int CT>
__global__ void __launch_bounds__(64 * kPW)
proj_kernel(const Elem* __restrict__ src, int map_axis, int64_t M, int64_t T, int64_t h, int64_t w, int64_t E,
            const float* __restrict__ Wf, const float* __restrict__ Wb, int NX, float* __restrict__ xdbl) {
    __shared__ float red[kPW][CT][256];  // each wave's partial tiles, [lane * 4 + r]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int ri = lane & 15, kk = lane >> 4;
    const int NO = 2 * NX;
    const int64_t m0 = (int64_t)blockIdx.x * 16;

    const int64_t m = m0 + ri;
    const Elem* rowp = nullptr;
    if (m < M) {
        int64_t tok = m;  // pooled tokens and row-major order: row m is token m
        if (map_axis == FASTVIM_POOL_NONE_COLMAJOR) {
            const int64_t b = m / T, t = m - b * T;
            tok = b * h * w + unpooled_token(map_axis, t, h, w);
        }
        rowp = src + tok * E;
    }
    const float* wrow[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int o = ct * 16 + ri;
        wrow[ct] = o < NX ? Wf + (int64_t)o * E : (o < NO ? Wb + (int64_t)(o - NX) * E : nullptr);
    }

    f32x4 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    // operands of the next step are loaded while the current step's MFMAs run
    float a4[4], b4[CT][4];
    auto load_step = [&](int64_t k0) {
        const int64_t k = k0 + 4 * kk;  // E is a multiple of 4: a run is all in or all out
        a4[0] = a4[1] = a4[2] = a4[3] = 0.f;
        if (rowp && k < E) load4(rowp + k, a4);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            b4[ct][0] = b4[ct][1] = b4[ct][2] = b4[ct][3] = 0.f;
            if (wrow[ct] && k < E) load4(wrow[ct] + k, b4[ct]);
        }
    };
    int64_t k0 = 16 * wv;
    load_step(k0);
    for (; k0 < E; k0 += 16 * kPW) {
        float a[4], b[CT][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = a4[i];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) b[ct][i] = b4[ct][i];
        if (k0 + 16 * kPW < E) load_step(k0 + 16 * kPW);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[ct][i], acc[ct], 0, 0, 0);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wv][ct][lane * 4 + r] = acc[ct][r];
    __syncthreads();
    // row-major walk of each 16 x 16 tile, so consecutive threads store consecutive columns
    for (int e = threadIdx.x; e < CT * 256; e += 64 * kPW) {
        const int ct = e >> 8, i = (e >> 4) & 15, j = e & 15;
        const int src_idx = (16 * (i >> 2) + j) * 4 + (i & 3);
        float v = red[0][ct][src_idx];
#pragma unroll
        for (int q = 1; q < kPW; ++q) v += red[q][ct][src_idx];
        const int64_t mm = m0 + i;
        const int o = ct * 16 + j;
        if (mm < M && o < NO) xdbl[mm * NO + o] = v;
    }
}

template <class Elem, int CT>
hipError_t proj_launch(const Elem* src, int map_axis, const Geom& g, const fastvim_params& p, const Workspace& ws,
                       hipStream_t st) {
    const int64_t M = g.B * g.T;
    const unsigned blocks = (unsigned)((M + 15) / 16);
    hipLaunchKernelGGL((proj_kernel<Elem, CT>), dim3(blocks), dim3(64 * kPW), 0, st, src, map_axis, M, g.T, g.h,
                       g.w, g.E, p.fwd.x_proj_w, p.bwd.x_proj_w, (int)g.NX, ws.xdbl);
    return hipGetLastError();
}

template <class Elem>
hipError_t proj_dispatch(const Elem* src, int map_axis, const Geom& g, const fastvim_params& p,
                         const Workspace& ws, hipStream_t st) {
    const int ct = (int)((2 * g.NX + 15) / 16);  // 2NX in [66, 192]
    switch (ct) {
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
