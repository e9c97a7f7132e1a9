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
#include <type_traits>

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
            const float* __restrict__ Wf, const float* __restrict__ Wb, int NX, int nout, float* __restrict__ xdbl) {
    __shared__ float red[kPW][CT][256];  // each wave's partial tiles, [lane * 4 + r]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int ri = lane & 15, kk = lane >> 4;
    const int NO = 2 * NX;
    const int64_t m0 = (int64_t)blockIdx.x * 16;
    const int c0 = (int)blockIdx.y * CT * 16;  // this workgroup's first output column

    // Rows past M and columns past the computed ones read a valid row instead
    // (the last token, a weight row in range): their outputs are never stored,
    // so the loads need no per-lane guards.
    const int64_t m = m0 + ri < M ? m0 + ri : M - 1;
    int64_t tok = m;  // pooled tokens and row-major order: row m is token m
    if (map_axis == FASTVIM_POOL_NONE_COLMAJOR) {
        const int64_t b = m / T, t = m - b * T;
        tok = b * h * w + unpooled_token(map_axis, t, h, w);
    }
    const Elem* rowp = src + tok * E + 4 * kk;
    const float* wrow[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int o = c0 + ct * 16 + ri;
        wrow[ct] = (o < NX ? Wf + (int64_t)o * E : (o < NO ? Wb + (int64_t)(o - NX) * E : Wf)) + 4 * kk;
    }

    f32x4 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto load_step = [&](int k0, float (&av)[4], float (&bv)[CT][4]) {
        load4(rowp + k0, av);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) load4(wrow[ct] + k0, bv[ct]);
    };
    auto mfma_step = [&](const float (&av)[4], const float (&bv)[CT][4]) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[ct][i], acc[ct], 0, 0, 0);
    };
    // Full 16-wide steps of this wave (k0 = 16 wv + 64 i, k0 + 16 <= E),
    // double-buffered in two register sets: the next step's operands load
    // while the current step's MFMAs run.
    const int step = 16 * kPW;
    const int Ef = (int)(E / 16) * 16;  // end of the full steps
    float a0[4], b0[CT][4], a1[4], b1[CT][4];
    int k0 = 16 * wv;
    if (k0 < Ef) load_step(k0, a0, b0);
    for (; k0 < Ef; k0 += 2 * step) {
        const bool has1 = k0 + step < Ef;
        if (has1) load_step(k0 + step, a1, b1);
        mfma_step(a0, b0);
        if (k0 + 2 * step < Ef) load_step(k0 + 2 * step, a0, b0);
        if (has1) mfma_step(a1, b1);
    }
    // The tail of E (E % 16 != 0, a multiple of 4): one step with guarded
    // loads, taken by the wave whose turn it is.
    if (Ef < E && wv == (Ef / 16) % kPW) {
        const bool in = Ef + 4 * kk < E;
        a0[0] = a0[1] = a0[2] = a0[3] = 0.f;
        if (in) load4(rowp + Ef, a0);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            b0[ct][0] = b0[ct][1] = b0[ct][2] = b0[ct][3] = 0.f;
            if (in) load4(wrow[ct] + Ef, b0[ct]);
        }
        mfma_step(a0, b0);
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
        const int o = c0 + ct * 16 + j;
        if (mm < M && o < nout) xdbl[mm * NO + o] = v;
    }
}

// Few tokens, long E (short, wide pooled layers: the masked Vim-B layer has
// 3.6 k tokens of E = 1536): proj_kernel's 16-row workgroups each read the
// whole weight slice from L2 for 16 tokens.  Here a workgroup takes RT
// 16-row tiles, so every weight fragment it loads feeds RT tiles' MFMAs, and
// kWidePW = 8 waves take interleaved 16-wide steps of E (two waves per SIMD,
// as two proj_kernel workgroups per CU would have).  The waves' partial
// tiles are added in a fixed order: waves w and w + 4 through LDS, then the
// four sums as in proj_kernel (deterministic).  Operand layout as
// proj_kernel; pooled tokens (fp32 u, row m is token m) only.
constexpr int kWidePW = 8;

template <int CT, int RT>
__global__ void __launch_bounds__(64 * kWidePW)
proj_wide_kernel(const float* __restrict__ u, int64_t M, int64_t E, const float* __restrict__ Wf,
                 const float* __restrict__ Wb, int NX, int nout, float* __restrict__ xdbl) {
    __shared__ float red[kWidePW / 2][RT][CT][256];  // partial tiles, [lane * 4 + r]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int ri = lane & 15, kk = lane >> 4;
    const int NO = 2 * NX;
    const int64_t m0 = (int64_t)blockIdx.x * 16 * RT;
    const int c0 = (int)blockIdx.y * CT * 16;
    const float* rowp[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int64_t m = m0 + rt * 16 + ri < M ? m0 + rt * 16 + ri : M - 1;  // past M: a valid row, never stored
        rowp[rt] = u + m * E + 4 * kk;
    }
    const float* wrow[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int o = c0 + ct * 16 + ri;
        wrow[ct] = (o < NX ? Wf + (int64_t)o * E : (o < NO ? Wb + (int64_t)(o - NX) * E : Wf)) + 4 * kk;
    }
    f32x4 acc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto load_step = [&](int k0, float (&av)[RT][4], float (&bv)[CT][4]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) load4(rowp[rt] + k0, av[rt]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) load4(wrow[ct] + k0, bv[ct]);
    };
    auto mfma_step = [&](const float (&av)[RT][4], const float (&bv)[CT][4]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[rt][i], bv[ct][i], acc[rt][ct], 0, 0, 0);
    };
    // this wave's full 16-wide steps k0 = 16 wv + 16 kWidePW i, double-buffered
    const int step = 16 * kWidePW;
    const int Ef = (int)(E / 16) * 16;
    float a0[RT][4], b0[CT][4], a1[RT][4], b1[CT][4];
    int k0 = 16 * wv;
    if (k0 < Ef) load_step(k0, a0, b0);
    for (; k0 < Ef; k0 += 2 * step) {
        const bool has1 = k0 + step < Ef;
        if (has1) load_step(k0 + step, a1, b1);
        mfma_step(a0, b0);
        if (k0 + 2 * step < Ef) load_step(k0 + 2 * step, a0, b0);
        if (has1) mfma_step(a1, b1);
    }
    if (Ef < E && wv == (Ef / 16) % kWidePW) {  // the tail of E (a multiple of 4), by the wave whose turn it is
        const bool in = Ef + 4 * kk < E;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            a0[rt][0] = a0[rt][1] = a0[rt][2] = a0[rt][3] = 0.f;
            if (in) load4(rowp[rt] + Ef, a0[rt]);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            b0[ct][0] = b0[ct][1] = b0[ct][2] = b0[ct][3] = 0.f;
            if (in) load4(wrow[ct] + Ef, b0[ct]);
        }
        mfma_step(a0, b0);
    }
    // waves 4..7 hand their partials to waves 0..3, which add them to their own
    constexpr int kHalf = kWidePW / 2;
    if (wv >= kHalf) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[wv - kHalf][rt][ct][lane * 4 + r] = acc[rt][ct][r];
    }
    __syncthreads();
    if (wv < kHalf) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[rt][ct][r] += red[wv][rt][ct][lane * 4 + r];
    }
    __syncthreads();
    if (wv < kHalf) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[wv][rt][ct][lane * 4 + r] = acc[rt][ct][r];
    }
    __syncthreads();
    // row-major walk of each 16 x 16 tile, consecutive threads on consecutive columns
    for (int e = threadIdx.x; e < RT * CT * 256; e += 64 * kWidePW) {
        const int rt = e / (CT * 256), ct = (e >> 8) % CT, i = (e >> 4) & 15, j = e & 15;
        const int src_idx = (16 * (i >> 2) + j) * 4 + (i & 3);
        float v = red[0][rt][ct][src_idx];
#pragma unroll
        for (int q = 1; q < kHalf; ++q) v += red[q][rt][ct][src_idx];
        const int64_t mm = m0 + rt * 16 + i;
        const int o = c0 + ct * 16 + j;
        if (mm < M && o < nout) xdbl[mm * NO + o] = v;
    }
}

// Many tokens (unpooled layers): each wave owns RT 16-row tiles over all of
// E, so every weight fragment it loads feeds RT tiles' MFMAs (the weights are
// re-read from L2 once per 16 RT rows instead of once per 16) and no
// cross-wave reduction is needed; a workgroup's kPW waves cover 16 RT kPW rows.
// Same operand layout and out-of-range handling as proj_kernel.
template <class Elem, int CT, int RT>
__global__ void __launch_bounds__(64 * kPW)
proj_rows_kernel(const Elem* __restrict__ src, int map_axis, int64_t M, int64_t T, int64_t h, int64_t w, int64_t E,
                 const float* __restrict__ Wf, const float* __restrict__ Wb, int NX, int nout,
                 float* __restrict__ xdbl) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int ri = lane & 15, kk = lane >> 4;
    const int NO = 2 * NX;
    const int64_t m0 = ((int64_t)blockIdx.x * kPW + wv) * 16 * RT;
    if (m0 >= M) return;
    const Elem* rowp[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int64_t m = m0 + rt * 16 + ri < M ? m0 + rt * 16 + ri : M - 1;
        int64_t tok = m;
        if (map_axis == FASTVIM_POOL_NONE_COLMAJOR) {
            const int64_t b = m / T, t = m - b * T;
            tok = b * h * w + unpooled_token(map_axis, t, h, w);
        }
        rowp[rt] = src + tok * E + 4 * kk;
    }
    const float* wrow[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        const int o = ct * 16 + ri;
        wrow[ct] = (o < NX ? Wf + (int64_t)o * E : (o < NO ? Wb + (int64_t)(o - NX) * E : Wf)) + 4 * kk;
    }
    f32x4 acc[RT][CT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) acc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto load_step = [&](int k0, float (&av)[RT][4], float (&bv)[CT][4]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) load4(rowp[rt] + k0, av[rt]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) load4(wrow[ct] + k0, bv[ct]);
    };
    auto mfma_step = [&](const float (&av)[RT][4], const float (&bv)[CT][4]) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[rt][i], bv[ct][i], acc[rt][ct], 0, 0, 0);
    };
    const int Ef = (int)(E / 16) * 16;
    float a0[RT][4], b0[CT][4], a1[RT][4], b1[CT][4];
    int k0 = 0;
    if (k0 < Ef) load_step(k0, a0, b0);
    for (; k0 < Ef; k0 += 32) {
        const bool has1 = k0 + 16 < Ef;
        if (has1) load_step(k0 + 16, a1, b1);
        mfma_step(a0, b0);
        if (k0 + 32 < Ef) load_step(k0 + 32, a0, b0);
        if (has1) mfma_step(a1, b1);
    }
    if (Ef < E) {  // tail of E (a multiple of 4)
        const bool in = Ef + 4 * kk < E;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            a0[rt][0] = a0[rt][1] = a0[rt][2] = a0[rt][3] = 0.f;
            if (in) load4(rowp[rt] + Ef, a0[rt]);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            b0[ct][0] = b0[ct][1] = b0[ct][2] = b0[ct][3] = 0.f;
            if (in) load4(wrow[ct] + Ef, b0[ct]);
        }
        mfma_step(a0, b0);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t mm = m0 + rt * 16 + 4 * kk + r;
                const int o = ct * 16 + ri;
                if (mm < M && o < nout) xdbl[mm * NO + o] = acc[rt][ct][r];
            }
}

constexpr int kRowsRT = 2;                       // row tiles per wave in proj_rows_kernel
constexpr int64_t kRowsMinTokens = 64 * 1024;    // token count from which it is used
constexpr int kColSplit = 2;                     // column groups per row tile when row tiles are few ...
constexpr int64_t kColSplitBelow = 512;          // ... fewer than this (two workgroups per CU)
constexpr int kWideRT = 2;                       // row tiles per workgroup of proj_wide_kernel ...
constexpr int64_t kWideMinE = 1024;              // ... for E of at least this ...
constexpr int64_t kWideMinGroups = 192;          // ... when that still gives this many workgroups

template <class Elem, int CT>
hipError_t proj_launch(const Elem* src, int map_axis, const Geom& g, const fastvim_params& p, const Workspace& ws,
                       int nout, hipStream_t st) {
    const int64_t M = g.B * g.T;
    if (M < kRowsMinTokens && CT > 1) {
        // Few 16-row tiles: split the output columns over kColSplit
        // workgroups per row tile, so that there are enough workgroups (two
        // waves per SIMD) for the MFMAs of one to run while another waits for
        // its next operands.
        const int64_t rt = (M + 15) / 16;
        if (rt < kColSplitBelow) {
            constexpr int CTS = (CT + kColSplit - 1) / kColSplit;
            const int ns = (CT + CTS - 1) / CTS;
            const int64_t rt2 = (M + 16 * kWideRT - 1) / (16 * kWideRT);
            if (std::is_same<Elem, float>::value && map_axis == FASTVIM_POOL_COLS && g.E >= kWideMinE &&
                rt2 * ns >= kWideMinGroups) {
                // pooled tokens of a short, wide layer
                hipLaunchKernelGGL((proj_wide_kernel<CTS, kWideRT>), dim3((unsigned)rt2, (unsigned)ns),
                                   dim3(64 * kWidePW), 0, st, reinterpret_cast<const float*>(src), M, g.E,
                                   p.fwd.x_proj_w, p.bwd.x_proj_w, (int)g.NX, nout, ws.xdbl);
                return hipGetLastError();
            }
            hipLaunchKernelGGL((proj_kernel<Elem, CTS>), dim3((unsigned)rt, (unsigned)ns), dim3(64 * kPW), 0, st, src,
                               map_axis, M, g.T, g.h, g.w, g.E, p.fwd.x_proj_w, p.bwd.x_proj_w, (int)g.NX, nout,
                               ws.xdbl);
            return hipGetLastError();
        }
    }
    if (M >= kRowsMinTokens) {
        const int64_t rows = 16 * kRowsRT * kPW;
        hipLaunchKernelGGL((proj_rows_kernel<Elem, CT, kRowsRT>), dim3((unsigned)((M + rows - 1) / rows)),
                           dim3(64 * kPW), 0, st, src, map_axis, M, g.T, g.h, g.w, g.E, p.fwd.x_proj_w,
                           p.bwd.x_proj_w, (int)g.NX, nout, ws.xdbl);
    } else {
        hipLaunchKernelGGL((proj_kernel<Elem, CT>), dim3((unsigned)((M + 15) / 16)), dim3(64 * kPW), 0, st, src,
                           map_axis, M, g.T, g.h, g.w, g.E, p.fwd.x_proj_w, p.bwd.x_proj_w, (int)g.NX, nout,
                           ws.xdbl);
    }
    return hipGetLastError();
}

// Both directions' columns (2 NX), or only the forward direction's (NX) when
// LBMamba's local backward scan shares the forward projection.
template <class Elem>
hipError_t proj_dispatch(const Elem* src, int map_axis, const Geom& g, const fastvim_params& p,
                         const Workspace& ws, hipStream_t st) {
    const int nout = (int)((p.flags & FASTVIM_FLAG_LOCAL_BWD) ? g.NX : 2 * g.NX);  // in [33, 192]
    const int ct = (nout + 15) / 16;
    switch (ct) {
#define FASTVIM_CPT(n) \
    case n: return proj_launch<Elem, n>(src, map_axis, g, p, ws, nout, st);
        FASTVIM_CPT(3) FASTVIM_CPT(4) FASTVIM_CPT(5) FASTVIM_CPT(6) FASTVIM_CPT(7) FASTVIM_CPT(8)
        FASTVIM_CPT(9) FASTVIM_CPT(10) FASTVIM_CPT(11) FASTVIM_CPT(12)
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
