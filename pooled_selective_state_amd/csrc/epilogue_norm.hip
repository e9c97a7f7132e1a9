// Repeat + skip + post-SSM LayerNorm + gate: every output token written once,
//   y   = s_fwd[b, t] + s_bwd[b, t] + (D_fwd + D_bwd) x[b, cell]
//   out = ((y - mean(y)) / sqrt(var(y) + eps) * ln_weight + ln_bias) * silu(z[b, cell])
// with mean and (population) variance over the token's E channels and t the
// scan position of the cell (its row, its column, its raster position, or a
// kept token's row).
//
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解,
// bullet 5: the scan output is repeated, the skip connection added, then a
// LayerNorm; Pith review of 2502.00594: the post-SSM LayerNorm taken from
// VMamba, on the SSM output before the gate; Vim article (ijyty.com) 2.1:
// the two directions summed and gated by z.
//
// The norm needs all E channels of a token at once, so a team of TL lanes
// (16, 32 or 64; a DPP row, half a wave or a wave) owns one token: lane l of
// the team holds the 16-byte vectors v = 0 .. nv-1 at channel (v TL + l) V,
// so every vector step of the team reads TL consecutive vectors.  The team
// sums over its lanes with DPP inside a row of 16 and shuffles across rows;
// mean and variance take two passes over the registers (no cancellation).
// x and z are read for the last time (non-temporal), out written once
// (non-temporal); the scan rows and the per-channel vectors come through the
// caches.
#include "fastvim_internal.h"

namespace fastvim {
namespace {

enum { kModeCols = 0, kModeRows = 1, kModeNoneRow = 2, kModeNoneCol = 3, kModeMasked = 4 };
constexpr int kNormThreads = 256;

__device__ __forceinline__ float silu(float q) { return q * __builtin_amdgcn_rcpf(1.f + __expf(-q)); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the TL lanes of a team; every lane of the team gets the total.
template <int TL>
__device__ __forceinline__ float team_sum(float v) {
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x124>(v);  // row_ror:4
    v += dpp<0x128>(v);  // row_ror:8  -> sum over the row of 16
    if (TL >= 32) v += __shfl_xor(v, 16);
    if (TL >= 64) v += __shfl_xor(v, 32);
    return v;
}

// V floats: 16-byte vector loads (16-byte aligned data: scan rows, norm
// parameters) or plain loads (D, 4-byte aligned).
template <class IO>
__device__ __forceinline__ void load_f(const float* p, float (&v)[IO::V]) {
#pragma unroll
    for (int k = 0; k < IO::V; k += 4) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(p + k);
        v[k] = t.x; v[k + 1] = t.y; v[k + 2] = t.z; v[k + 3] = t.w;
    }
}

template <class IO>
__device__ __forceinline__ void load_f_scalar(const float* p, float (&v)[IO::V]) {
#pragma unroll
    for (int k = 0; k < IO::V; ++k) v[k] = p[k];
}

template <class IO, int TL, int NV>
__global__ void __launch_bounds__(kNormThreads)
epilogue_norm_kernel(const typename IO::elem* __restrict__ x, const typename IO::elem* __restrict__ z,
                     const float* __restrict__ sf, const float* __restrict__ sb, const float* __restrict__ Df,
                     const float* __restrict__ Db, const float* __restrict__ lnw, const float* __restrict__ lnb,
                     float eps, typename IO::elem* __restrict__ out, const int32_t* __restrict__ rows, int mode,
                     int64_t ntok, int64_t T, int64_t h, int64_t w, int64_t K, int E) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    constexpr int kTeams = kNormThreads / TL;
    const int lane = threadIdx.x % TL;
    const int64_t tok = (int64_t)blockIdx.x * kTeams + threadIdx.x / TL;  // team-uniform
    if (tok >= ntok) return;  // whole teams leave together; no barriers below
    // scan row of the token
    int64_t b, t;
    if (mode == kModeMasked) {
        b = tok / K;
        t = rows[tok];
    } else {
        const int64_t hw = h * w;
        b = tok / hw;
        const int64_t cell = tok - b * hw, i = cell / w, j = cell - i * w;
        t = mode == kModeCols ? i : mode == kModeRows ? j : mode == kModeNoneRow ? cell : j * h + i;
    }
    const int nv = (E / V + TL - 1) / TL;  // vectors of this lane's team per token (<= NV)
    typename IO::elem* ob = out + tok * E;
    if (t < 0) {  // masked token with an invalid index
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int c = (v * TL + lane) * V;
            if (v < nv && c < E) {
                float o[V];
#pragma unroll
                for (int k = 0; k < V; ++k) o[k] = __builtin_nanf("");
                store_vec<true>(ob + c, o);
            }
        }
        return;
    }
    const typename IO::elem* xb = x + tok * E;
    const typename IO::elem* zb = z + tok * E;
    const float* s1 = sf + (b * T + t) * E;
    const float* s2 = sb + (b * T + t) * E;
    raw xr[NV], zr[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int c = (v * TL + lane) * V;
        if (v < nv && c < E) {
            xr[v] = load_raw<true>(xb + c);
            zr[v] = load_raw<true>(zb + c);
        }
    }
    float y[NV][V];
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int c = (v * TL + lane) * V;
        if (v < nv && c < E) {
            float a1[V], a2[V], d1[V], d2[V];
            load_f<IO>(s1 + c, a1);
            load_f<IO>(s2 + c, a2);
            load_f_scalar<IO>(Df + c, d1);
            load_f_scalar<IO>(Db + c, d2);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                y[v][k] = a1[k] + a2[k] + (d1[k] + d2[k]) * raw_at(xr[v], k);
                sum += y[v][k];
            }
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) y[v][k] = 0.f;
        }
    }
    const float inv_e = 1.f / (float)E;
    const float mean = team_sum<TL>(sum) * inv_e;
    float sq = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int c = (v * TL + lane) * V;
        if (v < nv && c < E) {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float d = y[v][k] - mean;
                sq = fmaf(d, d, sq);
            }
        }
    }
    const float r = __builtin_amdgcn_rsqf(team_sum<TL>(sq) * inv_e + eps);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int c = (v * TL + lane) * V;
        if (v < nv && c < E) {
            float g[V], be[V], o[V];
            load_f<IO>(lnw + c, g);
            load_f<IO>(lnb + c, be);
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = ((y[v][k] - mean) * r * g[k] + be[k]) * silu(raw_at(zr[v], k));
            store_vec<true>(ob + c, o);
        }
    }
}

template <class IO, int TL, int NV>
hipError_t norm_launch(const Geom& g, const void* x, const void* z, const fastvim_params& p, const Workspace& ws,
                       void* out, hipStream_t st) {
    using elem = typename IO::elem;
    int mode;
    if (g.masked) mode = kModeMasked;
    else if (g.axis == FASTVIM_POOL_COLS) mode = kModeCols;
    else if (g.axis == FASTVIM_POOL_ROWS) mode = kModeRows;
    else if (g.axis == FASTVIM_POOL_NONE_ROWMAJOR) mode = kModeNoneRow;
    else mode = kModeNoneCol;
    const int64_t ntok = g.B * (g.masked ? g.K : g.h * g.w);
    constexpr int kTeams = kNormThreads / TL;
    hipLaunchKernelGGL((epilogue_norm_kernel<IO, TL, NV>), dim3((unsigned)((ntok + kTeams - 1) / kTeams)),
                       dim3(kNormThreads), 0, st, static_cast<const elem*>(x), static_cast<const elem*>(z), ws.s_f,
                       ws.s_b, p.fwd.D, p.bwd.D, p.ln_weight, p.ln_bias, p.ln_eps, static_cast<elem*>(out), ws.rows,
                       mode, ntok, g.T, g.h, g.w, g.K, (int)g.E);
    return hipGetLastError();
}

// The smallest team whose lanes hold a token in at most 8 vectors each (16
// for fp32 E > 2048): fewer idle lanes for narrow layers, fewer registers for
// wide ones.
template <class IO>
hipError_t norm_dispatch(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                         const Workspace& ws, void* out, hipStream_t st) {
    const int64_t vecs = g.E / IO::V;
    if (vecs <= 16 * 8) return norm_launch<IO, 16, 8>(g, x, z, p, ws, out, st);
    if (vecs <= 32 * 8) return norm_launch<IO, 32, 8>(g, x, z, p, ws, out, st);
    if (vecs <= 64 * 8) return norm_launch<IO, 64, 8>(g, x, z, p, ws, out, st);
    return norm_launch<IO, 64, 16>(g, x, z, p, ws, out, st);  // fp32, E <= 4096
}

}  // namespace

hipError_t launch_epilogue_norm(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                                const Workspace& ws, void* out, hipStream_t st) {
    return g.io == FASTVIM_BF16 ? norm_dispatch<IoBf16>(g, x, z, p, ws, out, st)
                                : norm_dispatch<IoF32>(g, x, z, p, ws, out, st);
}

}  // namespace fastvim
