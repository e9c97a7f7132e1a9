// Per-token repeat + skip + post-SSM LayerNorm + gate, shared by the
// epilogue-norm stage kernel (epilogue_norm.hip) and the single-launch
// layer's norm epilogue items (fused.hip):
//   y   = s_fwd[t] + s_bwd[t] + (D_fwd + D_bwd) x
//   out = ((y - mean(y)) / sqrt(var(y) + eps) * ln_weight + ln_bias) * silu(z)
// with mean and population variance over the token's E channels.
//
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解,
// bullet 5: repeat, skip connection, then a LayerNorm; Pith review of
// 2502.00594: VMamba's post-SSM LayerNorm, on the SSM output before the gate.
//
// A team of TL lanes (16, 32 or 64: a DPP row, half a wave or a wave) owns
// one token: lane l holds the 16-byte vectors v TL + l, v < NV, of the token,
// so each vector step of the team reads TL consecutive vectors.  Sums run
// over the team with DPP inside a row of 16 and shuffles across rows; mean
// and variance take two passes over the registers (no cancellation).
#pragma once

#include "fastvim_internal.h"

namespace fastvim {

__device__ __forceinline__ float norm_silu(float q) { return q * __builtin_amdgcn_rcpf(1.f + __expf(-q)); }

template <int CTRL>
__device__ __forceinline__ float norm_dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the TL lanes of a team; every lane of the team gets the total.
// Inside a row of 16 lanes by DPP; the row sums of a wave are then read with
// v_readlane (lanes 0, 16, 32, 48), which needs every lane of the wave
// active: teams are whole rows of a wave whose lanes all take part.
template <int TL>
__device__ __forceinline__ float team_sum(float v) {
    v += norm_dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += norm_dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += norm_dpp<0x124>(v);  // row_ror:4
    v += norm_dpp<0x128>(v);  // row_ror:8  -> sum over the row of 16
    if (TL >= 32) {
        const int vi = __float_as_int(v);  // the builtin moves 32-bit integers: pass the bits
        const float r0 = __int_as_float(__builtin_amdgcn_readlane(vi, 0));
        const float r1 = __int_as_float(__builtin_amdgcn_readlane(vi, 16));
        const float r2 = __int_as_float(__builtin_amdgcn_readlane(vi, 32));
        const float r3 = __int_as_float(__builtin_amdgcn_readlane(vi, 48));
        if (TL >= 64) v = (r0 + r1) + (r2 + r3);
        else v = (threadIdx.x & 32) ? r2 + r3 : r0 + r1;
    }
    return v;
}

// The token's x and z vectors held by this lane (non-temporal: read once).
template <class IO, int TL, int NV>
__device__ __forceinline__ void norm_load(const typename IO::elem* xb, const typename IO::elem* zb, int E, int lane,
                                          typename IO::raw (&xr)[NV], typename IO::raw (&zr)[NV]) {
    constexpr int V = IO::V;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int c = (v * TL + lane) * V;
        if (c < E) {
            xr[v] = load_raw<true>(xb + c);
            zr[v] = load_raw<true>(zb + c);
        }
    }
}

// The rest of the token: s rows, D, the norm and the gate, then the
// non-temporal store of out.  xv: the token's x values held by this lane
// (x itself, or x_conv when the producer Conv1D is computed on load).  s1,
// s2: the token's two scan rows and d1, d2 the two D vectors; SUMMED: s1
// already holds s_fwd + s_bwd and d1 holds D_fwd + D_bwd (s2, d2 unused) --
// staged in LDS by a caller that reuses them over many tokens.
template <class IO, int TL, int NV, bool SUMMED = false>
__device__ __forceinline__ void norm_finish_f(const float (&xv)[NV][IO::V], const typename IO::raw (&zr)[NV],
                                              const float* s1, const float* s2, const float* d1, const float* d2,
                                              const float* lnw, const float* lnb, float eps, typename IO::elem* ob,
                                              int E, int lane) {
    constexpr int V = IO::V;
    float y[NV][V];
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int c = (v * TL + lane) * V;
        if (c < E) {
#pragma unroll
            for (int k = 0; k < V; k += 4) {
                float sa[4], ds[4];
                const f32x4 a1 = *reinterpret_cast<const f32x4*>(s1 + c + k);
                if (SUMMED) {
                    const f32x4 dd = *reinterpret_cast<const f32x4*>(d1 + c + k);
                    sa[0] = a1.x; sa[1] = a1.y; sa[2] = a1.z; sa[3] = a1.w;
                    ds[0] = dd.x; ds[1] = dd.y; ds[2] = dd.z; ds[3] = dd.w;
                } else {
                    const f32x4 a2 = *reinterpret_cast<const f32x4*>(s2 + c + k);
                    sa[0] = a1.x + a2.x; sa[1] = a1.y + a2.y; sa[2] = a1.z + a2.z; sa[3] = a1.w + a2.w;
#pragma unroll
                    for (int q = 0; q < 4; ++q) ds[q] = d1[c + k + q] + d2[c + k + q];  // D: 4-byte aligned only
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    y[v][k + q] = fmaf(ds[q], xv[v][k + q], sa[q]);
                    sum += y[v][k + q];
                }
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
        if ((v * TL + lane) * V < E) {
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
        if (c < E) {
            float o[V];
#pragma unroll
            for (int k = 0; k < V; k += 4) {
                const f32x4 g = *reinterpret_cast<const f32x4*>(lnw + c + k);
                const f32x4 be = *reinterpret_cast<const f32x4*>(lnb + c + k);
                const float gg[4] = {g.x, g.y, g.z, g.w}, bb[4] = {be.x, be.y, be.z, be.w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    o[k + q] = fmaf((y[v][k + q] - mean) * r, gg[q], bb[q]) * norm_silu(raw_at(zr[v], k + q));
            }
            store_vec<true>(ob + c, o);
        }
    }
}

// norm_finish_f on the token's raw x vectors.
template <class IO, int TL, int NV, bool SUMMED = false>
__device__ __forceinline__ void norm_finish(const typename IO::raw (&xr)[NV], const typename IO::raw (&zr)[NV],
                                            const float* s1, const float* s2, const float* d1, const float* d2,
                                            const float* lnw, const float* lnb, float eps, typename IO::elem* ob,
                                            int E, int lane) {
    float xv[NV][IO::V];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int k = 0; k < IO::V; ++k) xv[v][k] = raw_at(xr[v], k);
    norm_finish_f<IO, TL, NV, SUMMED>(xv, zr, s1, s2, d1, d2, lnw, lnb, eps, ob, E, lane);
}

// NaN in every channel of the token (a masked token with an invalid index).
template <class IO, int TL, int NV>
__device__ __forceinline__ void norm_nan(typename IO::elem* ob, int E, int lane) {
    constexpr int V = IO::V;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int c = (v * TL + lane) * V;
        if (c < E) {
            float o[V];
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = __builtin_nanf("");
            store_vec<true>(ob + c, o);
        }
    }
}

}  // namespace fastvim
