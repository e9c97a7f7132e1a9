// Backward pass of the output of a pooled layer with the post-SSM LayerNorm
// (the forward arithmetic is in epilogue_norm.h; FastVim summary page,
// gptget.net, arXiv 2502.00594, section 方法详解, bullet 5: repeat, skip, then
// the LayerNorm, then the gate).  Per cell, with y = s_fwd[t] + s_bwd[t] +
// (D_fwd + D_bwd) x, its mean and population variance over the E channels,
// r = 1 / sqrt(var + eps), n = (y - mean) r, o = n ln_w + ln_b and
// out = o silu(z):
//   go  = dout silu(z),   dz = dout o silu'(z)
//   dn  = go ln_w,        g  = dL/dy = r (dn - mean(dn) - n mean(dn n))
//   gs[b, t] = sum of g over the cells of scan position t (both scans' adjoint input)
//   dD  = sum of g x,  d ln_w = sum of go n,  d ln_b = sum of go  (over all cells)
//   dx  = g (D_fwd + D_bwd) + du[b, t] / P
// g needs the scan outputs, so the caller runs the forward pool, projections
// and scans first.  Pass 1 (one workgroup per scan position (b, t)) reads x, z
// and dout once, writes dz, leaves g in dx, and writes gs and the (b, t)
// partial sums of dD, d ln_w and d ln_b; pass 2, after the scan adjoint has
// produced du, turns g into dx in place.
#include "bwd_internal.h"
#include "conv_common.h"
#include "epilogue_norm.h"
#include "mask_list.h"

namespace fastvim {
namespace {

constexpr int kNormBwdThreads = 256;

__device__ __forceinline__ float nb_sigmoid(float q) { return __builtin_amdgcn_rcpf(1.f + __expf(-q)); }

// Team partial sums of the workgroup: acc of each team goes through LDS and
// the kTeams values of a channel are added in team order into dst[0, E).
template <int TL, int NV, int V>
__device__ __forceinline__ void team_reduce_out(const float (&acc)[NV][V], float* red, float* __restrict__ dst,
                                                int E, int team, int lane) {
    constexpr int kTeams = kNormBwdThreads / TL;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int c = (v * TL + lane) * V;
        if (c < E) {
#pragma unroll
            for (int k = 0; k < V; ++k) red[team * E + c + k] = acc[v][k];
        }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < E; q += kNormBwdThreads) {
        float s = red[q];
        for (int tt = 1; tt < kTeams; ++tt) s += red[tt * E + q];
        dst[q] = s;
    }
    __syncthreads();
}

// Pass 1.  Workgroup (b, t); teams of TL lanes take the cells of scan position
// t one token at a time (lane l holds the 16-byte vectors v TL + l, v < NV, of
// the token, as in the forward norm).  MASKED: the cells are the image's kept
// tokens whose row is t, listed per slice of kNormBwdThreads tokens
// (mask_list.h); dense: cell p of the row or column, p < P.  LDS: the summed
// scan row, D_fwd + D_bwd, ln_w, ln_b (E each) and, with CONV, the conv's
// taps and bias (5 E) while the tokens are taken, then kTeams rows of E for
// the team sums.  CONV (dense layers): x is the producer Conv1D's input and
// the kernel computes x_conv where it reads x.
// x and dz may be one buffer (a layer whose conv output is written out passes
// it in dz): each cell's x is read before that cell's dz is written, so those
// two pointers carry no restrict.
template <class IO, int TL, int NV, bool MASKED, bool CONV>
__global__ void __launch_bounds__(kNormBwdThreads)
bwd_norm_pass1_kernel(const typename IO::elem* x, const typename IO::elem* __restrict__ z,
                      const typename IO::elem* __restrict__ dout, const float* __restrict__ sf,
                      const float* __restrict__ sb, const float* __restrict__ Df, const float* __restrict__ Db,
                      const float* __restrict__ lnw, const float* __restrict__ lnb, float eps,
                      const int32_t* __restrict__ rows, typename IO::elem* __restrict__ gout,
                      typename IO::elem* dz, float* __restrict__ gs, float* __restrict__ dDp,
                      float* __restrict__ dlnwp, float* __restrict__ dlnbp, int64_t T, int64_t h, int64_t w,
                      int64_t K, int64_t P, int cols_axis, int E, const float* __restrict__ cw,
                      const float* __restrict__ cb) {
    constexpr int V = IO::V;
    constexpr int kTeams = kNormBwdThreads / TL;
    using raw = typename IO::raw;
    extern __shared__ float sm[];
    // The per-channel rows in LDS (Ep = NV TL V entries each) are stored in
    // the lanes' order -- vector v, 16-byte quad j of the lane's vector, lane,
    // element -- so that the 16-byte reads of consecutive lanes are
    // consecutive and free of bank conflicts (for fp32 that is channel order;
    // bf16 lanes hold two quads).  The conv's taps: one 16-byte vector per
    // channel, in the order (vector v, element k, lane).
    constexpr int kQ = V / 4;
    const int Ep = NV * TL * V;
    float* srow = sm;
    float* dsum = sm + Ep;
    float* slw = sm + 2 * Ep;
    float* slb = sm + 3 * Ep;
    float* cwt = sm + 4 * Ep;  // CONV: Ep tap vectors, then Ep biases
    float* red = sm;           // [kTeams][E], after the last token
    __shared__ int list[MASKED ? kNormBwdThreads : 1];
    __shared__ int wave_cnt[kMaxListWaves];
    const int64_t bt = blockIdx.x;
    const int64_t b = bt / T, t = bt - b * T;
    const int tid = threadIdx.x, team = tid / TL, lane = tid % TL;
    // LDS position of channel q's row entry, and of the lane's element k of
    // its vector v; tap-vector index of the lane's element k of vector v
    auto lpos = [&](int q) {
        const int v = q / (TL * V), r = q - v * TL * V, ln = r / V, k = r - ln * V;
        return ((v * kQ + (k >> 2)) * TL + ln) * 4 + (k & 3);
    };
    auto lat = [&](int v, int k) { return ((v * kQ + (k >> 2)) * TL + lane) * 4 + (k & 3); };
    auto tat = [&](int v, int k) { return (v * V + k) * TL + lane; };
    for (int q = tid; q < E; q += kNormBwdThreads) {
        const int o = lpos(q);
        srow[o] = sf[bt * E + q] + sb[bt * E + q];
        dsum[o] = Df[q] + Db[q];
        slw[o] = lnw[q];
        slb[o] = lnb[q];
    }
    if (CONV)
        for (int q = tid; q < E; q += kNormBwdThreads) {
            const int v = q / (TL * V), r = q - v * TL * V, ln = r / V, k = r - ln * V;
            *reinterpret_cast<f32x4*>(cwt + ((v * V + k) * TL + ln) * kTaps) =
                *reinterpret_cast<const f32x4*>(cw + q * kTaps);
            cwt[4 * Ep + lpos(q)] = cb[q];
        }
    __syncthreads();
    const float inv_e = 1.f / (float)E;
    float ag[NV][V], ad[NV][V], aw[NV][V], ab[NV][V];
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int k = 0; k < V; ++k) ag[v][k] = ad[v][k] = aw[v][k] = ab[v][k] = 0.f;

    // one token (team-uniform call; every lane of the team takes part)
    auto token = [&](int64_t tok) {
        const typename IO::elem* xb = x + tok * E;
        const typename IO::elem* zb = z + tok * E;
        const typename IO::elem* db = dout + tok * E;
        raw xr[NV], zr[NV], dr[NV];
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int c = (v * TL + lane) * V;
            if (c < E) {
                xr[v] = load_raw<true>(xb + c);
                zr[v] = load_raw<true>(zb + c);
                dr[v] = load_raw<true>(db + c);
            }
        }
        float n[NV][V], dn[NV][V];
        float sum = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int c = (v * TL + lane) * V;
#pragma unroll
            for (int k = 0; k < V; ++k) {
                n[v][k] = c < E ? fmaf(dsum[lat(v, k)], raw_at(xr[v], k), srow[lat(v, k)]) : 0.f;
                sum += n[v][k];
            }
        }
        const float mean = team_sum<TL>(sum) * inv_e;
        float sq = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if ((v * TL + lane) * V < E) {
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float d = n[v][k] - mean;
                    sq = fmaf(d, d, sq);
                }
            }
        }
        const float r = __builtin_amdgcn_rsqf(team_sum<TL>(sq) * inv_e + eps);
        float m1 = 0.f, m2 = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int c = (v * TL + lane) * V;
            if (c < E) {
                float oz[V];
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float nv = (n[v][k] - mean) * r;
                    const float zv = raw_at(zr[v], k), dv = raw_at(dr[v], k);
                    const float sg = nb_sigmoid(zv);
                    const float go = dv * zv * sg;
                    const float lw = slw[lat(v, k)];
                    oz[k] = dv * fmaf(nv, lw, slb[lat(v, k)]) * sg * fmaf(zv, 1.f - sg, 1.f);
                    aw[v][k] = fmaf(go, nv, aw[v][k]);
                    ab[v][k] += go;
                    dn[v][k] = go * lw;
                    m1 += dn[v][k];
                    m2 = fmaf(dn[v][k], nv, m2);
                    n[v][k] = nv;
                }
                store_vec<true>(dz + tok * E + c, oz);
            }
        }
        m1 = team_sum<TL>(m1) * inv_e;
        m2 = team_sum<TL>(m2) * inv_e;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int c = (v * TL + lane) * V;
            if (c < E) {
                float og[V];
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float g = r * (dn[v][k] - m1 - n[v][k] * m2);
                    og[k] = g;
                    ag[v][k] += g;
                    ad[v][k] = fmaf(g, raw_at(xr[v], k), ad[v][k]);
                }
                store_vec<true>(gout + tok * E + c, og);
            }
        }
    };

    // CONV: the same for a token whose x_conv the caller computed, given as
    // xat(v, k) (channel (v TL + lane) V + k).  A copy of the arithmetic
    // above: one shared body raised the plain kernels' register count past
    // the three-waves-per-SIMD limit.
    auto token_core = [&](auto xat, const raw (&zr)[NV], const raw (&dr)[NV], int64_t tok) {
        float n[NV][V], dn[NV][V];
        float sum = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int c = (v * TL + lane) * V;
#pragma unroll
            for (int k = 0; k < V; ++k) {
                n[v][k] = c < E ? fmaf(dsum[lat(v, k)], xat(v, k), srow[lat(v, k)]) : 0.f;
                sum += n[v][k];
            }
        }
        const float mean = team_sum<TL>(sum) * inv_e;
        float sq = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if ((v * TL + lane) * V < E) {
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float d = n[v][k] - mean;
                    sq = fmaf(d, d, sq);
                }
            }
        }
        const float r = __builtin_amdgcn_rsqf(team_sum<TL>(sq) * inv_e + eps);
        float m1 = 0.f, m2 = 0.f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int c = (v * TL + lane) * V;
            if (c < E) {
                float oz[V];
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float nv = (n[v][k] - mean) * r;
                    const float zv = raw_at(zr[v], k), dv = raw_at(dr[v], k);
                    const float sg = nb_sigmoid(zv);
                    const float go = dv * zv * sg;
                    const float lw = slw[lat(v, k)];
                    oz[k] = dv * fmaf(nv, lw, slb[lat(v, k)]) * sg * fmaf(zv, 1.f - sg, 1.f);
                    aw[v][k] = fmaf(go, nv, aw[v][k]);
                    ab[v][k] += go;
                    dn[v][k] = go * lw;
                    m1 += dn[v][k];
                    m2 = fmaf(dn[v][k], nv, m2);
                    n[v][k] = nv;
                }
                store_vec<true>(dz + tok * E + c, oz);
            }
        }
        m1 = team_sum<TL>(m1) * inv_e;
        m2 = team_sum<TL>(m2) * inv_e;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int c = (v * TL + lane) * V;
            if (c < E) {
                float og[V];
#pragma unroll
                for (int k = 0; k < V; ++k) {
                    const float g = r * (dn[v][k] - m1 - n[v][k] * m2);
                    og[k] = g;
                    ag[v][k] += g;
                    ad[v][k] = fmaf(g, xat(v, k), ad[v][k]);
                }
                store_vec<true>(gout + tok * E + c, og);
            }
        }
    };
    auto load_zd = [&](int64_t tok, raw (&zr)[NV], raw (&dr)[NV]) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int c = (v * TL + lane) * V;
            if (c < E) {
                zr[v] = load_raw<true>(z + tok * E + c);
                dr[v] = load_raw<true>(dout + tok * E + c);
            }
        }
    };
    if (MASKED) {
        for (int64_t k0 = 0; k0 < K; k0 += kNormBwdThreads) {
            const int n = row_token_list(rows + b * K, K, t, k0, list, wave_cnt);
            for (int i = team; i < n; i += kTeams) token(b * K + k0 + list[i]);
        }
    } else if (CONV) {
        // the producer Conv1D on load: team `team` takes the run of cells
        // [team Lr, team Lr + Lr) of the line in sequence order (the grid row
        // t of a row-major sequence, the column t of a column-major one), each
        // lane sliding the conv's window of three raw vectors over its vectors
        // (a halo of three at the run's start, from the caches: x is read with
        // allocating loads)
        const int64_t base = b * h * w + (cols_axis ? t * w : t);
        const int64_t step = cols_axis ? 1 : w;
        const int Lr = (int)((P + kTeams - 1) / kTeams);
        const int pa = team * Lr, pb = pa + Lr < (int)P ? pa + Lr : (int)P;
        if (pa < pb) {
            const typename IO::elem* ximg = x + b * h * w * E;
            raw w3[NV], w2[NV], w1[NV];
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int c = (v * TL + lane) * V;
                if (c < E) {
                    if (cols_axis) load_halo<IO, true>(ximg, c, E, (int)t, pa, (int)h, (int)w, w3[v], w2[v], w1[v]);
                    else load_halo<IO, false>(ximg, c, E, pa, (int)t, (int)h, (int)w, w3[v], w2[v], w1[v]);
                }
            }
            for (int p = pa; p < pb; ++p) {
                const int64_t tok = base + p * step;
                raw xr[NV], zr[NV], dr[NV];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int c = (v * TL + lane) * V;
                    if (c < E) xr[v] = load_raw<false>(x + tok * E + c);
                }
                load_zd(tok, zr, dr);
                float xc[NV][V];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int c = (v * TL + lane) * V;
                    if (c < E) {
#pragma unroll
                        for (int q = 0; q < V; ++q) {
                            const f32x4 t4 = *reinterpret_cast<const f32x4*>(cwt + tat(v, q) * kTaps);
                            float av = fmaf(t4.w, raw_at(xr[v], q), cwt[4 * Ep + lat(v, q)]);
                            av = fmaf(t4.z, raw_at(w1[v], q), av);
                            av = fmaf(t4.y, raw_at(w2[v], q), av);
                            av = fmaf(t4.x, raw_at(w3[v], q), av);
                            xc[v][q] = conv_silu_f(av);
                        }
                        w3[v] = w2[v];
                        w2[v] = w1[v];
                        w1[v] = xr[v];
                    } else {
#pragma unroll
                        for (int q = 0; q < V; ++q) xc[v][q] = 0.f;
                    }
                }
                token_core([&](int v, int k) { return xc[v][k]; }, zr, dr, tok);
            }
        }
    } else {
        const int64_t base = b * h * w + (cols_axis ? t * w : t);
        const int64_t step = cols_axis ? 1 : w;
        for (int64_t p = team; p < P; p += kTeams) token(base + p * step);
    }
    __syncthreads();
    team_reduce_out<TL, NV, V>(ag, red, gs + bt * E, E, team, lane);
    team_reduce_out<TL, NV, V>(ad, red, dDp + bt * E, E, team, lane);
    team_reduce_out<TL, NV, V>(aw, red, dlnwp + bt * E, E, team, lane);
    team_reduce_out<TL, NV, V>(ab, red, dlnbp + bt * E, E, team, lane);
}

// Pass 2: dx = g (D_fwd + D_bwd) + du[b, t] / P in place over g, one 16-byte
// vector per lane and kP2 vectors per thread (all loads first).  MODE 0: t is
// the cell's grid row (COLS), 1: its column (ROWS), 2: the kept token's row
// (masked; -1 writes NaN into dx and dz).
constexpr int kP2 = 4;
template <class IO, int MODE>
__global__ void __launch_bounds__(256)
bwd_norm_pass2_kernel(typename IO::elem* __restrict__ dx, typename IO::elem* __restrict__ dz,
                      const float* __restrict__ du, const float* __restrict__ Df, const float* __restrict__ Db,
                      const int32_t* __restrict__ rows, int64_t T, int64_t w, int64_t ncell, int VE,
                      int64_t blocks_per_img, float inv_p) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    const int64_t blk = blockIdx.x;
    const int64_t b = blk / blocks_per_img;
    const uint32_t nvec = (uint32_t)(ncell * VE);  // h w E < 2^31
    const uint32_t i0 = (uint32_t)(blk - b * blocks_per_img) * (256u * kP2) + threadIdx.x;
    const int64_t E = (int64_t)VE * V;
    typename IO::elem* xb = dx + b * ncell * E;
    raw gr[kP2];
#pragma unroll
    for (int k = 0; k < kP2; ++k) {
        const uint32_t i = i0 + 256u * k;
        if (i < nvec) gr[k] = load_raw<true>(xb + (int64_t)i * V);
    }
#pragma unroll
    for (int k = 0; k < kP2; ++k) {
        const uint32_t i = i0 + 256u * k;
        if (i >= nvec) continue;
        const uint32_t cell = i / (uint32_t)VE, c = (i - cell * (uint32_t)VE) * V;
        int64_t t;
        if (MODE == 0) t = cell / (uint32_t)w;
        else if (MODE == 1) t = cell % (uint32_t)w;
        else t = rows[b * ncell + cell];
        float o[V];
        if (t < 0) {
#pragma unroll
            for (int q = 0; q < V; ++q) o[q] = __builtin_nanf("");
            store_vec<true>(dz + (b * ncell + cell) * E + c, o);
        } else {
            const float* ur = du + (b * T + t) * E + c;
#pragma unroll
            for (int q = 0; q < V; ++q) o[q] = fmaf(raw_at(gr[k], q), Df[c + q] + Db[c + q], ur[q] * inv_p);
        }
        store_vec<true>(xb + (int64_t)i * V, o);
    }
}

// Team width and vectors per lane: the narrowest team whose lanes hold at
// most 16 channels, else 64 lanes (E <= 2048 either way).
struct NormBwdShape {
    int TL, NV;
};
NormBwdShape norm_bwd_shape(const Geom& g) {
    const int V = g.io == FASTVIM_BF16 ? IoBf16::V : IoF32::V;
    const int64_t vecs = g.E / V, nvmax = 16 / V;
    for (int tl : {16, 32, 64})
        if (vecs <= tl * nvmax) return {tl, (int)((vecs + tl - 1) / tl)};
    return {64, (int)((vecs + 63) / 64)};
}

template <class IO, int TL, int NV>
hipError_t pass1_launch(const Geom& g, const void* x, const void* z, const void* dout, const fastvim_params& p,
                        const BwdWorkspace& ws, void* dx, void* dz, hipStream_t st) {
    using elem = typename IO::elem;
    constexpr int kTeams = kNormBwdThreads / TL;
    const bool conv = (p.flags & FASTVIM_FLAG_CONV) != 0;  // dense layers: x is the conv's input
    const int64_t Ep = (int64_t)NV * TL * IO::V;  // padded row length (see the kernel)
    const int64_t rows = (conv ? 9 : 4) * Ep, red = (int64_t)kTeams * g.E;
    const size_t lds = (size_t)(rows > red ? rows : red) * sizeof(float);
    const dim3 grid((unsigned)(g.B * g.T)), block(kNormBwdThreads);
    const elem *xe = static_cast<const elem*>(x), *ze = static_cast<const elem*>(z),
               *de = static_cast<const elem*>(dout);
    elem *ge = static_cast<elem*>(dx), *dze = static_cast<elem*>(dz);
    const int cols = g.axis == FASTVIM_POOL_COLS;
#define FASTVIM_P1(masked, cv)                                                                                     \
    hipLaunchKernelGGL((bwd_norm_pass1_kernel<IO, TL, NV, masked, cv>), grid, block, lds, st, xe, ze, de,         \
                       ws.fwd.s_f, ws.fwd.s_b, p.fwd.D, p.bwd.D, p.ln_weight, p.ln_bias, p.ln_eps, ws.fwd.rows, ge, \
                       dze, ws.gs, ws.du, ws.du_f, ws.du_b, g.T, g.h, g.w, g.K, g.P, cols, (int)g.E, p.conv_w,      \
                       p.conv_b)
    if (g.masked) FASTVIM_P1(true, false);
    else if (conv) FASTVIM_P1(false, true);
    else FASTVIM_P1(false, false);
#undef FASTVIM_P1
    return hipGetLastError();
}

template <class IO>
hipError_t pass1_dispatch(const Geom& g, const void* x, const void* z, const void* dout, const fastvim_params& p,
                          const BwdWorkspace& ws, void* dx, void* dz, hipStream_t st) {
    const NormBwdShape s = norm_bwd_shape(g);
#define FASTVIM_NB_CASE(tl, nv) \
    if (s.TL == tl && s.NV <= nv) return pass1_launch<IO, tl, nv>(g, x, z, dout, p, ws, dx, dz, st)
    if constexpr (IO::V == 4) {  // fp32: NV <= 4 below 64 lanes
        FASTVIM_NB_CASE(16, 1);
        FASTVIM_NB_CASE(16, 2);
        FASTVIM_NB_CASE(16, 3);
        FASTVIM_NB_CASE(16, 4);
        FASTVIM_NB_CASE(32, 3);
        FASTVIM_NB_CASE(32, 4);
        FASTVIM_NB_CASE(64, 3);
        FASTVIM_NB_CASE(64, 4);
        FASTVIM_NB_CASE(64, 8);
    } else {  // bf16: NV <= 2 below 64 lanes
        FASTVIM_NB_CASE(16, 1);
        FASTVIM_NB_CASE(16, 2);
        FASTVIM_NB_CASE(32, 2);
        FASTVIM_NB_CASE(64, 2);
        FASTVIM_NB_CASE(64, 4);
    }
#undef FASTVIM_NB_CASE
    return hipErrorInvalidValue;  // E > 2048: excluded by bwd_norm_supported
}

template <class IO>
hipError_t pass2_dispatch(const Geom& g, const fastvim_params& p, const BwdWorkspace& ws, void* dx, void* dz,
                          hipStream_t st) {
    using elem = typename IO::elem;
    const int64_t VE = g.E / IO::V, ncell = g.masked ? g.K : g.h * g.w;
    const int64_t bpi = (ncell * VE + 256 * kP2 - 1) / (256 * kP2);
    const dim3 grid((unsigned)(g.B * bpi)), block(256);
    elem *xe = static_cast<elem*>(dx), *ze = static_cast<elem*>(dz);
    const float ip = pool_norm(g);
    if (g.masked)
        hipLaunchKernelGGL((bwd_norm_pass2_kernel<IO, 2>), grid, block, 0, st, xe, ze, ws.du, p.fwd.D, p.bwd.D,
                           ws.fwd.rows, g.T, g.w, ncell, (int)VE, bpi, ip);
    else if (g.axis == FASTVIM_POOL_COLS)
        hipLaunchKernelGGL((bwd_norm_pass2_kernel<IO, 0>), grid, block, 0, st, xe, ze, ws.du, p.fwd.D, p.bwd.D,
                           ws.fwd.rows, g.T, g.w, ncell, (int)VE, bpi, ip);
    else
        hipLaunchKernelGGL((bwd_norm_pass2_kernel<IO, 1>), grid, block, 0, st, xe, ze, ws.du, p.fwd.D, p.bwd.D,
                           ws.fwd.rows, g.T, g.w, ncell, (int)VE, bpi, ip);
    return hipGetLastError();
}

}  // namespace

bool bwd_norm_supported(const Geom& g) { return g.E <= 2048; }

hipError_t launch_bwd_norm_pass1(const Geom& g, const void* x, const void* z, const void* dout,
                                 const fastvim_params& p, const BwdWorkspace& ws, void* dx, void* dz,
                                 hipStream_t st) {
    return g.io == FASTVIM_BF16 ? pass1_dispatch<IoBf16>(g, x, z, dout, p, ws, dx, dz, st)
                                : pass1_dispatch<IoF32>(g, x, z, dout, p, ws, dx, dz, st);
}

hipError_t launch_bwd_norm_pass2(const Geom& g, const fastvim_params& p, const BwdWorkspace& ws, void* dx,
                                 void* dz, hipStream_t st) {
    return g.io == FASTVIM_BF16 ? pass2_dispatch<IoBf16>(g, p, ws, dx, dz, st)
                                : pass2_dispatch<IoF32>(g, p, ws, dx, dz, st);
}

}  // namespace fastvim
