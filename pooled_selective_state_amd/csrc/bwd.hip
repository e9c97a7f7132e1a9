// Backward pass of the pooled layer, apart from the scan adjoint
// (scan_bwd.hip): the gradient of L = sum(dout * out) with respect to x, z
// and both directions' parameters, taken through the forward steps in reverse
// (FastVim summary page, gptget.net, arXiv 2502.00594, section 方法详解
// bullets 2-5 for the forward steps; the page's 实验结果 section for the
// training runs the gradient serves).  With y = s_fwd + s_bwd + (D_fwd + D_bwd) x
// and out = y silu(z):
//   g   = dL/dy = dout silu(z)
//   dz  = dout y silu'(z),   silu'(q) = sigmoid(q) (1 + q (1 - sigmoid(q)))
//   gs[b, t, e] = sum of g over the cells repeated from scan position t (the
//               repeat's adjoint), the same for both scan directions
//   dD_fwd = dD_bwd = sum over all cells of g x
//   dx  = g (D_fwd + D_bwd) + du[b, t(cell), e] / P   (the pool's adjoint)
// and du, the gradient of the pooled tokens, collects the scan adjoint of
// both directions and the x_proj adjoint du += x_proj_w^T dv.
//
// Kernels here, in launch order:
//   pass 1   (z and dout read once, and x unless the caller saved the pooled
//            tokens u from the forward call) gs, and u (the scan input,
//            which the backward otherwise recomputes);
//   dv       dL/dv from the scan adjoint's channel-group partials;
//   du       du = du_fwd + du_bwd + x_proj_w^T dv for both directions;
//   dwx      per-chunk partials of d x_proj_w = sum_m dv[m] u[m]^T;
//   pass 2   (x, z, dout read again) dx and dz written once, and per-workgroup
//            partials of dD;
//   colsum   fixed-order column sums: parameter gradients from per-image,
//            per-chunk or per-workgroup partials.
// Passes 1 and 2 move the full-resolution tensors and bound the pass; both
// stream 16-byte vectors with every load of a batch issued before any
// arithmetic, like the forward pool and epilogue kernels.
#include "bwd_internal.h"
#include "mask_list.h"

namespace fastvim {
namespace {

__device__ __forceinline__ float sigmoid_f(float q) { return __builtin_amdgcn_rcpf(1.f + __expf(-q)); }

// ------------------------------------------------------------------ pass 1
// One workgroup per pooled token (b, t): G groups of VE vector lanes, lane c
// owning the 16-byte column [c V, c V + V) of E, group g taking the pooled
// positions p = g, g + G, ...; the G partial sums are added through LDS in a
// fixed order.  POOL: also pool x into u (else u is the caller's saved copy
// and x is not read here).  NT: non-temporal loads (the pass reads more than
// the Infinity Cache holds, so nothing it reads is still there for pass 2).
template <class IO, bool POOL, bool NT>
__global__ void __launch_bounds__(1024)
bwd_pool_dense_kernel(const typename IO::elem* __restrict__ x, const typename IO::elem* __restrict__ z,
                      const typename IO::elem* __restrict__ dout, float* __restrict__ u, float* __restrict__ gs,
                      int64_t T, int64_t P, int VE, int G, int64_t E, int64_t img_stride, int64_t t_stride,
                      int64_t p_stride, float inv_p) {
    constexpr int V = IO::V;
    constexpr int kD = POOL ? 4 : 6;  // pooled positions in flight per lane (12 loads either way)
    using raw = typename IO::raw;
    extern __shared__ float red[];  // [POOL ? 2 : 1][G][VE * V]
    const int64_t bt = blockIdx.x;
    const int64_t b = bt / T, t = bt - b * T;
    const int tid = threadIdx.x;
    const int c = tid % VE, g = tid / VE;
    const int width = VE * V;
    if (g < G) {
        float au[V], ag[V];
#pragma unroll
        for (int k = 0; k < V; ++k) au[k] = ag[k] = 0.f;
        const int64_t off = b * img_stride + t * t_stride + (int64_t)c * V;
        for (int64_t p0 = g; p0 < P; p0 += kD * G) {
            raw xr[kD], zr[kD], dr[kD];
#pragma unroll
            for (int i = 0; i < kD; ++i) {
                const int64_t p = p0 + (int64_t)i * G;
                if (p < P) {
                    const int64_t o = off + p * p_stride;
                    if (POOL) xr[i] = load_raw<NT>(x + o);
                    zr[i] = load_raw<NT>(z + o);
                    dr[i] = load_raw<NT>(dout + o);
                }
            }
#pragma unroll
            for (int i = 0; i < kD; ++i) {
                if (p0 + (int64_t)i * G < P) {
#pragma unroll
                    for (int k = 0; k < V; ++k) {
                        const float zv = raw_at(zr[i], k);
                        ag[k] += raw_at(dr[i], k) * zv * sigmoid_f(zv);
                        if (POOL) au[k] += raw_at(xr[i], k);
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int64_t o = ((int64_t)g * VE + c) * V + k;
            red[o] = ag[k];
            if (POOL) red[(int64_t)G * width + o] = au[k];
        }
    }
    __syncthreads();
    for (int q = tid; q < width; q += blockDim.x) {
        float sg = red[q];
        for (int gg = 1; gg < G; ++gg) sg += red[gg * width + q];
        gs[bt * E + q] = sg;
        if (POOL) {
            float su = red[G * width + q];
            for (int gg = 1; gg < G; ++gg) su += red[(G + gg) * width + q];
            u[bt * E + q] = su * inv_p;
        }
    }
}

// Masked pass 1: workgroup (b, t) takes the kept tokens whose row is t; the
// pooled sum is divided by the fixed row length P.  Tokens with an invalid
// mask entry (row -1) belong to no row.  As in the forward pooling, the row's
// tokens of each slice of blockDim.x kept tokens are listed first
// (mask_list.h) and then loaded kB at a time per lane.
template <class IO, bool POOL>
__global__ void __launch_bounds__(1024)
bwd_pool_masked_kernel(const typename IO::elem* __restrict__ x, const typename IO::elem* __restrict__ z,
                       const typename IO::elem* __restrict__ dout, const int32_t* __restrict__ rows,
                       float* __restrict__ u, float* __restrict__ gs, int64_t T, int64_t K, int VE, int G,
                       int64_t E, float inv_p) {
    constexpr int V = IO::V;
    constexpr int kB = 16 / V;  // list entries in flight per lane (64 bytes of each stream)
    extern __shared__ float red[];  // [POOL ? 2 : 1][G][VE * V]
    __shared__ int list[1024];
    __shared__ int wave_cnt[kMaxListWaves];
    const int64_t bt = blockIdx.x;
    const int64_t b = bt / T, t = bt - b * T;
    const int tid = threadIdx.x;
    const int c = tid % VE, g = tid / VE;
    const int width = VE * V;
    float au[V], ag[V];
#pragma unroll
    for (int k = 0; k < V; ++k) au[k] = ag[k] = 0.f;
    for (int64_t k0 = 0; k0 < K; k0 += blockDim.x) {
        const int n = row_token_list(rows + b * K, K, t, k0, list, wave_cnt);
        if (g >= G) continue;
        const int64_t base = (b * K + k0) * E + (int64_t)c * V;
        for (int i0 = g; i0 < n; i0 += kB * G) {
            float xv[kB][V], zv[kB][V], dv[kB][V];
#pragma unroll
            for (int j = 0; j < kB; ++j)
                if (i0 + j * G < n) {
                    const int64_t o = base + (int64_t)list[i0 + j * G] * E;
                    if (POOL) load_vec<false>(x + o, xv[j]);
                    load_vec<false>(z + o, zv[j]);
                    load_vec<false>(dout + o, dv[j]);
                }
#pragma unroll
            for (int j = 0; j < kB; ++j)
                if (i0 + j * G < n) {
#pragma unroll
                    for (int q = 0; q < V; ++q) {
                        ag[q] += dv[j][q] * zv[j][q] * sigmoid_f(zv[j][q]);
                        if (POOL) au[q] += xv[j][q];
                    }
                }
        }
    }
    if (g < G) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int64_t o = ((int64_t)g * VE + c) * V + k;
            red[o] = ag[k];
            if (POOL) red[(int64_t)G * width + o] = au[k];
        }
    }
    __syncthreads();
    for (int q = tid; q < width; q += blockDim.x) {
        float sg = red[q];
        for (int gg = 1; gg < G; ++gg) sg += red[gg * width + q];
        gs[bt * E + q] = sg;
        if (POOL) {
            float su = red[G * width + q];
            for (int gg = 1; gg < G; ++gg) su += red[(G + gg) * width + q];
            u[bt * E + q] = su * inv_p;
        }
    }
}

// G groups of VE lanes, G <= n, about 512 threads.
void pick_groups_bwd(int64_t VE, int64_t n, int* G, int* threads) {
    int64_t g = 512 / VE;
    if (g > n) g = n;
    if (g < 1) g = 1;
    *G = (int)g;
    *threads = (int)((VE * g + 63) / 64 * 64);
}

template <class IO, bool POOL>
hipError_t bwd_pool_t(const Geom& g, const void* x, const void* z, const void* dout, const BwdWorkspace& ws,
                      hipStream_t st) {
    constexpr int64_t kMallBytes = 256ll << 20;  // Infinity Cache
    using elem = typename IO::elem;
    const int64_t VE = g.E / IO::V;
    int G, threads;
    pick_groups_bwd(VE, g.masked ? g.K : g.P, &G, &threads);
    const size_t lds = (POOL ? 2 : 1) * (size_t)G * VE * IO::V * sizeof(float);
    const elem *xe = static_cast<const elem*>(x), *ze = static_cast<const elem*>(z),
               *de = static_cast<const elem*>(dout);
    if (g.masked) {
        hipLaunchKernelGGL((bwd_pool_masked_kernel<IO, POOL>), dim3((unsigned)(g.B * g.T)), dim3(threads), lds, st,
                           xe, ze, de, ws.fwd.rows, ws.fwd.u, ws.gs, g.T, g.K, (int)VE, G, g.E,
                           pool_norm(g));
    } else {
        const int64_t t_stride = g.axis == FASTVIM_POOL_COLS ? g.w * g.E : g.E;
        const int64_t p_stride = g.axis == FASTVIM_POOL_COLS ? g.E : g.w * g.E;
        const int64_t bytes = (POOL ? 3 : 2) * g.B * g.h * g.w * g.E * (int64_t)sizeof(elem);
        if (bytes > kMallBytes)
            hipLaunchKernelGGL((bwd_pool_dense_kernel<IO, POOL, true>), dim3((unsigned)(g.B * g.T)), dim3(threads),
                               lds, st, xe, ze, de, ws.fwd.u, ws.gs, g.T, g.P, (int)VE, G, g.E, g.h * g.w * g.E,
                               t_stride, p_stride, pool_norm(g));
        else
            hipLaunchKernelGGL((bwd_pool_dense_kernel<IO, POOL, false>), dim3((unsigned)(g.B * g.T)), dim3(threads),
                               lds, st, xe, ze, de, ws.fwd.u, ws.gs, g.T, g.P, (int)VE, G, g.E, g.h * g.w * g.E,
                               t_stride, p_stride, pool_norm(g));
    }
    return hipGetLastError();
}

template <class IO>
hipError_t bwd_pool_io(const Geom& g, const void* x, const void* z, const void* dout, const BwdWorkspace& ws,
                       hipStream_t st) {
    return ws.u_saved ? bwd_pool_t<IO, false>(g, x, z, dout, ws, st) : bwd_pool_t<IO, true>(g, x, z, dout, ws, st);
}

// ---------------------------------------------------------------------- dv
// dv[b, t, d, o] = sum over channel groups of the scan adjoint's partials,
// taken from the LDS row layout: o < R is the low-rank input r = o at
// position (r mod 4) RMAX/4 + r div 4, o >= R is B / C at RMAX + o - R.
__global__ void __launch_bounds__(256)
bwd_dv_kernel(const float* __restrict__ dvp, float* __restrict__ dv, int64_t B, int64_t T, int64_t G, int S, int R,
              int NX, int RMAX) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = B * T * 2 * NX;
    if (idx >= total) return;
    const int o = (int)(idx % NX);
    const int64_t rest = idx / NX;
    const int d = (int)(rest % 2);
    const int64_t bt = rest / 2, b = bt / T, t = bt - b * T;
    const int pos = o < R ? (o % 4) * (RMAX / 4) + o / 4 : RMAX + (o - R);
    const float* src = dvp + ((d * B + b) * G) * T * S + t * S + pos;
    float s = 0.f;
    for (int64_t gg = 0; gg < G; ++gg) s += src[gg * T * S];
    dv[idx] = s;
}

// ---------------------------------------------------------------------- du
// du[m, e] = du_f[m, e] + du_b[m, e] + sum_o (W_f[o, e] dv[m, 0, o] + W_b[o, e] dv[m, 1, o]).
// A workgroup takes 64 channels (lane = channel) and 4 kDuTok tokens (wave w
// the tokens w kDuTok ...); the tokens' dv rows of both directions are staged
// in LDS and read as broadcasts, each weight entry is loaded once per wave.
constexpr int kDuTok = 16;
__global__ void __launch_bounds__(256)
bwd_du_kernel(const float* __restrict__ du_f, const float* __restrict__ du_b, const float* __restrict__ dv,
              const float* __restrict__ Wf, const float* __restrict__ Wb, float* __restrict__ du, int64_t M, int64_t E,
              int NX) {
    __shared__ float dvs[4 * kDuTok * 2 * 96];  // [token][d][o]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t e = (int64_t)blockIdx.y * 64 + lane;
    const int64_t ec = e < E ? e : E - 1;
    const int64_t mblk = (int64_t)blockIdx.x * 4 * kDuTok;
    const int nm = (int)(mblk + 4 * kDuTok < M ? 4 * kDuTok : M - mblk);
    const int row = 2 * NX;
    for (int idx = threadIdx.x; idx < nm * row; idx += 256) dvs[idx] = dv[mblk * row + idx];
    __syncthreads();
    const int t0 = wave * kDuTok;
    if (t0 >= nm) return;
    float acc[kDuTok];
#pragma unroll
    for (int k = 0; k < kDuTok; ++k) {
        const int64_t m = mblk + (t0 + k < nm ? t0 + k : nm - 1);
        acc[k] = du_f[m * E + ec] + du_b[m * E + ec];
    }
    for (int d = 0; d < 2; ++d) {
        const float* W = d ? Wb : Wf;
        for (int o = 0; o < NX; ++o) {
            const float wv = W[(int64_t)o * E + ec];
#pragma unroll
            for (int k = 0; k < kDuTok; ++k) {
                const int mm = t0 + k < nm ? t0 + k : nm - 1;
                acc[k] = fmaf(wv, dvs[mm * row + d * NX + o], acc[k]);
            }
        }
    }
    if (e < E) {
#pragma unroll
        for (int k = 0; k < kDuTok; ++k)
            if (t0 + k < nm) du[(mblk + t0 + k) * E + e] = acc[k];
    }
}

// --------------------------------------------------------------------- dwx
// Partial of d x_proj_w over one chunk of kBwdTokChunk pooled tokens, both
// directions at once (rows o < NO = 2 NX: [0, NX) forward, [NX, NO) backward):
//   dWxp[chunk, o, e] = sum_{m in chunk} dv[m, o] u[m, e]
// an (NO x chunk) . (chunk x E) contraction on the matrix cores
// (v_mfma_f32_16x16x4f32, fp32 products and sums).  A workgroup takes one
// chunk and 64 channels.  The chunk's dv rows are staged in LDS transposed,
// dvt[o][k], zero past the chunk and past NO, so a lane reads its A operand
// (row o = 16 rt + l % 16, tokens k0 + 4 (l / 16) .. + 3) as one 16-byte
// vector.  Wave w owns channels e0 + 16 w .. + 15 and every row tile, and
// loads its B operand (token k0 + 4 (l / 16) + i, channel e0 + 16 w + l % 16)
// from u; MFMA i of a 16-token step covers token k0 + 4 (l / 16) + i for both
// operands.  Accumulator register r of lane l holds row 16 rt + 4 (l / 16) + r,
// channel e0 + 16 w + l % 16.
// RT row tiles cover NO (instances per dt-rank bound: NO <= 2 (RMAX + 32)).
constexpr int kDwxLd = kBwdTokChunk + 4;  // LDS row stride of dvt (spreads the rows over the banks)
template <int RT>
__global__ void __launch_bounds__(256)
bwd_dwx_kernel(const float* __restrict__ dv, const float* __restrict__ u, float* __restrict__ dWxp, int64_t M,
               int64_t E, int NO) {
    __shared__ __attribute__((aligned(16))) float dvt[16 * RT * kDwxLd];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int ri = lane & 15, kk = lane >> 4;
    const int64_t chunk = blockIdx.x;
    const int64_t m0 = chunk * kBwdTokChunk;
    const int nm = (int)(m0 + kBwdTokChunk < M ? kBwdTokChunk : M - m0);
    constexpr int rows = 16 * RT;
    for (int idx = threadIdx.x; idx < rows * kBwdTokChunk; idx += 256) {
        const int k = idx / rows, o = idx - k * rows;  // consecutive threads read consecutive entries of a dv row
        dvt[o * kDwxLd + k] = (k < nm && o < NO) ? dv[(m0 + k) * NO + o] : 0.f;
    }
    __syncthreads();
    const int64_t e = (int64_t)blockIdx.y * 64 + wv * 16 + ri;
    const int64_t ec = e < E ? e : E - 1;
    f32x4 acc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < kBwdTokChunk; k0 += 16) {
        float bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = k0 + 4 * kk + i;
            bv[i] = k < nm ? u[(m0 + k) * E + ec] : 0.f;
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const f32x4 a4 = *reinterpret_cast<const f32x4*>(dvt + (rt * 16 + ri) * kDwxLd + k0 + 4 * kk);
            acc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.x, bv[0], acc[rt], 0, 0, 0);
            acc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.y, bv[1], acc[rt], 0, 0, 0);
            acc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.z, bv[2], acc[rt], 0, 0, 0);
            acc[rt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a4.w, bv[3], acc[rt], 0, 0, 0);
        }
    }
    if (e < E) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = rt * 16 + 4 * kk + r;
                if (o < NO) dWxp[(chunk * NO + o) * E + e] = acc[rt][r];
            }
        }
    }
}

// ------------------------------------------------------------------ colsum
// out[c, j] = sum_{i in rows [c rpb, (c + 1) rpb)} in[i ld + j].  A workgroup
// takes 32 columns and one row chunk: 8 row groups of 32 lanes, group g
// summing rows g, g + 8, ...; the 8 group sums are added in a fixed order.
constexpr int kColTile = 32;
constexpr int kColGroups = 8;
// Columns [tile * kColTile, + kColTile) of rows [r0, r1), into out[j] (and out2).
__device__ __forceinline__ void colsum_tile(const float* __restrict__ in, int64_t r0, int64_t r1, int64_t cols,
                                            int64_t ld, int64_t tile, float* __restrict__ out,
                                            float* __restrict__ out2) {
    __shared__ float part[kColGroups][kColTile];
    const int cl = threadIdx.x % kColTile, g = threadIdx.x / kColTile;
    const int64_t j = tile * kColTile + cl;
    float s = 0.f;
    if (j < cols)
        for (int64_t i = r0 + g; i < r1; i += kColGroups) s += in[i * ld + j];
    part[g][cl] = s;
    __syncthreads();
    if (g == 0 && j < cols) {
#pragma unroll
        for (int k = 1; k < kColGroups; ++k) s += part[k][cl];
        out[j] = s;
        if (out2) out2[j] = s;
    }
}

__global__ void __launch_bounds__(256)
colsum_kernel(const float* __restrict__ in, int64_t rows, int64_t cols, int64_t ld, int64_t rpb,
              float* __restrict__ out, float* __restrict__ out2) {
    const int64_t c = blockIdx.y;
    const int64_t r0 = c * rpb, r1 = r0 + rpb < rows ? r0 + rpb : rows;
    colsum_tile(in, r0, r1, cols, ld, blockIdx.x, out + c * cols, out2 ? out2 + c * cols : nullptr);
}

// Several single-stage column sums in one launch: segment k takes workgroups
// [blk0[k], blk0[k + 1]), one column tile each, with the arithmetic of
// colsum_kernel.
__global__ void __launch_bounds__(256) colsum_batch_kernel(ColsumBatch bt) {
    int k = 0;
    while (k + 1 < bt.n && (int64_t)blockIdx.x >= bt.seg[k + 1].blk0) ++k;
    const ColsumSeg& sg = bt.seg[k];
    colsum_tile(sg.in, 0, sg.rows, sg.cols, sg.ld, (int64_t)blockIdx.x - sg.blk0, sg.out, sg.out2);
}

__global__ void __launch_bounds__(256) fill_zero_kernel(float* __restrict__ p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// ------------------------------------------------------------------ pass 2
enum { kModeCols = 0, kModeRows = 1, kModeMasked = 4 };
constexpr int kU = 4;  // tokens per thread

template <int V>
__device__ __forceinline__ void row_vec(const float* a, const float* b, int64_t off, float (&r)[V]) {
#pragma unroll
    for (int v = 0; v < V; v += 4) {
        const f32x4 p1 = load_raw<false>(a + off + v), p2 = load_raw<false>(b + off + v);
        r[v] = p1.x + p2.x;
        r[v + 1] = p1.y + p2.y;
        r[v + 2] = p1.z + p2.z;
        r[v + 3] = p1.w + p2.w;
    }
}
template <int V>
__device__ __forceinline__ void row_vec1(const float* a, int64_t off, float (&r)[V]) {
#pragma unroll
    for (int v = 0; v < V; v += 4) {
        const f32x4 p1 = load_raw<false>(a + off + v);
        r[v] = p1.x;
        r[v + 1] = p1.y;
        r[v + 2] = p1.z;
        r[v + 3] = p1.w;
    }
}

// A workgroup takes a run of G * kU consecutive tokens of one segment: a grid
// row (dense; its tokens are contiguous in memory) or one image's kept tokens
// (masked).  Lane (c, g) handles the tokens p0 + g + G k, k < kU, all loads
// issued first, and sums dL/dy * x over them; the G group sums are added
// through LDS in a fixed order into the workgroup's row of dDp.  x and dz
// may be one buffer (a layer with the producer Conv1D passes its conv output
// in dz): each token's x is read before its dz is written, so those two
// pointers carry no restrict.
template <class IO, int MODE>
__global__ void __launch_bounds__(1024)
bwd_epilogue_kernel(const typename IO::elem* x, const typename IO::elem* __restrict__ z,
                    const typename IO::elem* __restrict__ dout, const float* __restrict__ sf,
                    const float* __restrict__ sb, const float* __restrict__ du, const float* __restrict__ Df,
                    const float* __restrict__ Db, typename IO::elem* __restrict__ dx,
                    typename IO::elem* dz, const int32_t* __restrict__ rows, float* __restrict__ dDp,
                    int64_t T, int64_t h, int64_t w, int64_t K, int64_t E, int VE, int G, int64_t seg_len,
                    int64_t blocks_per_seg, int64_t segs_per_img, float inv_p) {
    constexpr int V = IO::V;
    using raw = typename IO::raw;
    extern __shared__ float red[];  // [G][VE * V]
    const int tid = threadIdx.x, c = tid % VE, g = tid / VE;
    const int width = VE * V;
    const int64_t blk = blockIdx.x;
    const int64_t seg = blk / blocks_per_seg;
    const int64_t p0 = (blk - seg * blocks_per_seg) * (int64_t)G * kU;
    const int64_t b = seg / segs_per_img, sgi = seg - b * segs_per_img;
    const int64_t col = (int64_t)c * V;
    if (g < G) {
        int64_t tok[kU];
        bool ok[kU];
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            const int64_t p = p0 + g + (int64_t)G * k;
            ok[k] = p < seg_len;
            tok[k] = MODE == kModeMasked ? b * K + p : (b * h + sgi) * w + p;
        }
        raw xr[kU], zr[kU], dr[kU];
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            if (ok[k]) {
                xr[k] = load_raw<true>(x + tok[k] * E + col);
                zr[k] = load_raw<true>(z + tok[k] * E + col);
                dr[k] = load_raw<true>(dout + tok[k] * E + col);
            }
        }
        float dsum[V], ad[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            dsum[v] = Df[col + v] + Db[col + v];
            ad[v] = 0.f;
        }
        float srow[V], urow[V];
        if (MODE == kModeCols) {
            row_vec<V>(sf, sb, (b * T + sgi) * E + col, srow);
            row_vec1<V>(du, (b * T + sgi) * E + col, urow);
        }
#pragma unroll
        for (int k = 0; k < kU; ++k) {
            if (!ok[k]) continue;
            float sv[V], uv[V];
            bool valid = true;
            if (MODE == kModeCols) {
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    sv[v] = srow[v];
                    uv[v] = urow[v];
                }
            } else {
                const int64_t t = MODE == kModeRows ? p0 + g + (int64_t)G * k : rows[tok[k]];
                valid = t >= 0;
                if (valid) {
                    row_vec<V>(sf, sb, (b * T + t) * E + col, sv);
                    row_vec1<V>(du, (b * T + t) * E + col, uv);
                }
            }
            float ox[V], oz[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const float xv = raw_at(xr[k], v), zv = raw_at(zr[k], v), dv = raw_at(dr[k], v);
                const float sg = sigmoid_f(zv);
                const float gv = dv * zv * sg;
                const float y = fmaf(dsum[v], xv, sv[v]);
                if (valid) ad[v] = fmaf(gv, xv, ad[v]);
                ox[v] = valid ? fmaf(gv, dsum[v], uv[v] * inv_p) : __builtin_nanf("");
                oz[v] = valid ? dv * y * sg * fmaf(zv, 1.f - sg, 1.f) : __builtin_nanf("");
            }
            store_vec<true>(dx + tok[k] * E + col, ox);
            store_vec<true>(dz + tok[k] * E + col, oz);
        }
#pragma unroll
        for (int v = 0; v < V; ++v) red[g * width + col + v] = ad[v];
    }
    __syncthreads();
    for (int q = tid; q < width; q += blockDim.x) {
        float sd = red[q];
        for (int gg = 1; gg < G; ++gg) sd += red[gg * width + q];
        dDp[blk * E + q] = sd;
    }
}

// Launch shape of pass 2: G groups of VE lanes per workgroup, kU tokens per
// lane, runs of G * kU tokens within a segment.
struct BwdEpiShape {
    int64_t VE, G, seg_len, segs_per_img, blocks_per_seg, blocks;
    int threads;
};

BwdEpiShape bwd_epi_shape(const Geom& g) {
    BwdEpiShape s;
    s.VE = g.E / (g.io == FASTVIM_BF16 ? IoBf16::V : IoF32::V);
    s.seg_len = g.masked ? g.K : g.w;
    s.segs_per_img = g.masked ? 1 : g.h;
    s.G = 512 / s.VE;
    if (s.G * kU > s.seg_len) s.G = (s.seg_len + kU - 1) / kU;
    if (s.G < 1) s.G = 1;
    s.blocks_per_seg = (s.seg_len + s.G * kU - 1) / (s.G * kU);
    s.blocks = g.B * s.segs_per_img * s.blocks_per_seg;
    s.threads = (int)((s.VE * s.G + 63) / 64 * 64);
    return s;
}

template <class IO, int MODE>
hipError_t bwd_epi_launch(const Geom& g, const void* x, const void* z, const void* dout, const fastvim_params& p,
                          const BwdWorkspace& ws, void* dx, void* dz, hipStream_t st) {
    const BwdEpiShape sh = bwd_epi_shape(g);
    const size_t lds = (size_t)(sh.G * g.E) * sizeof(float);
    using elem = typename IO::elem;
    hipLaunchKernelGGL((bwd_epilogue_kernel<IO, MODE>), dim3((unsigned)sh.blocks), dim3(sh.threads), lds, st,
                       static_cast<const elem*>(x), static_cast<const elem*>(z), static_cast<const elem*>(dout),
                       ws.fwd.s_f, ws.fwd.s_b, ws.du, p.fwd.D, p.bwd.D, static_cast<elem*>(dx),
                       static_cast<elem*>(dz), ws.fwd.rows, ws.dDp, g.T, g.h, g.w, g.K, g.E, (int)sh.VE, (int)sh.G,
                       sh.seg_len, sh.blocks_per_seg, sh.segs_per_img, pool_norm(g));
    return hipGetLastError();
}

template <class IO>
hipError_t bwd_epi_dispatch(const Geom& g, const void* x, const void* z, const void* dout, const fastvim_params& p,
                            const BwdWorkspace& ws, void* dx, void* dz, hipStream_t st) {
    if (g.masked) return bwd_epi_launch<IO, kModeMasked>(g, x, z, dout, p, ws, dx, dz, st);
    if (g.axis == FASTVIM_POOL_COLS) return bwd_epi_launch<IO, kModeCols>(g, x, z, dout, p, ws, dx, dz, st);
    return bwd_epi_launch<IO, kModeRows>(g, x, z, dout, p, ws, dx, dz, st);
}

}  // namespace

int64_t bwd_dd_parts(const Geom& g) { return bwd_epi_shape(g).blocks; }

hipError_t launch_bwd_pool(const Geom& g, const void* x, const void* z, const void* dout, const BwdWorkspace& ws,
                           hipStream_t st) {
    return g.io == FASTVIM_BF16 ? bwd_pool_io<IoBf16>(g, x, z, dout, ws, st) : bwd_pool_io<IoF32>(g, x, z, dout, ws, st);
}

hipError_t launch_bwd_dv(const Geom& g, const BwdWorkspace& ws, hipStream_t st) {
    const int64_t total = g.B * g.T * 2 * g.NX;
    hipLaunchKernelGGL(bwd_dv_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, ws.dvp, ws.dv, g.B,
                       g.T, ws.G, (int)ws.S, (int)g.R, (int)g.NX, bwd_rmax(g.R));
    return hipGetLastError();
}

hipError_t launch_bwd_du(const Geom& g, const fastvim_params& p, const BwdWorkspace& ws, hipStream_t st) {
    const int64_t M = g.B * g.T;
    const dim3 grid((unsigned)((M + 4 * kDuTok - 1) / (4 * kDuTok)), (unsigned)((g.E + 63) / 64));
    hipLaunchKernelGGL(bwd_du_kernel, grid, dim3(256), 0, st, ws.du_f, ws.du_b, ws.dv, p.fwd.x_proj_w,
                       p.bwd.x_proj_w, ws.du, M, g.E, (int)g.NX);
    return hipGetLastError();
}

hipError_t launch_bwd_dwx(const Geom& g, const BwdWorkspace& ws, hipStream_t st) {
    const int64_t M = g.B * g.T;
    const int NO = (int)(2 * g.NX);
    const dim3 grid((unsigned)ws.MC, (unsigned)((g.E + 63) / 64));
    switch (bwd_rmax(g.R)) {  // NO <= 2 (RMAX + 32)
        case 16: hipLaunchKernelGGL(bwd_dwx_kernel<6>, grid, dim3(256), 0, st, ws.dv, ws.fwd.u, ws.dWxp, M, g.E, NO); break;
        case 32: hipLaunchKernelGGL(bwd_dwx_kernel<8>, grid, dim3(256), 0, st, ws.dv, ws.fwd.u, ws.dWxp, M, g.E, NO); break;
        case 48: hipLaunchKernelGGL(bwd_dwx_kernel<10>, grid, dim3(256), 0, st, ws.dv, ws.fwd.u, ws.dWxp, M, g.E, NO); break;
        default: hipLaunchKernelGGL(bwd_dwx_kernel<12>, grid, dim3(256), 0, st, ws.dv, ws.fwd.u, ws.dWxp, M, g.E, NO); break;
    }
    return hipGetLastError();
}

hipError_t launch_colsum(const float* in, int64_t rows, int64_t cols, int64_t ld, float* out, float* out2,
                         float* tmp, hipStream_t st) {
    const unsigned cb = (unsigned)((cols + kColTile - 1) / kColTile);
    if (rows <= kColRowsPerBlock) {
        hipLaunchKernelGGL(colsum_kernel, dim3(cb, 1), dim3(256), 0, st, in, rows, cols, ld, rows, out, out2);
        return hipGetLastError();
    }
    const int64_t nc = (rows + kColRowsPerBlock - 1) / kColRowsPerBlock;
    hipLaunchKernelGGL(colsum_kernel, dim3(cb, (unsigned)nc), dim3(256), 0, st, in, rows, cols, ld,
                       (int64_t)kColRowsPerBlock, tmp, (float*)nullptr);
    hipLaunchKernelGGL(colsum_kernel, dim3(cb, 1), dim3(256), 0, st, (const float*)tmp, nc, cols, cols, nc, out,
                       out2);
    return hipGetLastError();
}

hipError_t launch_colsum_batch(ColsumBatch bt, hipStream_t st) {
    int64_t blk = 0;
    for (int k = 0; k < bt.n; ++k) {
        bt.seg[k].blk0 = blk;
        blk += (bt.seg[k].cols + kColTile - 1) / kColTile;
    }
    if (blk == 0) return hipSuccess;
    hipLaunchKernelGGL(colsum_batch_kernel, dim3((unsigned)blk), dim3(256), 0, st, bt);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
    return hipGetLastError();
}

hipError_t launch_bwd_epilogue(const Geom& g, const void* x, const void* z, const void* dout,
                               const fastvim_params& p, const BwdWorkspace& ws, void* dx, void* dz, hipStream_t st) {
    return g.io == FASTVIM_BF16 ? bwd_epi_dispatch<IoBf16>(g, x, z, dout, p, ws, dx, dz, st)
                                : bwd_epi_dispatch<IoF32>(g, x, z, dout, p, ws, dx, dz, st);
}

}  // namespace fastvim
