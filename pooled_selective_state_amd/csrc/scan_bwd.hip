// Adjoint of the selective scan (backward pass of the layer): for one image,
// one direction and 64 channels, the gradients of L with respect to the
// scanned tokens u, the x_proj outputs (low-rank step input, B_t, C_t) and the
// direction's dt_proj_w, dt_proj_b and A_log, given gs = dL/ds.
//
// The forward recurrence is the one of scan_core.h (FastVim summary page,
// gptget.net, arXiv 2502.00594, section 方法详解 bullets 3-4; section 术语表,
// "State Space Model").  With k the traversal step, a_k[n] = exp(Delta_k A[n])
// and H_k = a_k H_{k-1} + Delta_k B_k[n] u_k, its adjoint runs backwards in k:
//   lambda_k[n] = C_k[n] gs_k + a_{k+1}[n] lambda_{k+1}[n]
//   dDelta_k    = sum_n lambda_k[n] (A[n] a_k[n] H_{k-1}[n] + B_k[n] u_k)
//   du_k        = Delta_k sum_n lambda_k[n] B_k[n]
//   dB_k[n]     = sum_e lambda_k[e, n] Delta_k[e] u_k[e]
//   dC_k[n]     = sum_e gs_k[e] H_k[e, n]
//   dA_log[n]  += lambda_k[n] a_k[n] Delta_k H_{k-1}[n] A[n]
// and through Delta = softplus(q), q = dt_proj_w delta_lowrank + dt_proj_b,
//   dq_k = dDelta_k sigmoid(q_k),  d dt_proj_b += dq_k,
//   d dt_proj_w[e, r] += dq_k delta_k[r],  ddelta_k[r] = sum_e dt_proj_w[e, r] dq_k[e].
//
// One 256-thread workgroup takes (image b, channel group g, direction d),
// with the lane layout of the forward scan: 4 lanes per channel, lane q
// holding the states n = 4q .. 4q + 3.  All x_proj rows of the sequence are
// staged in LDS once (the forward scan's row layout, zero-filled past T; in
// dynamic LDS, so the longest sequence is the one whose rows and the flush
// buffer fit in a workgroup's 160 KB: bwd_tmax); a
// lane loads the token values u and adjoint inputs gs of its own steps
// q + 4j one chunk ahead of their use.  Then:
//   1. a forward sweep (the forward scan's own chunk code) recomputes the
//      states, writes s^d (needed by the output adjoint) and stores the state
//      entering every chunk of kChunk steps to the lane's own checkpoint
//      region of the workspace (L2-resident until the reverse sweep);
//   2. a reverse sweep over the chunks, last first, reads the chunk's
//      checkpoint (one chunk ahead), recomputes the chunk's step sizes and its
//      kChunk states from it, then walks the chunk's steps backwards carrying
//      lambda.
// The sweeps are bound by instruction issue (three exp2 per state and step:
// forward, per chunk and per group of 4 steps), not by memory or occupancy.
// Sums over n stay inside a quad (DPP).  Sums over channels e (dB, dC and
// ddelta, needed per step) are taken over the 4 channels of each DPP row of
// 16 lanes with two row rotations, written by the row's first quad into an
// LDS buffer of kBwdFlush steps x 16 rows, and every kBwdFlush steps the
// workgroup adds the 16 row partials and stores one partial per channel
// group (B, G, T, S) for a later kernel to add over the groups.  Per-image
// partials of the parameter gradients (summed over t) go to (B, E, ...)
// buffers, summed over images by a later kernel.  No atomics: every sum has
// a fixed order.
//
// LOCAL: direction 1 is LBMamba's local backward scan (LBMamba article,
// 论文创新点 1-2), run on the forward direction's parameters (the caller
// passes them in pb) with its state reset at the top of every window of
// kChunk steps aligned at t = 0.  Its traversal is padded at the start to
// nrow = kChunk ceil(T / kChunk) steps, traversal step ti being
// t = nrow - 1 - ti, so that each chunk is exactly one window: the state
// entering every chunk is zero (no forward sweep, no checkpoints), no
// adjoint crosses a chunk boundary (the reset step's decay is zero), and the
// padding steps (t >= T: zero rows, inputs and adjoint inputs, step size 0)
// contribute nothing.  Its s_bwd comes from the forward scan kernel.
#include "scan_core.h"
#include "bwd_internal.h"

namespace fastvim {
namespace {

constexpr int kBwdThreads = 256;                   // one direction: 64 channels x 4 lanes
constexpr int kBwdFlush = 8;                       // steps per flush of the channel sums
constexpr int kBwdRows = kBwdThreads / 16;         // DPP rows of 16 lanes per workgroup
constexpr int kLdsBytes = 160 * 1024;             // LDS of one workgroup on gfx950
static_assert(kBwdThreads / kLps == kScanCh && kScanCh == kBwdCh, "a workgroup covers one channel group");
static_assert(kChunk % kBwdFlush == 0, "whole flushes per chunk");
static_assert(kChunk == FASTVIM_LOCAL_WINDOW, "the local scan's windows are the chunks");

template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Sum over the 4 quads of a DPP row of 16 lanes (lanes i, i+4, i+8, i+12).
__device__ __forceinline__ float row_quads_sum(float v) {
    v += dpp_row<0x124>(v);  // row_ror:4
    v += dpp_row<0x128>(v);  // row_ror:8
    return v;
}
__device__ __forceinline__ float sigmoid_f(float q) { return __builtin_amdgcn_rcpf(1.f + __expf(-q)); }

// Lane m of the quad's value (m a compile-time constant after unrolling).
__device__ __forceinline__ float qpick(int m, float v) {
    return m == 0 ? quad_bcast<0>(v) : m == 1 ? quad_bcast<1>(v) : m == 2 ? quad_bcast<2>(v) : quad_bcast<3>(v);
}

// One step of the forward recurrence on the lane's 4 states, from the LDS
// row of the step (B_t at RMAX + 4q).
template <int RMAX>
__device__ __forceinline__ void recompute_step(float (&hs)[kNs], const float* row, float dlt, float us,
                                               const float (&A2)[kNs], int q) {
    const f32x4 b4 = *reinterpret_cast<const f32x4*>(row + RMAX + kNs * q);
    const float bt[kNs] = {b4.x, b4.y, b4.z, b4.w};
    const float du = dlt * us;
#pragma unroll
    for (int n = 0; n < kNs; ++n) hs[n] = fmaf(__builtin_amdgcn_exp2f(dlt * A2[n]), hs[n], du * bt[n]);
}

template <int RMAX>
constexpr int red_floats() { return kBwdFlush * kBwdRows * row_stride_lds<RMAX>(); }

template <int RMAX, bool LOCAL>
__global__ void __launch_bounds__(kBwdThreads) scan_bwd_kernel(BwdScanArgs a) {
    constexpr int S = row_stride_lds<RMAX>();
    constexpr int kWQ = RMAX / 4;
    constexpr int kPre = (S + 15) / 16;          // row positions per lane (16 lanes per row)
    constexpr int kPasses = 8;                   // 16 rows per pass, staged 8 passes at a time
    extern __shared__ __attribute__((aligned(16))) float rows[];  // [16 ceil(T / 16)][S]
    __shared__ __attribute__((aligned(16))) float red[red_floats<RMAX>()];

    const int tid = threadIdx.x;
    const int dir = blockIdx.y;
    const int64_t b = blockIdx.x / a.G;
    const int gi = (int)(blockIdx.x % a.G);
    const int ch = tid / kLps, q = tid & 3;
    const int64_t e = (int64_t)gi * kScanCh + ch;
    const bool valid = e < a.E;
    const int64_t ec = valid ? e : a.E - 1;
    const int T = (int)a.T, R = a.R, NX = a.NX, E = (int)a.E;
    const fastvim_dir_params p = dir ? a.pb : a.pf;
    const float kLog2e = 1.4426950408889634f;

    ScanLane<RMAX> L;
    L.dir = dir;
    L.l = q;
    L.q = q;
    L.valid = valid;
    float An[kNs];
#pragma unroll
    for (int n = 0; n < kNs; ++n) {
        An[n] = -expf(p.A_log[ec * 16 + kNs * q + n]);
        L.A2[n] = An[n] * kLog2e;
        L.hs[n] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < kWQ; ++i) {
        const int r = q + 4 * i;
        L.wq[i] = r < R ? p.dt_proj_w[ec * R + r] : 0.f;
    }
    L.bias = p.dt_proj_b[ec];
    L.sstep = dir ? -(int64_t)E : (int64_t)E;
    L.sq = (dir ? a.s_b + (int64_t)(T - 1) * E : a.s_f) + b * T * E + ec + q * L.sstep;

    // stage this direction's x_proj rows at their traversal steps, zeros past T
    const int nch = (T + kChunk - 1) / kChunk;
    const int nrow = nch * kChunk;
    const bool lw = LOCAL && dir == 1;   // local backward scan: windows = chunks
    const int toff = lw ? nrow - T : 0;  // padding steps at the start of its traversal
    // time of traversal step ti (outside [0, T) for padding and steps past T)
    auto time_of = [&](int ti) { return dir ? T - 1 + toff - ti : ti; };
    {
        // row t at xb + 2 t NX; the local scan reads the forward direction's
        // rows (the projection stage writes only those in local mode)
        const float* xb = a.xdbl + (b * T * 2 + (lw ? 0 : dir)) * (int64_t)NX;
        const int prow = tid / 16, po = tid % 16;
        int scol[kPre];
#pragma unroll
        for (int i = 0; i < kPre; ++i) scol[i] = po + 16 * i < S ? lds_source_col<RMAX>(po + 16 * i, R) : -1;
        // 8 passes of 16 rows in flight at a time (all of a sequence up to 128 steps)
#pragma unroll 1
        for (int base = 0; base < nrow; base += 16 * kPasses) {
            float stage[kPasses][kPre];
#pragma unroll
            for (int ps = 0; ps < kPasses; ++ps) {
                const int ti = base + prow + 16 * ps;
                const int t = time_of(ti);
                const bool real = t >= 0 && t < T;
#pragma unroll
                for (int i = 0; i < kPre; ++i)
                    stage[ps][i] = (real && scol[i] >= 0) ? xb[2 * t * NX + scol[i]] : 0.f;
            }
#pragma unroll
            for (int ps = 0; ps < kPasses; ++ps) {
                const int ti = base + prow + 16 * ps;
                if (ti < nrow) {
#pragma unroll
                    for (int i = 0; i < kPre; ++i)
                        if (po + 16 * i < S) rows[ti * S + po + 16 * i] = stage[ps][i];
                }
            }
        }
    }
    // Token values and adjoint inputs of the lane's own steps of chunk c (zero
    // past T and for channels past E, which then contribute nothing to the
    // channel sums), loaded one chunk ahead of their use.
    const float* ub = a.u + b * T * E + ec;
    const float* gb = a.gs + b * T * E + ec;
    auto load_steps = [&](const float* src, int c, float (&v)[kJ]) {
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const int t = time_of(c * kChunk + q + 4 * j);
            v[j] = (valid && t >= 0 && t < T) ? src[(int64_t)t * E] : 0.f;
        }
    };
    // The lane's states entering chunk c, written by the forward sweep and
    // read back by the reverse sweep (its own region of the workspace).
    float* ck = a.ckpt + (((int64_t)dir * a.B + b) * a.G + gi) * a.nchk * kBwdThreads * 4 + tid * 4;
    float un[kJ];
    load_steps(ub, 0, un);
    __syncthreads();

    // 1. forward sweep: outputs s^d and the state entering every chunk (not
    // for the local scan, whose chunks all start from zero)
    ScanArgs sa{};
    sa.T = T;
#pragma unroll 1
    for (int c = 0; c < (lw ? 0 : nch); ++c) {
        *reinterpret_cast<f32x4*>(ck + c * kBwdThreads * 4) = f32x4{L.hs[0], L.hs[1], L.hs[2], L.hs[3]};
        float ucur[kJ];
#pragma unroll
        for (int j = 0; j < kJ; ++j) ucur[j] = un[j];
        if (c + 1 < nch) load_steps(ub, c + 1, un);
        scan_chunk<RMAX, false>(sa, L, rows + c * kChunk * S, ucur, (int64_t)c * kChunk);
    }

    // 2. reverse sweep
    float carry[kNs], dA[kNs], dW[kWQ], db = 0.f;
    float gn[kJ];
    f32x4 hn;
    load_steps(ub, nch - 1, un);
    load_steps(gb, nch - 1, gn);
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    hn = lw ? zero4 : *reinterpret_cast<const f32x4*>(ck + (nch - 1) * kBwdThreads * 4);
#pragma unroll
    for (int n = 0; n < kNs; ++n) carry[n] = dA[n] = 0.f;
#pragma unroll
    for (int i = 0; i < kWQ; ++i) dW[i] = 0.f;
    float* du_dir = (dir ? a.du_b : a.du_f) + b * T * E + ec;
    float* dvp = a.dvp + (((int64_t)dir * a.B + b) * a.G + gi) * T * S;
    const bool row_writer = (tid & 15) < 4;  // first quad of each DPP row
    float* red_row = red + (tid / 16) * S;

#pragma unroll 1
    for (int c = nch - 1; c >= 0; --c) {
        const float* dr = rows + c * kChunk * S;
        const int base = c * kChunk;
        float uc[kJ], gc[kJ];
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            uc[j] = un[j];
            gc[j] = gn[j];
        }
        const float h0[kNs] = {hn.x, hn.y, hn.z, hn.w};
        if (c > 0) {  // the next (earlier) chunk's inputs and state, while this one computes
            load_steps(ub, c - 1, un);
            load_steps(gb, c - 1, gn);
            hn = lw ? zero4 : *reinterpret_cast<const f32x4*>(ck + (c - 1) * kBwdThreads * 4);
        }
        // step sizes (and sigmoid of their pre-activation) of the own steps
        float qv[kJ], dl[kJ], sg[kJ];
        scan_step_preact<RMAX>(L, dr, qv);
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const int t = time_of(base + q + 4 * j);
            const bool in = t >= 0 && t < T;
            dl[j] = in ? softplus_f(qv[j]) : 0.f;
            sg[j] = in ? sigmoid_f(qv[j]) : 0.f;
        }
        // the states entering each group of 4 steps: hb[j] for steps 4j .. 4j + 3
        float hb[kJ][kNs];
        {
            float hs[kNs];
#pragma unroll
            for (int n = 0; n < kNs; ++n) hs[n] = hb[0][n] = h0[n];
#pragma unroll
            for (int s = 0; s + 4 < kChunk; ++s) {
                const int m = s & 3, j = s >> 2;
                recompute_step<RMAX>(hs, dr + s * S, qpick(m, dl[j]), qpick(m, uc[j]), L.A2, q);
                if (m == 3) {
#pragma unroll
                    for (int n = 0; n < kNs; ++n) hb[j + 1][n] = hs[n];
                }
            }
        }
        // Groups of 4 steps, last first, one group per iteration of a rolled
        // loop (so one group's values are live at a time): the group's inputs
        // sit at index kJ - 1 of arrays rotated right after each group.
#pragma unroll 1
        for (int j = kJ - 1; j >= 0; --j) {
            const float* gr = dr + 4 * j * S;  // LDS row of the group's first step
            float Hs[4][kNs], Av[4][kNs];
            {
                float hs[kNs];
#pragma unroll
                for (int n = 0; n < kNs; ++n) hs[n] = hb[kJ - 1][n];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float dlt = qpick(m, dl[kJ - 1]), us = qpick(m, uc[kJ - 1]);
                    const f32x4 b4 = *reinterpret_cast<const f32x4*>(gr + m * S + RMAX + kNs * q);
                    const float bt[kNs] = {b4.x, b4.y, b4.z, b4.w};
                    const float du = dlt * us;
#pragma unroll
                    for (int n = 0; n < kNs; ++n) {
                        Av[m][n] = __builtin_amdgcn_exp2f(dlt * L.A2[n]);
                        hs[n] = fmaf(Av[m][n], hs[n], du * bt[n]);
                        Hs[m][n] = hs[n];
                    }
                }
            }
            const int half = (4 * j) / kBwdFlush;
            float duo = 0.f;
#pragma unroll
            for (int m = 3; m >= 0; --m) {
                const float dlt = qpick(m, dl[kJ - 1]), ut = qpick(m, uc[kJ - 1]);
                const float g = qpick(m, gc[kJ - 1]), sgs = qpick(m, sg[kJ - 1]);
                const float* row = gr + m * S;
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(row + RMAX + kNs * q);
                const f32x4 c4 = *reinterpret_cast<const f32x4*>(row + RMAX + 16 + kNs * q);
                const float bt[kNs] = {b4.x, b4.y, b4.z, b4.w}, ct[kNs] = {c4.x, c4.y, c4.z, c4.w};
                float ddl = 0.f, dup = 0.f, cb[kNs], cc[kNs];
                const float dut = dlt * ut;
#pragma unroll
                for (int n = 0; n < kNs; ++n) {
                    const float av = Av[m][n];
                    const float hp = m > 0 ? Hs[m > 0 ? m - 1 : 0][n] : hb[kJ - 1][n];
                    const float lam = fmaf(ct[n], g, carry[n]);
                    ddl = fmaf(lam, fmaf(An[n] * av, hp, bt[n] * ut), ddl);
                    dup = fmaf(lam, bt[n], dup);
                    cb[n] = lam * dut;
                    cc[n] = g * Hs[m][n];
                    dA[n] = fmaf(lam * av, dlt * hp, dA[n]);
                    carry[n] = av * lam;
                }
                ddl = quad_sum(ddl);
                dup = quad_sum(dup);
                duo = (m == q) ? dlt * dup : duo;
                const float dq = ddl * sgs;
                db += dq;
                // d dt_proj_w over the lane's quarter r = q + 4i, and that
                // quarter's terms of ddelta
                float cd[kWQ];
                const float* dq_row = row + q * kWQ;
#pragma unroll
                for (int i = 0; i < kWQ; i += 4) {
                    const f32x4 d4 = *reinterpret_cast<const f32x4*>(dq_row + i);
                    dW[i] = fmaf(dq, d4.x, dW[i]);
                    dW[i + 1] = fmaf(dq, d4.y, dW[i + 1]);
                    dW[i + 2] = fmaf(dq, d4.z, dW[i + 2]);
                    dW[i + 3] = fmaf(dq, d4.w, dW[i + 3]);
                }
#pragma unroll
                for (int i = 0; i < kWQ; ++i) cd[i] = row_quads_sum(L.wq[i] * dq);
#pragma unroll
                for (int n = 0; n < kNs; ++n) {
                    cb[n] = row_quads_sum(cb[n]);
                    cc[n] = row_quads_sum(cc[n]);
                }
                if (row_writer) {
                    float* rr = red_row + (4 * j + m - half * kBwdFlush) * kBwdRows * S;
#pragma unroll
                    for (int i = 0; i < kWQ; i += 4)
                        *reinterpret_cast<f32x4*>(rr + q * kWQ + i) = f32x4{cd[i], cd[i + 1], cd[i + 2], cd[i + 3]};
                    *reinterpret_cast<f32x4*>(rr + RMAX + kNs * q) = f32x4{cb[0], cb[1], cb[2], cb[3]};
                    *reinterpret_cast<f32x4*>(rr + RMAX + 16 + kNs * q) = f32x4{cc[0], cc[1], cc[2], cc[3]};
                }
            }
            {
                const int t = time_of(base + 4 * j + q);
                if (valid && t >= 0 && t < T) du_dir[(int64_t)t * E] = duo;
            }
            if ((4 * j) % kBwdFlush == 0) {
                // add the 16 row partials of these kBwdFlush steps; one partial per channel group
                __syncthreads();
                for (int o = tid; o < kBwdFlush * S; o += kBwdThreads) {
                    const int st = o / S, pos = o - st * S;
                    const int t = time_of(base + half * kBwdFlush + st);
                    const float* src = red + st * kBwdRows * S + pos;
                    float sum = 0.f;
#pragma unroll
                    for (int r = 0; r < kBwdRows; ++r) sum += src[r * S];
                    if (t >= 0 && t < T) dvp[(int64_t)t * S + pos] = sum;
                }
                __syncthreads();
            }
            // next group's inputs to index kJ - 1
#pragma unroll
            for (int k = kJ - 1; k > 0; --k) {
                dl[k] = dl[k - 1];
                uc[k] = uc[k - 1];
                gc[k] = gc[k - 1];
                sg[k] = sg[k - 1];
#pragma unroll
                for (int n = 0; n < kNs; ++n) hb[k][n] = hb[k - 1][n];
            }
        }
        if (lw) {  // the chunk's first step is a reset: nothing carries into the previous window
#pragma unroll
            for (int n = 0; n < kNs; ++n) carry[n] = 0.f;
        }
    }

    // per-image partials of the parameter gradients
    if (valid) {
        const int64_t pe = ((int64_t)dir * a.B + b) * E + ec;
#pragma unroll
        for (int n = 0; n < kNs; ++n) a.dAp[pe * 16 + kNs * q + n] = dA[n] * An[n];
#pragma unroll
        for (int i = 0; i < kWQ; ++i) {
            const int r = q + 4 * i;
            if (r < R) a.dWdtp[pe * R + r] = dW[i];
        }
        if (q == 0) a.dbp[pe] = db;
    }
}

template <int RMAX>
size_t rows_bytes(int64_t T) {
    return (size_t)((T + kChunk - 1) / kChunk * kChunk) * row_stride_lds<RMAX>() * sizeof(float);
}

template <int RMAX, bool LOCAL>
hipError_t scan_bwd_launch_l(const BwdScanArgs& a, hipStream_t st) {
    const size_t lds = rows_bytes<RMAX>(a.T);
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&scan_bwd_kernel<RMAX, LOCAL>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((scan_bwd_kernel<RMAX, LOCAL>), dim3((unsigned)(a.B * a.G), 2), dim3(kBwdThreads), lds, st, a);
    return hipGetLastError();
}

template <int RMAX>
hipError_t scan_bwd_launch(const BwdScanArgs& a, hipStream_t st) {
    return a.local ? scan_bwd_launch_l<RMAX, true>(a, st) : scan_bwd_launch_l<RMAX, false>(a, st);
}

template <int RMAX>
int64_t tmax_for() {
    const int64_t per_row = row_stride_lds<RMAX>() * (int64_t)sizeof(float);
    return (kLdsBytes - red_floats<RMAX>() * (int64_t)sizeof(float)) / per_row / kChunk * kChunk;
}

}  // namespace

int bwd_rmax(int64_t R) { return R <= 16 ? 16 : R <= 32 ? 32 : R <= 48 ? 48 : 64; }

int64_t bwd_tmax(int64_t R) {
    switch (bwd_rmax(R)) {
        case 16: return tmax_for<16>();
        case 32: return tmax_for<32>();
        case 48: return tmax_for<48>();
        default: return tmax_for<64>();
    }
}

hipError_t launch_scan_bwd(const BwdScanArgs& a, hipStream_t st) {
    switch (bwd_rmax(a.R)) {
        case 16: return scan_bwd_launch<16>(a, st);
        case 32: return scan_bwd_launch<32>(a, st);
        case 48: return scan_bwd_launch<48>(a, st);
        default: return scan_bwd_launch<64>(a, st);
    }
}

}  // namespace fastvim
