// Selective-scan core shared by the standalone scan kernel and the fused
// layer kernel.
//
// FastVim summary page (gptget.net, arXiv 2502.00594): section 方法详解,
// bullet 3 -- Delta = softplus(Parameter + s_Delta(x)) from the scanned token,
// A discretised by zero-order hold; bullet 4 -- forward and backward selective
// scans; section 术语表, "State Space Model" -- h_t = A h_{t-1} + B x_t,
// y_t = C h_t.  Per channel e, A[e, n] = -exp(A_log[e, n]), H = 0 at the start:
//   H[n] <- exp(Delta_t A[e, n]) H[n] + Delta_t B_t[n] u_t,   s_t = sum_n C_t[n] H[n]
//
// One 512-thread workgroup scans 64 channels of one image in both directions:
// thread = dir * 256 + ch * 4 + q, where q selects the state quarter
// n = 4q .. 4q+3.  Splitting each sequence's 16 states over the 4 lanes of a
// quad keeps the sequential critical path of a step to 4 exp2 and a two-step
// quad reduction.  Time is walked in chunks of kChunk steps in traversal order
// (ascending t forward, descending t backward).  For each chunk:
//   1. its 2 * kChunk x_proj rows (low-rank step input, B_t, C_t of both
//      directions), loaded into registers while the previous chunk was
//      computing (8 lanes per row), go to LDS as they are;
//   2. the loads of the next chunk are issued;
//   3. each lane computes the step size and Delta * u of the kJ steps
//      s = q + 4j it owns (the step size never leaves registers);
//   4. the recurrence runs over the chunk's steps; step s takes its step size
//      from lane s mod 4 of the quad by a quad broadcast, B_t and C_t from LDS,
//      and lane 0 of the quad stores s_t.
#pragma once

#include "fastvim_internal.h"

namespace fastvim {

constexpr int kScanThreads = 512;
constexpr int kScanCh = 64;     // channels per workgroup
constexpr int kChunk = 32;      // steps per chunk
constexpr int kJ = kChunk / 4;  // steps per lane in the step-size phase
constexpr int kRMax = 64;       // largest dt rank
constexpr int kNXMax = kRMax + 32;
constexpr int kRowLanes = kScanThreads / (2 * kChunk);      // lanes per staged x_proj row (8)
constexpr int kPre = (kNXMax + kRowLanes - 1) / kRowLanes;  // x_proj values prefetched per lane (12)

struct alignas(16) ScanSmem {
    float xs[2 * kChunk * kNXMax];  // the chunk's x_proj rows [dir][s][0, NX), row stride kNXMax
};

// Source of the scanned token value u[b, t, e] (fp32 pooled tokens, or grid
// tokens of x in unpooled scan order).
struct USrcPooled {
    const float* u;
    int64_t T, E;
    __device__ __forceinline__ float operator()(int64_t b, int64_t t, int64_t e) const {
        return u[(b * T + t) * E + e];
    }
};
template <class Elem>
struct USrcGrid {
    const Elem* x;
    int axis;
    int64_t h, w, E;
    __device__ __forceinline__ float operator()(int64_t b, int64_t t, int64_t e) const {
        return load_elem(x + (b * h * w + unpooled_token(axis, t, h, w)) * E + e);
    }
};

struct ScanArgs {
    const float* xdbl;  // (B, T, 2, NX)
    fastvim_dir_params pf, pb;
    float* s_f;         // (B, T, E)
    float* s_b;
    int64_t T, E;
    int R, NX;
};

// Scan channels [e0, e0 + 64) of image b in both directions.  All 512 threads
// of the workgroup must call it (it synchronises the workgroup).
template <class USrc>
__device__ __forceinline__ void scan_tile(const ScanArgs& a, const USrc& usrc, int64_t b, int64_t e0,
                                          ScanSmem& sm) {
    const int tid = threadIdx.x;
    const int dir = tid >> 8;
    const int ch = (tid >> 2) & (kScanCh - 1);
    const int q = tid & 3;
    const int64_t e = e0 + ch;
    const bool valid = e < a.E;
    const int64_t ec = valid ? e : a.E - 1;
    const fastvim_dir_params p = dir ? a.pb : a.pf;
    const int R = a.R, NX = a.NX;
    const int64_t T = a.T;
    const int64_t row_stride = 2 * (int64_t)NX;
    const float kLog2e = 1.4426950408889634f;

    float A2[4], hs[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        A2[n] = -expf(p.A_log[ec * 16 + 4 * q + n]) * kLog2e;
        hs[n] = 0.f;
    }
    const float* wrow = p.dt_proj_w + ec * R;
    const float bias = p.dt_proj_b[ec];
    const float* xb = a.xdbl + b * T * row_stride;
    float* sdst = (dir ? a.s_b : a.s_f) + b * T * a.E + ec;

    // Prefetch of one chunk into registers: lane tid loads columns
    // o = tid % 8 + 8 i of x_proj row (d, s) = (tid / 256, tid / 8 % 32), and
    // its own u values for the steps q + 4j.
    const int prow = tid / kRowLanes, pd = prow / kChunk, ps = prow % kChunk, po = tid % kRowLanes;
    float pre_x[kPre], pre_u[kJ];
    auto prefetch = [&](int64_t base) {
        const int64_t ti = base + ps;
        const float* src = xb + (pd ? T - 1 - ti : ti) * row_stride + (int64_t)pd * NX;
#pragma unroll
        for (int i = 0; i < kPre; ++i) {
            const int o = po + kRowLanes * i;
            pre_x[i] = (ti < T && o < NX) ? src[o] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const int64_t tj = base + q + 4 * j;
            pre_u[j] = tj < T ? usrc(b, dir ? T - 1 - tj : tj, ec) : 0.f;
        }
    };

    const int64_t nchunks = (T + kChunk - 1) / kChunk;
    prefetch(0);
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t base = c * kChunk;  // traversal index of local step 0
        // 1. stage this chunk's x_proj rows
        __syncthreads();  // every lane is done reading the previous chunk's rows
#pragma unroll
        for (int i = 0; i < kPre; ++i) {
            const int o = po + kRowLanes * i;
            if (o < NX) sm.xs[prow * kNXMax + o] = pre_x[i];
        }
        float ucur[kJ];
#pragma unroll
        for (int j = 0; j < kJ; ++j) ucur[j] = pre_u[j];
        __syncthreads();
        // 2. loads of the next chunk
        if (c + 1 < nchunks) prefetch(base + kChunk);
        // 3. step sizes of this lane's steps (dt_proj row through the cache)
        float dl[kJ], du[kJ];
        {
            float qv[kJ];
#pragma unroll
            for (int j = 0; j < kJ; ++j) qv[j] = bias;
            const float* dr = sm.xs + (dir * kChunk + q) * kNXMax;
#pragma unroll 1
            for (int r = 0; r < R; ++r) {
                const float wv = wrow[r];
#pragma unroll
                for (int j = 0; j < kJ; ++j) qv[j] = fmaf(wv, dr[4 * j * kNXMax + r], qv[j]);
            }
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
                const bool in = base + q + 4 * j < T;
                const float d = qv[j] > 20.f ? qv[j] : log1pf(__expf(qv[j]));
                dl[j] = in ? d : 0.f;
                du[j] = in ? d * ucur[j] : 0.f;
            }
        }
        // 4. the recurrence, four steps (one per quad lane's step size) at a
        //    time; dl / du rotate so every register index stays constant
        const float* rows = sm.xs + dir * kChunk * kNXMax + R + 4 * q;
        for (int k = 0; k < kJ; ++k) {
            const float dk = dl[0], uk = du[0];
#pragma unroll
            for (int j = 0; j + 1 < kJ; ++j) {
                dl[j] = dl[j + 1];
                du[j] = du[j + 1];
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int s = 4 * k + m;
                const float dlt = __shfl(dk, m, 4);
                const float dus = __shfl(uk, m, 4);
                const float* row = rows + s * kNXMax;
                float part = 0.f;
#pragma unroll
                for (int n = 0; n < 4; ++n) {
                    const float dA = __builtin_amdgcn_exp2f(dlt * A2[n]);
                    hs[n] = fmaf(dA, hs[n], dus * row[n]);
                    part = fmaf(row[16 + n], hs[n], part);
                }
                part += __shfl_xor(part, 1, 4);
                part += __shfl_xor(part, 2, 4);
                const int64_t ti = base + s;
                if (q == 0 && valid && ti < T) sdst[(dir ? T - 1 - ti : ti) * a.E] = part;
            }
        }
    }
}

}  // namespace fastvim
