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
// One 512-thread workgroup scans kScanCh = 64 channels of one image in both
// directions: thread = dir * 256 + ch * kLps + l.  Each sequence's 16 states
// are split over its kLps = 4 lanes (lane l holds n = 4l .. 4l + 3), which
// keeps the sequential critical path of a step to 4 exp2 and a two-step quad
// reduction.  (Eight lanes per sequence, with a half-row mirror added to the
// reduction, also works but measured slower: twice the workgroups, each with
// the same chunk staging and step-size work.)  Time is walked in chunks of kChunk steps in traversal order
// (ascending t forward, descending t backward).  For each chunk:
//   1. its 2 * kChunk x_proj rows (low-rank step input, B_t, C_t of both
//      directions), loaded into registers while the previous chunk was
//      computing (16 lanes per row), go to LDS as they are;
//   2. the loads of the next chunk are issued;
//   3. each quad computes every step's dt_proj dot product, each lane over
//      its quarter of the (register-resident) dt_proj row, summed across the
//      quad; the lane q of the quad that owns step s (s = q + 4j) keeps its
//      step size and Delta * u in registers (the step size never goes to
//      memory; with more than one quad per sequence every quad holds them);
//   4. the recurrence runs over the chunk's steps; step s takes its step size
//      from lane s mod 4 of the quad by a quad broadcast, B_t and C_t from LDS,
//      and lane 0 of the sequence stores s_t.  Broadcasts and the reduction
//      over the sequence's lanes are DPP lane moves, with no LDS round trip.
#pragma once

#include "fastvim_internal.h"

namespace fastvim {

constexpr int kScanThreads = 512;
constexpr int kLps = 4;                            // lanes per (channel, direction) sequence
constexpr int kNs = 16 / kLps;                     // states per lane
constexpr int kScanCh = kScanThreads / 2 / kLps;   // channels per workgroup (64)
static_assert(kLps == 4 || kLps == 8, "a sequence spans one quad or one half row");
constexpr int kChunk = 16;      // steps per chunk
constexpr int kJ = kChunk / 4;  // steps per lane in the step-size phase
constexpr int kRMax = 64;       // largest dt rank
constexpr int kNXMax = kRMax + 32;
constexpr int kRowLanes = kScanThreads / (2 * kChunk);      // lanes per staged x_proj row (16)
constexpr int kPre = (kNXMax + kRowLanes - 1) / kRowLanes;  // x_proj values prefetched per lane (6)

// DPP quad permute: lane i of every quad of 4 takes the value of lane
// ((CTRL >> 2*(i)) & 3) of its quad.
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int M>  // broadcast lane M of each quad
__device__ __forceinline__ float quad_bcast(float v) {
    return quad_perm<M | (M << 2) | (M << 4) | (M << 6)>(v);
}
__device__ __forceinline__ float quad_sum(float v) {
    v += quad_perm<0xB1>(v);  // lanes [1, 0, 3, 2]
    v += quad_perm<0x4E>(v);  // lanes [2, 3, 0, 1]
    return v;
}
// sum over the kLps lanes of a sequence (for 8: quad sums, then lane i adds
// lane 7 - i of its half row)
__device__ __forceinline__ float seq_sum(float v) {
    v = quad_sum(v);
    if (kLps == 8) v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    return v;
}

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

// Scan channels [e0, e0 + kScanCh) of image b in both directions.  All 512 threads
// of the workgroup must call it (it synchronises the workgroup).  With
// WRITE_THROUGH the outputs are stored with agent-scope atomic stores (written
// through to the device-coherent level), for consumers on other XCDs that
// synchronise without an L2 write-back.  RMAX bounds the dt rank R.
template <int RMAX, bool WRITE_THROUGH, class USrc>
__device__ __forceinline__ void scan_tile(const ScanArgs& a, const USrc& usrc, int64_t b, int64_t e0,
                                          ScanSmem& sm) {
    const int tid = threadIdx.x;
    const int dir = tid >> 8;
    const int ch = (tid & 255) / kLps;
    const int l = tid & (kLps - 1);  // lane within the sequence
    const int q = tid & 3;           // lane within its quad
    const int64_t e = e0 + ch;
    const bool valid = e < a.E;
    const int64_t ec = valid ? e : a.E - 1;
    const fastvim_dir_params p = dir ? a.pb : a.pf;
    const int R = a.R, NX = a.NX;
    const int64_t T = a.T;
    const int64_t row_stride = 2 * (int64_t)NX;
    const float kLog2e = 1.4426950408889634f;

    float A2[kNs], hs[kNs];
#pragma unroll
    for (int n = 0; n < kNs; ++n) {
        A2[n] = -expf(p.A_log[ec * 16 + kNs * l + n]) * kLog2e;
        hs[n] = 0.f;
    }
    // this lane's quarter of the dt_proj row: r = q + 4i
    static_assert(RMAX % 4 == 0 && RMAX <= kRMax, "dt rank bound");
    constexpr int kWQ = RMAX / 4;
    float wq[kWQ];
#pragma unroll
    for (int i = 0; i < kWQ; ++i) {
        const int r = q + 4 * i;
        wq[i] = r < R ? p.dt_proj_w[ec * R + r] : 0.f;
    }
    const int nwq = (R + 3) / 4;
    const float bias = p.dt_proj_b[ec];
    const float* xb = a.xdbl + b * T * row_stride;
    float* sdst = (dir ? a.s_b : a.s_f) + b * T * a.E + ec;

    // Prefetch of one chunk into registers: lane tid loads columns
    // o = tid % 16 + 16 i of x_proj row (d, s) = (tid / 256, tid / 16 % 16),
    // and its own u values for the steps q + 4j.
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
        // 3. step sizes: quad-wide dot products, kept by the owning lane
        float dl[kJ], du[kJ];
        {
            float qv[kJ];
            const float* dr = sm.xs + dir * kChunk * kNXMax + q;
            // one group of 4 steps per iteration; qv rotates so its indices stay constant
#pragma unroll 1
            for (int j = 0; j < kJ; ++j) {
                float own = 0.f;
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const float* row = dr + (4 * j + m) * kNXMax;
                    float pq = 0.f;
#pragma unroll
                    for (int i = 0; i < kWQ; ++i)
                        if (i < nwq) pq = fmaf(wq[i], row[4 * i], pq);
                    pq = quad_sum(pq);
                    own = (m == q) ? pq : own;
                }
#pragma unroll
                for (int t = 0; t + 1 < kJ; ++t) qv[t] = qv[t + 1];
                qv[kJ - 1] = own + bias;
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
        const float* rows = sm.xs + dir * kChunk * kNXMax + R + kNs * l;
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
                const float dlt = m == 0 ? quad_bcast<0>(dk) : m == 1 ? quad_bcast<1>(dk)
                                : m == 2 ? quad_bcast<2>(dk) : quad_bcast<3>(dk);
                const float dus = m == 0 ? quad_bcast<0>(uk) : m == 1 ? quad_bcast<1>(uk)
                                : m == 2 ? quad_bcast<2>(uk) : quad_bcast<3>(uk);
                const float* row = rows + s * kNXMax;
                float part = 0.f;
#pragma unroll
                for (int n = 0; n < kNs; ++n) {
                    const float dA = __builtin_amdgcn_exp2f(dlt * A2[n]);
                    hs[n] = fmaf(dA, hs[n], dus * row[n]);
                    part = fmaf(row[16 + n], hs[n], part);
                }
                part = seq_sum(part);
                const int64_t ti = base + s;
                if (l == 0 && valid && ti < T) {
                    float* dst = sdst + (dir ? T - 1 - ti : ti) * a.E;
                    if (WRITE_THROUGH) __hip_atomic_store(dst, part, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else *dst = part;
                }
            }
        }
    }
}

}  // namespace fastvim
