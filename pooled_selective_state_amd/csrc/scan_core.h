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
// the same row staging and step-size work.)
//
// Time is walked in chunks of kChunk steps in traversal order (ascending t
// forward, descending t backward).  The x_proj rows of the steps (low-rank
// step input, B_t, C_t of both directions) sit in LDS, row stride RMAX + 32:
// positions [0, RMAX) hold the low-rank input permuted so that the quarter
// r = q + 4i of quad lane q is contiguous (position q * RMAX/4 + i, zero past
// R), then B_t at [RMAX, RMAX + 16) and C_t at [RMAX + 16, RMAX + 32), so
// every lane reads its operands as 16-byte vectors.  Every chunk runs two
// phases:
//   3. each quad computes every step's dt_proj dot product, each lane over
//      its quarter of the (register-resident) dt_proj row, summed across the
//      quad; the lane q of the quad that owns step s (s = q + 4j) keeps its
//      step size and Delta * u in registers (the step size never goes to
//      memory; with more than one quad per sequence every quad holds them);
//   4. the recurrence runs over the chunk's steps; step s takes its step size
//      from lane s mod 4 of the quad by a quad broadcast, B_t and C_t from LDS,
//      and lane 0 of the sequence stores s_t.  Broadcasts and the reduction
//      over the sequence's lanes are DPP lane moves, with no LDS round trip.
// Phase 3 runs on the VALU (scan_step_preact) or, in the standalone scan
// kernel, on the matrix cores (scan_step_preact_mfma): the chunk's 16 steps x
// the wave's 16 channels of pre-activations are one (16 x RMAX) . (RMAX x 16)
// product, RMAX / 4 v_mfma_f32_16x16x4f32 steps per wave and chunk instead of
// 16 dot products of RMAX / 4 terms, two quad sums and a select per lane.
// Two ways to fill the LDS rows:
//   scan_tile           any length: one chunk of rows at a time, the next
//                       chunk's rows loaded into registers while the current
//                       one computes (one memory round trip per chunk);
//   scan_tile_resident  T <= resident_tmax<RMAX>(): all rows and all token
//                       values of the sequence loaded at once, before the
//                       first chunk, so a sequence waits for memory once and
//                       its chunk loop holds no loads (a load there would
//                       also wait for the outputs stored so far, which share
//                       its counter); the fused kernel's scans sit on the
//                       critical path of their image while the memory system
//                       is saturated by other work.
#pragma once

#include "fastvim_internal.h"

namespace fastvim {

constexpr int kScanThreads = 512;
constexpr int kLps = 4;                            // lanes per (channel, direction) sequence
constexpr int kNs = 16 / kLps;                     // states per lane
constexpr int kScanCh = kScanThreads / 2 / kLps;   // channels per workgroup (64)
static_assert(kLps == 4 || kLps == 8, "a sequence spans one quad or one half row");
static_assert(kLps == 4, "the LDS row layout gives each lane 4 states as one vector");
constexpr int kChunk = 16;      // steps per chunk
constexpr int kJ = kChunk / 4;  // steps per lane in the step-size phase
constexpr int kRMax = 64;       // largest dt rank
constexpr int kRowLanes = kScanThreads / (2 * kChunk);  // lanes per staged x_proj row (16)
constexpr int kScanLdsFloats = 12288;                   // 48 KB of rows

// LDS row stride and the longest sequence whose rows fit at once.
template <int RMAX>
constexpr int row_stride_lds() { return RMAX + 32; }
template <int RMAX>
constexpr int resident_tmax() { return kScanLdsFloats / (2 * row_stride_lds<RMAX>()); }  // 128, 96, 64
template <int RMAX>
constexpr int row_loads() { return (row_stride_lds<RMAX>() + kRowLanes - 1) / kRowLanes; }  // per lane per row

// Column of an x_proj row that feeds LDS position p of a staged row, or -1
// for the zero padding of the low-rank part (see the layout above).
template <int RMAX>
__device__ __forceinline__ int lds_source_col(int p, int R) {
    constexpr int kWQ = RMAX / 4;
    if (p < RMAX) {
        const int r = 4 * (p % kWQ) + p / kWQ;
        return r < R ? r : -1;
    }
    return R + (p - RMAX);
}

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
    float xs[kScanLdsFloats];  // x_proj rows [dir][step][0, RMAX + 32), laid out as described above
};

// Source of the scanned token values: image(b) gives an accessor of u[b, t, e]
// with 32-bit offsets from the image's base (an image holds fewer than 2^31
// elements): fp32 pooled tokens, or the grid tokens of x in unpooled scan
// order (row-major t = i w + j, or column-major t = j h + i).
struct USrcPooled {
    const float* u;
    int64_t T, E;
    struct Image {
        const float* p;
        int E;
        __device__ __forceinline__ float operator()(int t, int e) const { return p[t * E + e]; }
    };
    __device__ __forceinline__ Image image(int64_t b) const { return Image{u + b * T * E, (int)E}; }
};
template <class Elem, bool COLMAJOR>
struct USrcGrid {
    const Elem* x;
    int64_t h, w, E;
    struct Image {
        const Elem* p;
        int h, w, E;
        __device__ __forceinline__ float operator()(int t, int e) const {
            const int tok = COLMAJOR ? (t % h) * w + t / h : t;
            return load_elem(p + (tok * E + e));
        }
    };
    __device__ __forceinline__ Image image(int64_t b) const {
        return Image{x + b * h * w * E, (int)h, (int)w, (int)E};
    }
};

// Step size softplus(q) = ln(1 + e^q) in fp32.  Above q = 20 it is q (the log
// term is below half an ulp of q).  Below, log1p(y) with y = e^q by Kahan's
// identity log1p(y) = ln(u) * y / (u - 1), u = 1 + y rounded (y itself when
// u == 1), which keeps the relative error within a few ulp using the
// hardware base-2 exp and log (D. Goldberg, "What every computer scientist
// should know about floating-point arithmetic", 1991, Theorem 4).
__device__ __forceinline__ float softplus_f(float q) {
    const float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
    const float y = __builtin_amdgcn_exp2f(q * kLog2e);
    const float u = 1.f + y;
    const float l = u == 1.f ? y : __builtin_amdgcn_logf(u) * kLn2 * (y * __builtin_amdgcn_rcpf(u - 1.f));
    return q > 20.f ? q : l;
}

struct ScanArgs {
    const float* xdbl;  // (B, T, 2, NX)
    fastvim_dir_params pf, pb;
    float* s_f;         // (B, T, E)
    float* s_b;
    int64_t T, E;
    int R, NX;
};

// Per-lane state of one sequence: decay rates, the lane's states, its quarter
// of the dt_proj row, the bias, and where its outputs go: quad lane q stores
// the outputs of the steps q + 4j, at sq + (traversal step) * sstep.
// wq: VALU phase 3, the lane's quarter of its dt_proj row (r = q + 4i);
// MFMA phase 3, the lane's B operand: wq[i] = dt_proj_w[c][4i + lane / 16]
// for channel c = the wave's first + lane % 16.
template <int RMAX>
struct ScanLane {
    static constexpr int kWQ = RMAX / 4;
    int dir, l, q;
    bool valid;
    float A2[kNs], hs[kNs], wq[kWQ], bias;
    float* sq;
    int64_t sstep;
    float* sqb;  // local backward scan: the lane's first output in s_bwd (its step q)
};

// LOCAL: every lane scans forward (with kScanThreads / 2 lanes a workgroup
// covers the kScanCh channels [e0, e0 + 64); with more, the next 64).
template <int RMAX, bool LOCAL = false, bool MFMA = false>
__device__ __forceinline__ void scan_lane_setup(const ScanArgs& a, int64_t b, int64_t e0, ScanLane<RMAX>& L,
                                                int64_t& ec) {
    static_assert(RMAX % 16 == 0 && RMAX <= kRMax, "dt rank bound: 16-byte aligned rows and lane quarters");
    const int tid = threadIdx.x;
    L.dir = LOCAL ? 0 : tid >> 8;
    const int ch = (tid & 255) / kLps + (LOCAL ? kScanCh * (tid >> 8) : 0);
    L.l = tid & (kLps - 1);
    L.q = tid & 3;
    const int64_t e = e0 + ch;
    L.valid = e < a.E;
    ec = L.valid ? e : a.E - 1;
    const fastvim_dir_params p = L.dir ? a.pb : a.pf;
    const int R = a.R;
    const float kLog2e = 1.4426950408889634f;
#pragma unroll
    for (int n = 0; n < kNs; ++n) {
        L.A2[n] = -expf(p.A_log[ec * 16 + kNs * L.l + n]) * kLog2e;
        L.hs[n] = 0.f;
    }
    if (MFMA) {
        // B operand of the wave's product: channel (wave's first) + lane % 16,
        // r = 4i + lane / 16, zero past R (and a valid row past E)
        const int lane = tid & 63;
        int64_t eb = e0 + (((tid & 255) >> 6) << 4) + (lane & 15) + (LOCAL ? kScanCh * (tid >> 8) : 0);
        eb = eb < a.E ? eb : a.E - 1;
#pragma unroll
        for (int i = 0; i < ScanLane<RMAX>::kWQ; ++i) {
            const int r = 4 * i + (lane >> 4);
            L.wq[i] = r < R ? p.dt_proj_w[eb * R + r] : 0.f;
        }
    } else {
        // this lane's quarter of the dt_proj row: r = q + 4i, zero past R (the
        // step-size phase then reads every r < RMAX of a row unconditionally:
        // still inside the row, whose stride is RMAX + 32)
#pragma unroll
        for (int i = 0; i < ScanLane<RMAX>::kWQ; ++i) {
            const int r = L.q + 4 * i;
            L.wq[i] = r < R ? p.dt_proj_w[ec * R + r] : 0.f;
        }
    }
    L.bias = p.dt_proj_b[ec];
    // traversal step ti is t = ti forward, t = T - 1 - ti backward
    L.sstep = L.dir ? -a.E : a.E;
    L.sq = (L.dir ? a.s_b + (a.T - 1) * a.E : a.s_f) + b * a.T * a.E + ec + L.q * L.sstep;
    L.sqb = a.s_b + b * a.T * a.E + ec + L.q * a.E;
}

// Phase 3 for the kChunk steps of LDS rows dr: qv[j] is the step-size
// pre-activation dt_proj_w[e] . delta_lowrank + dt_proj_b[e] of the lane's
// own step q + 4j.
// nv: steps of the chunk inside the sequence (kChunk unless it is the last,
// partial chunk); the dot products of the steps past them are skipped (their
// step sizes are never used).
template <int RMAX>
__device__ __forceinline__ void scan_step_preact(const ScanLane<RMAX>& L, const float* dr, float (&qv)[kJ],
                                                 int nv = kChunk) {
    constexpr int S = row_stride_lds<RMAX>();
    const float* dq = dr + L.q * ScanLane<RMAX>::kWQ;
    // one group of 4 steps per iteration; qv rotates so its indices stay constant
#pragma unroll 1
    for (int j = 0; j < kJ; ++j) {
        float own = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (4 * j + m >= nv) break;  // wave-uniform
            const float* row = dq + (4 * j + m) * S;
            float pq = 0.f;
#pragma unroll
            for (int i = 0; i < ScanLane<RMAX>::kWQ; i += 4) {  // weights and inputs past R are zero
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(row + i);
                pq = fmaf(L.wq[i], d4.x, pq);
                pq = fmaf(L.wq[i + 1], d4.y, pq);
                pq = fmaf(L.wq[i + 2], d4.z, pq);
                pq = fmaf(L.wq[i + 3], d4.w, pq);
            }
            pq = quad_sum(pq);
            own = (m == L.q) ? pq : own;
        }
#pragma unroll
        for (int t = 0; t + 1 < kJ; ++t) qv[t] = qv[t + 1];
        qv[kJ - 1] = own + L.bias;
    }
}

// Phase 3 on the matrix cores, for the wave's 16 channels and the chunk's 16
// steps: A[m][k] = low-rank input r = k0 + k of step m, read from the LDS rows
// (lane l supplies step l % 16, r = 4i + l / 16: with the row layout above
// that is position (l / 16) * RMAX/4 + i, so 4 consecutive i are one 16-byte
// read), B[k][n] = dt_proj_w[channel n][r] (the lane's wq).  Accumulator
// register i of lane l then holds step 4 (l / 16) + i of channel l % 16; it
// goes through the wave's 256 floats of LDS at qs ([channel][step]) to the
// lanes that scan those steps (lane 4c + q takes channel c's steps q + 4j).
// Two accumulators halve the chain of dependent MFMAs.  LDS operations of a
// wave complete in order, so the wave reads back what it wrote.
template <int RMAX>
__device__ __forceinline__ void scan_step_preact_mfma(const ScanLane<RMAX>& L, const float* dr, float* qs,
                                                      float (&qv)[kJ]) {
    constexpr int S = row_stride_lds<RMAX>();
    constexpr int kWQ = ScanLane<RMAX>::kWQ;
    static_assert(kWQ % 4 == 0, "k-steps in groups of 4");
    const int lane = threadIdx.x & 63;
    const float* arow = dr + (lane & 15) * S + (lane >> 4) * kWQ;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < kWQ; i += 4) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(arow + i);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, L.wq[i], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, L.wq[i + 1], acc1, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, L.wq[i + 2], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, L.wq[i + 3], acc1, 0, 0, 0);
    }
    f32x4 acc;
    acc.x = acc0.x + acc1.x;
    acc.y = acc0.y + acc1.y;
    acc.z = acc0.z + acc1.z;
    acc.w = acc0.w + acc1.w;
    *reinterpret_cast<f32x4*>(qs + (lane & 15) * 16 + 4 * (lane >> 4)) = acc;
    const float* mine = qs + (lane >> 2) * 16 + (lane & 3);
#pragma unroll
    for (int j = 0; j < kJ; ++j) qv[j] = mine[4 * j] + L.bias;
}

// Phases 3 and 4 of one chunk.  dr: this direction's LDS row of the chunk's
// local step 0; ucur: token values of the lane's steps q + 4j; base:
// traversal index of local step 0.
// LOCAL (forward lanes only): after the chunk's forward steps the lane runs
// LBMamba's local backward scan over the same kChunk steps, last first, from
// a zero state -- the window of kChunk steps aligned at t = 0 -- and stores
// it to s_bwd.  Step t of that scan decays by the same exp(Delta_t A) as step
// t of the forward scan.  KEEP_DECAYS: the chunk's decays are kept in
// registers (64 more per lane) and the local scan needs no exponential;
// otherwise it keeps the step sizes and recomputes them (where occupancy
// matters more than the exponentials).  Neither needs a second step-size pass.
// qs (MFMA phase 3 only): the wave's 256 floats of LDS.
// SLDS: every output is also stored to so, the workgroup's LDS copy
// [direction][t][channel] (T x kScanCh floats per direction, t in scan
// position order), for a consumer in the same workgroup; the workgroup then
// covers kScanCh channels (the lanes' channel is (thread % 256) / kLps).
// TAIL: the chunk may run past the sequence end (the last chunk of a length
// that is not a multiple of kChunk): the steps past it are skipped (they
// would carry zero inputs and unit decays, so skipping them changes no
// output); without TAIL every step runs.
template <int RMAX, bool WRITE_THROUGH, bool LOCAL = false, bool KEEP_DECAYS = true, bool MFMA = false,
          bool SLDS = false, bool TAIL = false>
__device__ __forceinline__ void scan_chunk(const ScanArgs& a, ScanLane<RMAX>& L, const float* dr,
                                           const float (&ucur)[kJ], int64_t base, float* qs = nullptr,
                                           float* so = nullptr) {
    constexpr int S = row_stride_lds<RMAX>();
    constexpr bool kKeep = LOCAL && KEEP_DECAYS;
    const int64_t T = a.T;
    const int chl = (threadIdx.x & 255) / kLps;  // SLDS: the lane's channel in the workgroup
    // steps of the chunk inside the sequence (wave-uniform)
    const int nv = TAIL ? (T - base < kChunk ? (int)(T - base) : kChunk) : kChunk;
    float dl[kJ], du[kJ], du0[kJ], dl0[kJ];
    float aS[kKeep ? kChunk : 1][kNs];  // decays of the chunk's steps (LOCAL, KEEP_DECAYS)
    {
        float qv[kJ];
        if (MFMA) scan_step_preact_mfma<RMAX>(L, dr, qs, qv);
        else scan_step_preact<RMAX>(L, dr, qv, nv);
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const bool in = base + L.q + 4 * j < T;
            const float d = softplus_f(qv[j]);
            dl[j] = in ? d : 0.f;
            du[j] = in ? d * ucur[j] : 0.f;
            du0[j] = du[j];
            dl0[j] = dl[j];
        }
    }
    // the recurrence, four steps (one per quad lane's step size) at a time;
    // dl / du rotate so every register index stays constant
    // B_t and C_t of the next step are read while the current one computes;
    // the outputs of each group of 4 steps are stored one per quad lane
    static_assert(kNs == 4, "one 16-byte vector of B_t and of C_t per lane");
    const float* rows = dr + RMAX + kNs * L.l;
    f32x4 bn = *reinterpret_cast<const f32x4*>(rows), cn = *reinterpret_cast<const f32x4*>(rows + 16);
    float* sp = L.sq + base * L.sstep;
#pragma unroll
    for (int k = 0; k < kJ; ++k) {
        if (TAIL && 4 * k >= nv) break;  // wave-uniform: the rest of the chunk is past the end
        float keep = 0.f;
        const float dk = dl[0], uk = du[0];
#pragma unroll
        for (int j = 0; j + 1 < kJ; ++j) {
            dl[j] = dl[j + 1];
            du[j] = du[j + 1];
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int s = 4 * k + m;
            if (TAIL && s >= nv) break;  // wave-uniform
            const float dlt = m == 0 ? quad_bcast<0>(dk) : m == 1 ? quad_bcast<1>(dk)
                            : m == 2 ? quad_bcast<2>(dk) : quad_bcast<3>(dk);
            const float dus = m == 0 ? quad_bcast<0>(uk) : m == 1 ? quad_bcast<1>(uk)
                            : m == 2 ? quad_bcast<2>(uk) : quad_bcast<3>(uk);
            const f32x4 b4 = bn, c4 = cn;
            if (s + 1 < kChunk) {
                bn = *reinterpret_cast<const f32x4*>(rows + (s + 1) * S);
                cn = *reinterpret_cast<const f32x4*>(rows + (s + 1) * S + 16);
            }
            const float bt[kNs] = {b4.x, b4.y, b4.z, b4.w}, ct[kNs] = {c4.x, c4.y, c4.z, c4.w};
            float part = 0.f;
#pragma unroll
            for (int n = 0; n < kNs; ++n) {
                const float dA = __builtin_amdgcn_exp2f(dlt * L.A2[n]);
                if (kKeep) aS[kKeep ? s : 0][n] = dA;
                L.hs[n] = fmaf(dA, L.hs[n], dus * bt[n]);
                part = fmaf(ct[n], L.hs[n], part);
            }
            part = seq_sum(part);
            keep = (m == L.q) ? part : keep;
        }
        if (L.valid && base + 4 * k + L.q < T) {
            if (WRITE_THROUGH) __hip_atomic_store(sp, keep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else *sp = keep;
            if (SLDS) {
                const int ti = (int)base + 4 * k + L.q;  // traversal step; backward: t = T - 1 - ti
                so[((L.dir ? 2 * (int)T - 1 - ti : ti) * kScanCh) + chl] = keep;
            }
        }
        sp += 4 * L.sstep;
    }
    if (LOCAL) {
        // the local backward scan over the chunk (steps past T have zero input
        // and decay 1, so the state stays zero through them)
        float hl[kNs] = {0.f, 0.f, 0.f, 0.f};
        // B_t and C_t are read from LDS again: an offset the compiler cannot
        // see through keeps it from holding the forward pass's 16 steps of
        // them in registers instead (about 128 more per lane)
        int zero = 0;
        __asm__ volatile("" : "+v"(zero));
        const float* lrows = dr + RMAX + kNs * L.l + zero;
#pragma unroll
        for (int k = kJ - 1; k >= 0; --k) {
            float keep = 0.f;
#pragma unroll
            for (int m = 3; m >= 0; --m) {
                const int s = 4 * k + m;
                if (TAIL && s >= nv) continue;  // wave-uniform: the state stays zero past the end
                const float dus = m == 0 ? quad_bcast<0>(du0[k]) : m == 1 ? quad_bcast<1>(du0[k])
                                : m == 2 ? quad_bcast<2>(du0[k]) : quad_bcast<3>(du0[k]);
                const float dlt = kKeep ? 0.f
                                : m == 0 ? quad_bcast<0>(dl0[k]) : m == 1 ? quad_bcast<1>(dl0[k])
                                : m == 2 ? quad_bcast<2>(dl0[k]) : quad_bcast<3>(dl0[k]);
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(lrows + s * S);
                const f32x4 c4 = *reinterpret_cast<const f32x4*>(lrows + s * S + 16);
                const float bt[kNs] = {b4.x, b4.y, b4.z, b4.w}, ct[kNs] = {c4.x, c4.y, c4.z, c4.w};
                float part = 0.f;
#pragma unroll
                for (int n = 0; n < kNs; ++n) {
                    const float dA = kKeep ? aS[kKeep ? s : 0][n] : __builtin_amdgcn_exp2f(dlt * L.A2[n]);
                    hl[n] = fmaf(dA, hl[n], dus * bt[n]);
                    part = fmaf(ct[n], hl[n], part);
                }
                part = seq_sum(part);
                keep = (m == L.q) ? part : keep;
            }
            if (L.valid && base + 4 * k + L.q < T) {
                float* dst = L.sqb + (base + 4 * k) * a.E;
                if (WRITE_THROUGH) __hip_atomic_store(dst, keep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                else *dst = keep;
                if (SLDS) so[(((int)T + (int)base + 4 * k + L.q) * kScanCh) + chl] = keep;
            }
        }
    }
}

// Scan channels [e0, e0 + kScanCh) of image b in both directions, any T, with
// chunk_lds_floats<RMAX>() floats of LDS at xs, and (MFMA phase 3) 256 floats
// per wave at qs.  All threads of the workgroup must call it (it synchronises
// the workgroup).
// With WRITE_THROUGH the outputs are stored with agent-scope atomic stores
// (written through to the device-coherent level), for consumers on other XCDs
// that synchronise without an L2 write-back.  RMAX bounds the dt rank R.
template <int RMAX>
constexpr int chunk_lds_floats() { return 2 * kChunk * row_stride_lds<RMAX>(); }

// KEEP_DECAYS and SLDS (with so) as scan_chunk (KEEP_DECAYS: LOCAL only).
template <int RMAX, bool WRITE_THROUGH, class USrc, bool LOCAL = false, bool MFMA = false, bool KEEP_DECAYS = true,
          bool SLDS = false>
__device__ __forceinline__ void scan_tile(const ScanArgs& a, const USrc& usrc, int64_t b, int64_t e0,
                                          float* xs /* chunk_lds_floats<RMAX>() */, float* qs = nullptr,
                                          float* so = nullptr) {
    constexpr int S = row_stride_lds<RMAX>();
    constexpr int kPre = row_loads<RMAX>();
    ScanLane<RMAX> L;
    int64_t ec;
    scan_lane_setup<RMAX, LOCAL, MFMA>(a, b, e0, L, ec);
    float* wqs = MFMA ? qs + (threadIdx.x >> 6) * 256 : nullptr;
    const int tid = threadIdx.x;
    const int NX = a.NX;
    const int64_t T = a.T;
    const int row_stride = 2 * NX;
    const float* xb = a.xdbl + b * T * row_stride;  // this image's rows: 32-bit offsets below
    const auto ui = usrc.image(b);
    const int iT = (int)T, iec = (int)ec;

    // Prefetch of one chunk into registers: lane tid fills LDS positions
    // p = tid % 16 + 16 i of x_proj row (d, s) = (tid / 256, tid / 16 % 16),
    // and loads its own u values for the steps q + 4j.
    const int prow = tid / kRowLanes, pd = prow / kChunk, ps = prow % kChunk, po = tid % kRowLanes;
    int scol[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) scol[i] = lds_source_col<RMAX>(po + kRowLanes * i, a.R);
    float pre_x[kPre], pre_u[kJ];
    const int pdr = LOCAL ? 0 : pd;  // LOCAL: both halves hold the forward rows (only the first is read)
    auto prefetch = [&](int base) {
        const int ti = base + ps;
        const float* src = xb + ((pdr ? iT - 1 - ti : ti) * row_stride + pdr * NX);
#pragma unroll
        for (int i = 0; i < kPre; ++i) pre_x[i] = (ti < iT && scol[i] >= 0) ? src[scol[i]] : 0.f;
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const int tj = base + L.q + 4 * j;
            pre_u[j] = tj < iT ? ui(L.dir ? iT - 1 - tj : tj, iec) : 0.f;
        }
    };

    const int nchunks = (iT + kChunk - 1) / kChunk;
    prefetch(0);
    for (int c = 0; c < nchunks; ++c) {
        const int base = c * kChunk;  // traversal index of local step 0
        __syncthreads();  // every lane is done reading the previous chunk's rows
#pragma unroll
        for (int i = 0; i < kPre; ++i) xs[prow * S + po + kRowLanes * i] = pre_x[i];
        float ucur[kJ];
#pragma unroll
        for (int j = 0; j < kJ; ++j) ucur[j] = pre_u[j];
        __syncthreads();
        if (c + 1 < nchunks) prefetch(base + kChunk);
        if (c + 1 == nchunks && iT % kChunk != 0)  // the last, partial chunk
            scan_chunk<RMAX, WRITE_THROUGH, LOCAL, KEEP_DECAYS, MFMA, SLDS, true>(a, L, xs + L.dir * kChunk * S,
                                                                                ucur, base, wqs, so);
        else
            scan_chunk<RMAX, WRITE_THROUGH, LOCAL, KEEP_DECAYS, MFMA, SLDS>(a, L, xs + L.dir * kChunk * S, ucur,
                                                                          base, wqs, so);
    }
}

// The same for T <= resident_tmax<RMAX>(), with every x_proj row and every
// token value of the sequence loaded at once.  Rows (t, d) are contiguous in
// xdbl; lane tid fills LDS positions tid % 16 + 16 i of rows
// r = tid / 16 + 32 p (r = 2t + d), stored at traversal step t (forward) or
// T - 1 - t (backward).  Each lane holds the token values of its steps
// q + 4j for the whole sequence (resident_tmax / 4 registers), rotated one
// chunk at a time so register indices stay constant.  One barrier in all.
// LOCAL: every lane scans forward, the workgroup covering 2 kScanCh channels
// from e0, and each chunk's local backward scan follows it (scan_chunk, its
// decays recomputed: this variant serves the single-launch kernel, whose
// streaming items share the scan items' register budget).
template <int RMAX, bool WRITE_THROUGH, class USrc, bool LOCAL = false>
__device__ __forceinline__ void scan_tile_resident(const ScanArgs& a, const USrc& usrc, int64_t b, int64_t e0,
                                                   ScanSmem& sm) {
    constexpr int S = row_stride_lds<RMAX>();
    constexpr int TM = resident_tmax<RMAX>();
    constexpr int kCM = TM / kChunk;                         // chunks at most: 8, 6, 4
    constexpr int kPre = row_loads<RMAX>();
    constexpr int kRowsPerPass = kScanThreads / kRowLanes;  // 32
    constexpr int kPasses = 2 * TM / kRowsPerPass;          // 8, 6, 4
    static_assert(2 * TM % kRowsPerPass == 0 && TM % kChunk == 0, "whole passes and chunks");
    ScanLane<RMAX> L;
    int64_t ec;
    scan_lane_setup<RMAX, LOCAL>(a, b, e0, L, ec);
    const int tid = threadIdx.x;
    const int NX = a.NX;
    const int64_t T = a.T;
    const float* xb = a.xdbl + b * T * 2 * (int64_t)NX;
    const int nrows = 2 * (int)T;
    const int prow = tid / kRowLanes, po = tid % kRowLanes;
    int scol[kPre];
#pragma unroll
    for (int i = 0; i < kPre; ++i) scol[i] = lds_source_col<RMAX>(po + kRowLanes * i, a.R);

    float stage[kPasses][kPre];
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int r = prow + kRowsPerPass * p;
#pragma unroll
        for (int i = 0; i < kPre; ++i) stage[p][i] = (r < nrows && scol[i] >= 0) ? xb[r * NX + scol[i]] : 0.f;
    }
    float uall[kCM][kJ];
    const auto ui = usrc.image(b);
#pragma unroll
    for (int c = 0; c < kCM; ++c)
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            const int tj = c * kChunk + L.q + 4 * j;
            uall[c][j] = tj < T ? ui(L.dir ? (int)T - 1 - tj : tj, (int)ec) : 0.f;
        }
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
        const int r = prow + kRowsPerPass * p;
        const int t = r >> 1, d = r & 1;
        const int ti = d ? (int)T - 1 - t : t;
        if (r < nrows) {
            float* dst = sm.xs + (d * TM + ti) * S + po;
#pragma unroll
            for (int i = 0; i < kPre; ++i) dst[kRowLanes * i] = stage[p][i];
        }
    }
    __syncthreads();

    const int nchunks = (int)((T + kChunk - 1) / kChunk);
    const float* dr = sm.xs + L.dir * TM * S;
#pragma unroll 1
    for (int c = 0; c < nchunks; ++c) {
        float ucur[kJ];
#pragma unroll
        for (int j = 0; j < kJ; ++j) ucur[j] = uall[0][j];
#pragma unroll
        for (int k = 0; k + 1 < kCM; ++k)
#pragma unroll
            for (int j = 0; j < kJ; ++j) uall[k][j] = uall[k + 1][j];
        scan_chunk<RMAX, WRITE_THROUGH, LOCAL, false>(a, L, dr + c * kChunk * S, ucur, (int64_t)c * kChunk);
    }
}

}  // namespace fastvim
