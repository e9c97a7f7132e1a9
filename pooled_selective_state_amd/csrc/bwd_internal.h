// Internal declarations of the backward pass (gradients of the pooled layer).
// Not part of the public ABI.
#pragma once

#include "fastvim_internal.h"

namespace fastvim {

constexpr int kBwdCkptMin = 8;       // checkpoint chunks reserved at least (the Conv1D pass reuses the region)
constexpr int kBwdCh = 64;           // channels per scan-adjoint workgroup (one channel group)
constexpr int kBwdTokChunk = 64;     // pooled tokens per partial of d x_proj_w
constexpr int kColRowsPerBlock = 256;  // rows per first-stage block of a column sum
constexpr int kBwdStatusWords = 2;     // header of a backward workspace: [0] unused, [1] status word

// Workspace of one backward call (every region 256-byte aligned).  fwd views
// the part shared with the forward stages (u, xdbl, s_f, s_b, rows, bad) and
// its sync points to the workspace's header (kBwdStatusWords words at its
// start; word 1 is the call's status word, as in a forward workspace).
struct BwdWorkspace {
    Workspace fwd;
    float* gs;     // (B, T, E) dL/ds: the gated upstream gradient summed over the pooled axis
    float* dDp;    // (bwd_dd_parts, E) per second-pass workgroup: sum over its tokens of dL/dy * x
    float* du_f;   // (B, T, E) scan part of dL/du, forward direction; with the LayerNorm first
                   //           the (b, t) partials of d ln_w
    float* du_b;   // (B, T, E) the same, backward direction; with the LayerNorm first those of d ln_b
    float* du;     // (B, T, E) dL/du, both directions, scan and x_proj; with the LayerNorm first
                   //           the (b, t) partials of dD
    float* dvp;    // (2, B, G, T, S) channel-group partials of dL/dv, in the scan's LDS row layout
    float* ckpt;   // (2, B, G, nchk, 256, 4) scan adjoint: each lane's states entering each chunk
    float* dv;     // (B, T, 2, NX) dL/dv of both directions
    float* dAp;    // (2, B, E, 16) per-image d A_log
    float* dWdtp;  // (2, B, E, R) per-image d dt_proj_w
    float* dbp;    // (2, B, E) per-image d dt_proj_b
    float* dWxp;   // (MC, 2, NX, E) per token chunk d x_proj_w
    float* tmp;    // first-stage sums of the column reductions
    int64_t G, S, MC, tmp_floats;
    int nchk;      // checkpoint chunks per lane: max(ceil(T / 16), kBwdCkptMin)
    bool u_saved = false;  // fwd.u is the caller's saved pooled tokens (pass 1 does not pool x)
    // front: the regions before du (u, xdbl, s_f, s_b, gs, dDp, du_f, du_b),
    // free once the scan adjoint and its sums have run
    float* front = nullptr;
};

struct BwdScanArgs {
    const float* xdbl;  // (B, T, 2, NX)
    const float* u;     // (B, T, E)
    const float* gs;    // (B, T, E)
    fastvim_dir_params pf, pb;
    float *s_f, *s_b;     // (B, T, E) recomputed scan outputs
    float *du_f, *du_b;   // (B, T, E)
    float* dvp;           // (2, B, G, T, S)
    float* ckpt;          // (2, B, G, nchk, 256, 4)
    float *dAp, *dWdtp, *dbp;
    int64_t B, T, E;
    int R, NX, G;
    bool local;  // direction 1 is the local backward scan (pb holds the forward parameters)
    int nchk;    // checkpoint chunks per lane in ckpt
};

int bwd_rmax(int64_t R);  // the dt-rank bound (16, 32, 48, 64) whose kernel instance serves R
// Longest scan the scan adjoint takes at dt rank R: the sequence's x_proj rows
// and the flush buffer fit in one workgroup's LDS (720, 512, 384, 288 steps).
int64_t bwd_tmax(int64_t R);
// Second-pass workgroups (each a run of consecutive tokens of one grid row,
// or of one image's kept tokens when masked): the rows of dDp.
int64_t bwd_dd_parts(const Geom& g);
// front_floats (optional): floats of the regions before du (BwdWorkspace::front).
size_t bwd_workspace_layout(const Geom& g, void* base, BwdWorkspace* ws, int64_t* front_floats = nullptr);

hipError_t launch_bwd_pool(const Geom& g, const void* x, const void* z, const void* dout, const BwdWorkspace& ws,
                           hipStream_t st);
hipError_t launch_scan_bwd(const BwdScanArgs& a, hipStream_t st);
hipError_t launch_bwd_dv(const Geom& g, const BwdWorkspace& ws, hipStream_t st);
hipError_t launch_bwd_du(const Geom& g, const fastvim_params& p, const BwdWorkspace& ws, hipStream_t st);
hipError_t launch_bwd_dwx(const Geom& g, const BwdWorkspace& ws, hipStream_t st);
// out[j] = sum_i in[i * ld + j] for j < cols (and the same into out2 when
// given), in a fixed order; more than kColRowsPerBlock rows go through tmp
// (ceil(rows / kColRowsPerBlock) * cols floats).
hipError_t launch_colsum(const float* in, int64_t rows, int64_t cols, int64_t ld, float* out, float* out2,
                         float* tmp, hipStream_t st);
// Up to kColsumSegs column sums of at most kColRowsPerBlock rows each, in one
// launch, with the arithmetic of launch_colsum (blk0 is filled in).
constexpr int kColsumSegs = 8;
struct ColsumSeg {
    const float* in;
    int64_t rows, cols, ld;
    float *out, *out2;
    int64_t blk0;
};
struct ColsumBatch {
    ColsumSeg seg[kColsumSegs];
    int n;
};
hipError_t launch_colsum_batch(ColsumBatch bt, hipStream_t st);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t st);
hipError_t launch_bwd_epilogue(const Geom& g, const void* x, const void* z, const void* dout,
                               const fastvim_params& p, const BwdWorkspace& ws, void* dx, void* dz, hipStream_t st);

// Backward through the post-SSM LayerNorm (bwd_norm.hip), for E <= 2048.
// Pass 1 needs fwd.s_f and fwd.s_b; it writes dz, g = dL/dy into dx, gs, and
// the (B T, E) partials of dD, d ln_w and d ln_b into du, du_f and du_b.
// Pass 2 needs du and turns dx into dL/dx.
bool bwd_norm_supported(const Geom& g);

// Backward second pass of a layer whose x is the producer Conv1D's input
// (conv.hip): dx (through the conv) and dz, and bwd_conv_parts(g) rows of
// partials [dD (E) | d conv_b (E) | d conv_w (E, 4)] into parts.
int64_t bwd_conv_parts(const Geom& g);
hipError_t launch_bwd_conv_epilogue(const Geom& g, const void* x, const void* z, const void* dout,
                                    const fastvim_params& p, const float* sf, const float* sb, const float* du,
                                    float* parts, void* dx, void* dz, hipStream_t st);
// The producer Conv1D written out (conv_seq.hip), for masked layers (along
// the kept tokens), layers with the post-SSM LayerNorm and unpooled layers:
// x_conv of the layer's sequence into xc (x's layout and element type); and
// its adjoint in place -- dx holds dL/dx_conv on entry and dL/dx on exit --
// with `floats` of scratch, the conv's weight and bias gradients into dcw,
// dcb.  conv_adjoint_fits: the scratch is large enough.
// fg (dense layers with the post-SSM LayerNorm): dx holds the norm's g, not
// dL/dx_conv, and the adjoint forms dL/dx_conv = g (D_fwd + D_bwd) + du[b,
// t] inv_p where it reads it (the norm's second pass folded in).
struct DxcFromG {
    const float* du;  // (B, T, E)
    const float *Df, *Db;
    int64_t T;
    float inv_p;
};
hipError_t launch_conv_seq(const Geom& g, const void* x, const fastvim_params& p, void* xc, hipStream_t st);
hipError_t launch_conv_adjoint(const Geom& g, const void* x, void* dx, const fastvim_params& p, float* scratch,
                               int64_t floats, float* dcw, float* dcb, hipStream_t st,
                               const DxcFromG* fg = nullptr);
bool conv_adjoint_fits(const Geom& g, int64_t floats);

hipError_t launch_bwd_norm_pass1(const Geom& g, const void* x, const void* z, const void* dout,
                                 const fastvim_params& p, const BwdWorkspace& ws, void* dx, void* dz,
                                 hipStream_t st);
hipError_t launch_bwd_norm_pass2(const Geom& g, const fastvim_params& p, const BwdWorkspace& ws, void* dx,
                                 void* dz, hipStream_t st);

}  // namespace fastvim
