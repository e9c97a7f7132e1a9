// Host side of the C ABI: argument validation, workspace layout, stage
// dispatch and intermediate-result export.  Every check runs on the host
// before anything is enqueued, so an argument error launches nothing.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "bwd_internal.h"

namespace fastvim {
namespace {

constexpr int64_t kMaxE = 4096;
constexpr int64_t kMaxR = 64;
constexpr int64_t kMaskedMaxCells = 16384;  // per-image occurrence counters live in 64 KB of LDS
constexpr int64_t kMaxElems = int64_t(1) << 60;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool mul_ok(int64_t a, int64_t b, int64_t* r) {
    if (a != 0 && b > kMaxElems / a) return false;
    *r = a * b;
    return true;
}

// Sizes only (no pointers): fills g.  Returns FASTVIM_OK or a status.
int resolve_geom(const fastvim_dims* d, int axis, Geom* g) {
    if (!d) return FASTVIM_ERR_NULL;
    if (axis < FASTVIM_POOL_COLS || axis > FASTVIM_POOL_NONE_COLMAJOR) return FASTVIM_ERR_ARG;
    if (d->io_dtype != FASTVIM_F32 && d->io_dtype != FASTVIM_BF16) return FASTVIM_ERR_ARG;
    if (d->B < 0 || d->h <= 0 || d->w <= 0 || d->E <= 0 || d->N <= 0 || d->R <= 0 || d->K < 0)
        return FASTVIM_ERR_DIMS;
    const bool masked = d->K > 0;
    const bool pooled = axis == FASTVIM_POOL_COLS || axis == FASTVIM_POOL_ROWS;
    int64_t hw, tmp;
    if (!mul_ok(d->h, d->w, &hw)) return FASTVIM_ERR_DIMS;
    if (masked && (!pooled || d->K > hw)) return FASTVIM_ERR_DIMS;
    if (d->N != 16 || d->R > kMaxR || d->E > kMaxE) return FASTVIM_ERR_UNSUPPORTED;
    if (d->E % (d->io_dtype == FASTVIM_F32 ? 4 : 8) != 0) return FASTVIM_ERR_UNSUPPORTED;
    if (masked && hw > kMaskedMaxCells) return FASTVIM_ERR_UNSUPPORTED;
    // kernels address within an image with 32-bit offsets
    if (!mul_ok(hw, d->E, &tmp) || tmp > INT32_MAX) return FASTVIM_ERR_UNSUPPORTED;
    const int64_t tokens = masked ? d->K : hw;
    if (!mul_ok(d->B, tokens, &tmp) || !mul_ok(tmp, d->E, &tmp)) return FASTVIM_ERR_DIMS;
    g->B = d->B; g->h = d->h; g->w = d->w; g->E = d->E; g->N = d->N; g->R = d->R; g->K = d->K;
    g->axis = axis;
    g->masked = masked;
    g->pooled = pooled;
    g->io = d->io_dtype;
    g->NX = d->R + 2 * d->N;
    if (axis == FASTVIM_POOL_COLS) { g->T = d->h; g->P = d->w; }
    else if (axis == FASTVIM_POOL_ROWS) { g->T = d->w; g->P = d->h; }
    else { g->T = hw; g->P = 1; }
    return FASTVIM_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return a && b && na && nb && pa < pb + nb && pb < pa + na;
}

// Bytes of x (and of z, out, dout, dx, dz) of a call.
size_t io_span(const Geom& g) {
    return (size_t)(g.B * (g.masked ? g.K : g.h * g.w) * g.E) * (g.io == FASTVIM_F32 ? 4 : 2);
}

// x_proj_w is read with 16-byte vector loads, the others with scalar loads.
int check_dir(const fastvim_dir_params& d) {
    const float* ps[5] = {d.x_proj_w, d.dt_proj_w, d.dt_proj_b, d.A_log, d.D};
    for (const float* p : ps)
        if (!p) return FASTVIM_ERR_NULL;
    for (const float* p : ps)
        if (!aligned(p, p == d.x_proj_w ? 16 : 4)) return FASTVIM_ERR_ALIGN;
    return FASTVIM_OK;
}

// The parameters the kernels see.  With FASTVIM_FLAG_LOCAL_BWD the backward
// slot carries the forward direction's projection, step size and decay (the
// local backward scan shares them) and the caller's backward D.
fastvim_params effective_params(const fastvim_params& p) {
    fastvim_params q = p;
    if (p.flags & FASTVIM_FLAG_LOCAL_BWD) {
        q.bwd.x_proj_w = p.fwd.x_proj_w;
        q.bwd.dt_proj_w = p.fwd.dt_proj_w;
        q.bwd.dt_proj_b = p.fwd.dt_proj_b;
        q.bwd.A_log = p.fwd.A_log;
    }
    return q;
}

// With FASTVIM_FLAG_CONV, the layers whose stages cannot slide the conv
// window where they read x get x_conv written out first (conv_seq.hip):
// masked layers (the conv runs along the kept tokens), layers with the
// post-SSM LayerNorm and unpooled layers.  Dense pooled layers without the
// norm compute it in their pool and output stages (conv.hip); the forward
// pass's single launch computes it on load for dense layers, with or without
// the norm (fused.hip; run_fwd asks it first), and so does the backward pass
// of dense layers with the norm (conv_written_bwd).
bool conv_written(const Geom& g, uint32_t flags) {
    return (flags & FASTVIM_FLAG_CONV) && (g.masked || !g.pooled || (flags & FASTVIM_FLAG_POST_NORM));
}

// Scratch of the written-out conv's adjoint: the backward workspace past its
// header, free once the layer's own backward pass has run.
constexpr size_t kBwdHeaderBytes = 256;

// FASTVIM_FLAG_POOL_SCALE: a finite factor, pooled layers only, into g.
int apply_pool_scale(const fastvim_params& p, Geom* g) {
    if (!(p.flags & FASTVIM_FLAG_POOL_SCALE)) return FASTVIM_OK;
    if (!g->pooled || !std::isfinite(p.pool_scale)) return FASTVIM_ERR_ARG;
    g->pool_scale = p.pool_scale;
    return FASTVIM_OK;
}

// Flags and tuning word of a call.
int check_flags(const fastvim_params& p) {
    const uint32_t paths = FASTVIM_FLAG_STAGED | FASTVIM_FLAG_FUSED;
    const uint32_t options = FASTVIM_FLAG_POST_NORM | FASTVIM_FLAG_CONV | FASTVIM_FLAG_LOCAL_BWD |
                             FASTVIM_FLAG_POOL_SCALE | FASTVIM_FLAG_CHECK_IDX;
    if ((p.flags & ~(paths | options)) || (p.flags & paths) == paths) return FASTVIM_ERR_ARG;
    if (p.tuning & ~(FASTVIM_TUNING_LS(0xff) | FASTVIM_TUNING_LE(0xff) | FASTVIM_TUNING_POLL1 |
                     FASTVIM_TUNING_BWD_GROUPS(0x3f) | FASTVIM_TUNING_SCAN_OUT(3)))
        return FASTVIM_ERR_ARG;
    if (((p.tuning >> 26) & 3u) == 3u) return FASTVIM_ERR_ARG;
    return FASTVIM_OK;
}

// Validation of a layer call's arguments other than the workspace.  *empty is
// set for B == 0.
int validate(const void* x, const void* z, const fastvim_params* prm, const fastvim_dims* d, int axis,
             const int32_t* idx, const void* out, Geom* g, bool* empty) {
    if (!prm) return FASTVIM_ERR_NULL;
    int st = check_flags(*prm);
    if (st) return st;
    if ((st = resolve_geom(d, axis, g))) return st;
    g->tuning = prm->tuning;
    if ((st = apply_pool_scale(*prm, g))) return st;
    if (!g->masked && idx) return FASTVIM_ERR_ARG;
    if (prm->saved_u && !g->pooled) return FASTVIM_ERR_ARG;
    *empty = g->B == 0;
    if (*empty) return FASTVIM_OK;
    if (!x || !z || !out || (g->masked && !idx)) return FASTVIM_ERR_NULL;
    const fastvim_params eff = effective_params(*prm);
    if ((st = check_dir(eff.fwd)) || (st = check_dir(eff.bwd))) return st;
    if (prm->flags & FASTVIM_FLAG_POST_NORM) {
        if (!prm->ln_weight || !prm->ln_bias) return FASTVIM_ERR_NULL;
        if (!aligned(prm->ln_weight, 16) || !aligned(prm->ln_bias, 16)) return FASTVIM_ERR_ALIGN;
        if (!(prm->ln_eps > 0.f) || !(prm->ln_eps < 3.4e38f)) return FASTVIM_ERR_ARG;
    }
    if (prm->flags & FASTVIM_FLAG_CONV) {
        if (!prm->conv_w || !prm->conv_b) return FASTVIM_ERR_NULL;
        if (!aligned(prm->conv_w, 16) || !aligned(prm->conv_b, 4)) return FASTVIM_ERR_ALIGN;
    }
    if (!aligned(x, 16) || !aligned(z, 16) || !aligned(out, 16) || (idx && !aligned(idx, 4)))
        return FASTVIM_ERR_ALIGN;
    const size_t io_bytes = io_span(*g);
    if (overlap(out, io_bytes, x, io_bytes) || overlap(out, io_bytes, z, io_bytes)) return FASTVIM_ERR_OVERLAP;
    if (prm->saved_u) {
        const void* su = prm->saved_u;
        const size_t ub = (size_t)(g->B * g->T * g->E) * sizeof(float);
        if (!aligned(su, 16)) return FASTVIM_ERR_ALIGN;
        if (overlap(su, ub, x, io_bytes) || overlap(su, ub, z, io_bytes) || overlap(su, ub, out, io_bytes))
            return FASTVIM_ERR_OVERLAP;
    }
    return FASTVIM_OK;
}

// The caller's workspace of a validated layer call: present, aligned, large
// enough and clear of x, z, out and saved_u.  Lays it out into *ws.
int bind_workspace(const Geom& g, const void* x, const void* z, const fastvim_params& prm, const void* out,
                   Workspace* ws) {
    if (!prm.workspace) return FASTVIM_ERR_WORKSPACE;
    if (!aligned(prm.workspace, 256)) return FASTVIM_ERR_ALIGN;
    const size_t need = workspace_layout(g, nullptr, nullptr);
    if (prm.workspace_bytes < need) return FASTVIM_ERR_WORKSPACE;
    const size_t io_bytes = io_span(g);
    const void* w = prm.workspace;
    if (overlap(w, need, x, io_bytes) || overlap(w, need, z, io_bytes) || overlap(w, need, out, io_bytes) ||
        overlap(w, need, prm.saved_u, prm.saved_u ? (size_t)(g.B * g.T * g.E) * sizeof(float) : 0))
        return FASTVIM_ERR_OVERLAP;
    workspace_layout(g, prm.workspace, ws);
    if (prm.saved_u) ws->u = prm.saved_u;
    return FASTVIM_OK;
}

// Scratch of a call made with a NULL workspace, from the stream-ordered
// allocator: taken on the call's stream before its kernels are enqueued and
// given back on it after them, so it is never held between calls.
struct StreamScratch {
    void* raw = nullptr;
    hipStream_t s = nullptr;
    // bytes, 256-byte aligned, into *base
    int take(size_t bytes, hipStream_t st, void** base) {
        s = st;
        if (hipMallocAsync(&raw, bytes + 256, st) != hipSuccess) {
            raw = nullptr;
            (void)hipGetLastError();
            return FASTVIM_ERR_HIP;
        }
        *base = reinterpret_cast<void*>((reinterpret_cast<uintptr_t>(raw) + 255) & ~uintptr_t(255));
        return FASTVIM_OK;
    }
    // Enqueues the free; folds a failure into st.
    int give_back(int st) {
        if (raw && hipFreeAsync(raw, s) != hipSuccess && st == FASTVIM_OK) st = FASTVIM_ERR_HIP;
        raw = nullptr;
        return st;
    }
};

int run_stage(int stage, const Geom& g, const void* x, const void* z, const fastvim_params& p,
              const int32_t* idx, void* out, const Workspace& ws, hipStream_t st) {
    hipError_t e = hipSuccess;
    switch (stage) {
        case FASTVIM_STAGE_ROWS:
            if (g.masked)
                e = launch_mask_rows(g, idx, ws, (p.flags & FASTVIM_FLAG_CHECK_IDX) ? ws.sync + 1 : nullptr, st);
            break;
        case FASTVIM_STAGE_POOL:
            if (g.pooled)
                e = (p.flags & FASTVIM_FLAG_CONV) ? launch_conv_pool(g, x, p, ws, st) : launch_pool(g, x, ws, st);
            break;
        case FASTVIM_STAGE_PROJ: e = launch_proj(g, x, p, ws, st); break;
        case FASTVIM_STAGE_SCAN: e = launch_scan(g, x, p, ws, st); break;
        case FASTVIM_STAGE_EPILOGUE:
            e = (p.flags & FASTVIM_FLAG_POST_NORM) ? launch_epilogue_norm(g, x, z, p, ws, out, st)
                : (p.flags & FASTVIM_FLAG_CONV)    ? launch_conv_epilogue(g, x, z, p, ws, out, st)
                                                   : launch_epilogue(g, x, z, p, ws, out, st);
            break;
        default: return FASTVIM_ERR_ARG;
    }
    return e == hipSuccess ? FASTVIM_OK : FASTVIM_ERR_HIP;
}

size_t export_bytes(const Geom& g, int what) {
    switch (what) {
        case FASTVIM_EXPORT_U: return g.pooled ? (size_t)(g.B * g.T * g.E) * 4 : 0;
        case FASTVIM_EXPORT_XDBL: return (size_t)(g.B * g.T * 2 * g.NX) * 4;
        case FASTVIM_EXPORT_S_FWD:
        case FASTVIM_EXPORT_S_BWD: return (size_t)(g.B * g.T * g.E) * 4;
        case FASTVIM_EXPORT_ROWS: return g.masked ? (size_t)(g.B * g.K) * 4 : 0;
        case FASTVIM_EXPORT_BAD_TOKENS: return g.masked ? (size_t)g.B * 4 : 0;
        case FASTVIM_EXPORT_STATUS: return 4;
        default: return 0;
    }
}

// The backward pass covers the pooled layer (dense or masked), with scans of
// at most bwd_tmax(R) steps; with the post-SSM norm, E <= 2048 (bwd_norm.hip).
bool bwd_supported(const Geom& g) { return g.pooled && g.T <= bwd_tmax(g.R); }

int bwd_nchk(const Geom& g) {
    const int64_t n = (g.T + 15) / 16;
    return (int)(n > kBwdCkptMin ? n : kBwdCkptMin);
}

struct Span {
    const void* p;
    size_t n;
};

size_t bwd_total_bytes(const Geom& g);

// Full validation of a backward call.  *empty is set for B == 0.  A NULL
// workspace passes (the call then takes its own stream-ordered scratch);
// a caller's workspace is checked for alignment, size and overlap.
int validate_bwd(const void* x, const void* z, const void* dout, const fastvim_params* prm, const fastvim_dims* d,
                 int axis, const int32_t* idx, const void* dx, const void* dz, const fastvim_grads* gr, Geom* g,
                 bool* empty) {
    if (!prm) return FASTVIM_ERR_NULL;
    const uint32_t unsupported = FASTVIM_FLAG_FUSED;
    const uint32_t options = FASTVIM_FLAG_STAGED | FASTVIM_FLAG_POST_NORM | FASTVIM_FLAG_POOL_SCALE |
                             FASTVIM_FLAG_LOCAL_BWD | FASTVIM_FLAG_CONV | FASTVIM_FLAG_CHECK_IDX;
    if (prm->flags & ~(options | unsupported)) return FASTVIM_ERR_ARG;
    // the backward pass has no single launch to tune: only its image groups
    if (prm->tuning & ~FASTVIM_TUNING_BWD_GROUPS(0x3f)) return FASTVIM_ERR_ARG;
    if (((prm->tuning >> 20) & 0x3fu) > 32) return FASTVIM_ERR_ARG;
    if (prm->flags & unsupported) return FASTVIM_ERR_UNSUPPORTED;
    const bool norm = (prm->flags & FASTVIM_FLAG_POST_NORM) != 0;
    const bool conv = (prm->flags & FASTVIM_FLAG_CONV) != 0;
    int st = resolve_geom(d, axis, g);
    if (st) return st;
    g->tuning = prm->tuning;
    if ((st = apply_pool_scale(*prm, g))) return st;
    if (!bwd_supported(*g) || (norm && !bwd_norm_supported(*g))) return FASTVIM_ERR_UNSUPPORTED;
    if (conv && (g->masked || norm) &&
        !conv_adjoint_fits(*g, (int64_t)((bwd_total_bytes(*g) - kBwdHeaderBytes) / 4)))
        return FASTVIM_ERR_UNSUPPORTED;
    if (!g->masked && idx) return FASTVIM_ERR_ARG;
    if (!gr) return FASTVIM_ERR_NULL;
    if (conv) {
        if (!prm->conv_w || !prm->conv_b || !gr->conv_w || !gr->conv_b) return FASTVIM_ERR_NULL;
        if (!aligned(prm->conv_w, 16) || !aligned(prm->conv_b, 4) || !aligned(gr->conv_w, 4) ||
            !aligned(gr->conv_b, 4))
            return FASTVIM_ERR_ALIGN;
    }
    if (norm) {
        if (!prm->ln_weight || !prm->ln_bias || !gr->ln_weight || !gr->ln_bias) return FASTVIM_ERR_NULL;
        if (!aligned(prm->ln_weight, 16) || !aligned(prm->ln_bias, 16) || !aligned(gr->ln_weight, 4) ||
            !aligned(gr->ln_bias, 4))
            return FASTVIM_ERR_ALIGN;
        if (!(prm->ln_eps > 0.f) || !(prm->ln_eps < 3.4e38f)) return FASTVIM_ERR_ARG;
    }
    const fastvim_dir_grads* gd[2] = {&gr->fwd, &gr->bwd};
    const size_t gsz[5] = {(size_t)(g->NX * g->E), (size_t)(g->E * g->R), (size_t)g->E, (size_t)(g->E * g->N),
                           (size_t)g->E};
    Span gs[14];
    for (int k = 0; k < 2; ++k) {
        const float* ps[5] = {gd[k]->x_proj_w, gd[k]->dt_proj_w, gd[k]->dt_proj_b, gd[k]->A_log, gd[k]->D};
        for (int i = 0; i < 5; ++i) {
            if (!ps[i]) return FASTVIM_ERR_NULL;
            if (!aligned(ps[i], 4)) return FASTVIM_ERR_ALIGN;
            gs[5 * k + i] = Span{ps[i], gsz[i] * sizeof(float)};
        }
    }
    int ngs = 10;
    if (norm) {
        gs[ngs++] = Span{gr->ln_weight, (size_t)g->E * sizeof(float)};
        gs[ngs++] = Span{gr->ln_bias, (size_t)g->E * sizeof(float)};
    }
    if (conv) {
        gs[ngs++] = Span{gr->conv_w, (size_t)(g->E * FASTVIM_CONV_TAPS) * sizeof(float)};
        gs[ngs++] = Span{gr->conv_b, (size_t)g->E * sizeof(float)};
    }
    for (int i = 0; i < ngs; ++i)
        for (int j = i + 1; j < ngs; ++j)
            if (overlap(gs[i].p, gs[i].n, gs[j].p, gs[j].n)) return FASTVIM_ERR_OVERLAP;
    *empty = g->B == 0;
    if (*empty) return FASTVIM_OK;
    if (!x || !z || !dout || !dx || !dz || (g->masked && !idx)) return FASTVIM_ERR_NULL;
    const fastvim_params eff = effective_params(*prm);
    if ((st = check_dir(eff.fwd)) || (st = check_dir(eff.bwd))) return st;
    if (!aligned(x, 16) || !aligned(z, 16) || !aligned(dout, 16) || !aligned(dx, 16) || !aligned(dz, 16) ||
        (idx && !aligned(idx, 4)))
        return FASTVIM_ERR_ALIGN;
    const size_t need = bwd_total_bytes(*g);
    if (prm->workspace) {
        if (!aligned(prm->workspace, 256)) return FASTVIM_ERR_ALIGN;
        if (prm->workspace_bytes < need) return FASTVIM_ERR_WORKSPACE;
    }
    const size_t io = io_span(*g);
    // outputs (dx, dz, the workspace and every gradient) overlap neither each
    // other nor an input; parameters count as inputs
    Span ins[18] = {{x, io}, {z, io}, {dout, io}};
    int nin = 3;
    for (const fastvim_dir_params* pd : {&eff.fwd, &eff.bwd}) {
        const float* ps[5] = {pd->x_proj_w, pd->dt_proj_w, pd->dt_proj_b, pd->A_log, pd->D};
        for (int i = 0; i < 5; ++i) ins[nin++] = Span{ps[i], gsz[i] * sizeof(float)};
    }
    if (prm->saved_u && !aligned(prm->saved_u, 16)) return FASTVIM_ERR_ALIGN;
    ins[nin++] = Span{prm->saved_u, prm->saved_u ? (size_t)(g->B * g->T * g->E) * sizeof(float) : 0};
    if (norm) {
        ins[nin++] = Span{prm->ln_weight, (size_t)g->E * sizeof(float)};
        ins[nin++] = Span{prm->ln_bias, (size_t)g->E * sizeof(float)};
    }
    if (conv) {
        ins[nin++] = Span{prm->conv_w, (size_t)(g->E * FASTVIM_CONV_TAPS) * sizeof(float)};
        ins[nin++] = Span{prm->conv_b, (size_t)g->E * sizeof(float)};
    }
    Span outs[17] = {{dx, io}, {dz, io}, {prm->workspace, need}};
    const int nout = 3 + ngs;
    for (int i = 0; i < ngs; ++i) outs[3 + i] = gs[i];
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return FASTVIM_ERR_OVERLAP;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return FASTVIM_ERR_OVERLAP;
    }
    return FASTVIM_OK;
}

// Lays out a backward workspace at base (the caller's or the call's own).
void bind_bwd_workspace(const Geom& g, const fastvim_params& prm, void* base, BwdWorkspace* ws) {
    bwd_workspace_layout(g, base, ws);
    if (prm.saved_u) {
        ws->fwd.u = prm.saved_u;
        ws->u_saved = true;
    }
}

// The three phases of a backward call over one group of images, on one
// stream.  front: the first pass over the grid (and what it needs: the mask
// rows; with the LayerNorm, the forward stages and the norm's own sums).
// mid: the scan adjoint, dv, du, d x_proj_w's partials and the parameter
// sums (gr).  back: the second pass, which writes dx and dz, and its sums.
int bwd_front(const Geom& g, const void* x, const void* z, const void* dout, const fastvim_params& p,
              const int32_t* idx, void* dx, void* dz, const fastvim_grads& gr, const BwdWorkspace& ws,
              hipStream_t s) {
    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t r) {
        if (e == hipSuccess) e = r;
        return e == hipSuccess;
    };
    const bool norm = (p.flags & FASTVIM_FLAG_POST_NORM) != 0;
    const bool local = (p.flags & FASTVIM_FLAG_LOCAL_BWD) != 0;  // p holds the effective parameters
    const bool conv = (p.flags & FASTVIM_FLAG_CONV) != 0;
    if (g.masked &&
        !ok(launch_mask_rows(g, idx, ws.fwd, (p.flags & FASTVIM_FLAG_CHECK_IDX) ? ws.fwd.sync + 1 : nullptr, s)))
        return FASTVIM_ERR_HIP;
    if (norm) {
        // the norm's adjoint needs y, hence both scans' outputs: recompute the
        // forward stages first, then the first pass with the norm, whose
        // per-(b, t) partials of dD, d ln_w and d ln_b (in du, du_f, du_b) are
        // summed before the scan adjoint overwrites those buffers
        // (with the conv, x is its input: the pool and the first pass compute
        // x_conv where they read x)
        if ((!ws.u_saved && !ok(conv ? launch_conv_pool(g, x, p, ws.fwd, s) : launch_pool(g, x, ws.fwd, s))) ||
            !ok(launch_proj(g, x, p, ws.fwd, s)) || !ok(launch_scan(g, x, p, ws.fwd, s)) ||
            !ok(launch_bwd_norm_pass1(g, x, z, dout, p, ws, dx, dz, s)))
            return FASTVIM_ERR_HIP;
        const int64_t M = g.B * g.T;
        if (!ok(launch_colsum(ws.du, M, g.E, g.E, gr.fwd.D, gr.bwd.D, ws.tmp, s)) ||
            !ok(launch_colsum(ws.du_f, M, g.E, g.E, gr.ln_weight, nullptr, ws.tmp, s)) ||
            !ok(launch_colsum(ws.du_b, M, g.E, g.E, gr.ln_bias, nullptr, ws.tmp, s)))
            return FASTVIM_ERR_HIP;
    } else if (conv) {
        // u pools the conv's output (unless saved); the first pass then sums g only
        BwdWorkspace wg = ws;
        wg.u_saved = true;
        if ((!ws.u_saved && !ok(launch_conv_pool(g, x, p, ws.fwd, s))) ||
            !ok(launch_bwd_pool(g, x, z, dout, wg, s)) || !ok(launch_proj(g, x, p, ws.fwd, s)))
            return FASTVIM_ERR_HIP;
        if (local && !ok(launch_scan(g, x, p, ws.fwd, s))) return FASTVIM_ERR_HIP;
    } else {
        if (!ok(launch_bwd_pool(g, x, z, dout, ws, s)) || !ok(launch_proj(g, x, p, ws.fwd, s)))
            return FASTVIM_ERR_HIP;
        // the local backward scan's outputs (the second pass needs s_bwd) come
        // from the forward scan; the scan adjoint does not rerun that scan
        if (local && !ok(launch_scan(g, x, p, ws.fwd, s))) return FASTVIM_ERR_HIP;
    }
    return FASTVIM_OK;
}

int bwd_mid(const Geom& g, const fastvim_params& p, const fastvim_grads& gr, const BwdWorkspace& ws,
            hipStream_t s) {
    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t r) {
        if (e == hipSuccess) e = r;
        return e == hipSuccess;
    };
    const bool local = (p.flags & FASTVIM_FLAG_LOCAL_BWD) != 0;
    BwdScanArgs a{ws.fwd.xdbl, ws.fwd.u, ws.gs, p.fwd, p.bwd, ws.fwd.s_f, ws.fwd.s_b, ws.du_f, ws.du_b, ws.dvp,
                  ws.ckpt, ws.dAp, ws.dWdtp, ws.dbp, g.B, g.T, g.E, (int)g.R, (int)g.NX, (int)ws.G, local, ws.nchk};
    if (!ok(launch_scan_bwd(a, s)) || !ok(launch_bwd_dv(g, ws, s)) || !ok(launch_bwd_du(g, p, ws, s)) ||
        !ok(launch_bwd_dwx(g, ws, s)))
        return FASTVIM_ERR_HIP;
    // parameter gradients: sums of per-chunk and per-image partials; those of
    // at most kColRowsPerBlock rows share one launch
    const fastvim_dir_grads* gd[2] = {&gr.fwd, &gr.bwd};
    const int64_t E = g.E, NX = g.NX, R = g.R, B = g.B;
    ColsumBatch batch{};
    if (local) {
        // the local scan's parameters are the forward direction's: its partials
        // join the forward sums below; the backward set's four are zero
        const fastvim_dir_grads& gb = gr.bwd;
        if (!ok(launch_fill_zero(gb.x_proj_w, NX * E, s)) || !ok(launch_fill_zero(gb.A_log, E * 16, s)) ||
            !ok(launch_fill_zero(gb.dt_proj_w, E * R, s)) || !ok(launch_fill_zero(gb.dt_proj_b, E, s)))
            return FASTVIM_ERR_HIP;
    }
    for (int d = 0; d < (local ? 1 : 2); ++d) {
        // with the local scan, direction 0's sums run over both directions'
        // partials (d x_proj_w: (MC, 2) rows; the others: (2, B) rows)
        const int64_t k = local ? 2 : 1;
        const ColsumSeg segs[4] = {
            {ws.dWxp + d * NX * E, k * ws.MC, NX * E, (local ? 1 : 2) * NX * E, gd[d]->x_proj_w, nullptr, 0},
            {ws.dAp + d * B * E * 16, k * B, E * 16, E * 16, gd[d]->A_log, nullptr, 0},
            {ws.dWdtp + d * B * E * R, k * B, E * R, E * R, gd[d]->dt_proj_w, nullptr, 0},
            {ws.dbp + d * B * E, k * B, E, E, gd[d]->dt_proj_b, nullptr, 0}};
        for (const ColsumSeg& sg : segs) {
            if (sg.rows <= kColRowsPerBlock) {
                batch.seg[batch.n++] = sg;
            } else if (!ok(launch_colsum(sg.in, sg.rows, sg.cols, sg.ld, sg.out, nullptr, ws.tmp, s))) {
                return FASTVIM_ERR_HIP;
            }
        }
    }
    return ok(launch_colsum_batch(batch, s)) ? FASTVIM_OK : FASTVIM_ERR_HIP;
}

int bwd_back(const Geom& g, const void* x, const void* z, const void* dout, const fastvim_params& p, void* dx,
             void* dz, const fastvim_grads& gr, const BwdWorkspace& ws, hipStream_t s) {
    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t r) {
        if (e == hipSuccess) e = r;
        return e == hipSuccess;
    };
    const int64_t E = g.E;
    if ((p.flags & FASTVIM_FLAG_POST_NORM) && (p.flags & FASTVIM_FLAG_CONV)) {
        // (x is the conv's input) dx holds the norm's g; the conv's adjoint
        // forms dL/dx_conv = g (D_fwd + D_bwd) + du / P where it reads it, its
        // scratch the regions before du
        const DxcFromG fg{ws.du, p.fwd.D, p.bwd.D, g.T, pool_norm(g)};
        return ok(launch_conv_adjoint(g, x, dx, p, ws.front, ws.du - ws.front, gr.conv_w, gr.conv_b, s, &fg))
                   ? FASTVIM_OK
                   : FASTVIM_ERR_HIP;
    }
    if (p.flags & FASTVIM_FLAG_POST_NORM)
        return ok(launch_bwd_norm_pass2(g, p, ws, dx, dz, s)) ? FASTVIM_OK : FASTVIM_ERR_HIP;
    if (p.flags & FASTVIM_FLAG_CONV) {
        // second pass through the conv; its partial rows go to the checkpoint
        // region (free once the scan adjoint has run; large enough: see
        // bwd_workspace_layout)
        const int64_t np = bwd_conv_parts(g);
        const int64_t ckpt_floats = 2 * g.B * ws.G * ws.nchk * 256 * 4;
        if (np * 6 * E > ckpt_floats) return FASTVIM_ERR_WORKSPACE;  // cannot happen with the sizes above
        if (!ok(launch_bwd_conv_epilogue(g, x, z, dout, p, ws.fwd.s_f, ws.fwd.s_b, ws.du, ws.ckpt, dx, dz, s)) ||
            !ok(launch_colsum(ws.ckpt, np, E, 6 * E, gr.fwd.D, gr.bwd.D, ws.tmp, s)) ||
            !ok(launch_colsum(ws.ckpt + E, np, E, 6 * E, gr.conv_b, nullptr, ws.tmp, s)) ||
            !ok(launch_colsum(ws.ckpt + 2 * E, np, 4 * E, 6 * E, gr.conv_w, nullptr, ws.tmp, s)))
            return FASTVIM_ERR_HIP;
        return FASTVIM_OK;
    }
    if (!ok(launch_bwd_epilogue(g, x, z, dout, p, ws, dx, dz, s))) return FASTVIM_ERR_HIP;
    if (!ok(launch_colsum(ws.dDp, bwd_dd_parts(g), E, E, gr.fwd.D, gr.bwd.D, ws.tmp, s))) return FASTVIM_ERR_HIP;
    return FASTVIM_OK;
}

// ---------------------------------------------------------------- image groups
// A large backward call runs as groups of images: the first passes of all
// groups, then the second passes, on the call's stream, while each group's
// mid phase runs on a second stream as soon as its first pass is done.  The
// mid phase (scan adjoint, projections' adjoints, parameter sums: latency
// bound, little HBM traffic) then hides under the streaming passes.  Each
// group has a backward workspace of its own and writes its parameter sums to
// a record of its own; the records are added in group order at the end, so
// results stay bitwise deterministic for a given grouping.

constexpr int kMaxBwdGroups = 32;

// Floats of one group's record of parameter sums: per direction x_proj_w,
// dt_proj_w, dt_proj_b, A_log, D; then ln_w, ln_b, conv_w, conv_b.
int64_t bwd_record_floats(const Geom& g) {
    const int64_t E = g.E;
    return 2 * (g.NX * E + E * g.R + E + E * 16 + E) + 2 * E + 4 * E + E;
}

// The record's layout as a fastvim_grads.
fastvim_grads bwd_record(const Geom& g, float* r) {
    const int64_t E = g.E;
    fastvim_grads gr{};
    fastvim_dir_grads* d[2] = {&gr.fwd, &gr.bwd};
    for (fastvim_dir_grads* dd : d) {
        dd->x_proj_w = r; r += g.NX * E;
        dd->dt_proj_w = r; r += E * g.R;
        dd->dt_proj_b = r; r += E;
        dd->A_log = r; r += E * 16;
        dd->D = r; r += E;
    }
    gr.ln_weight = r; r += E;
    gr.ln_bias = r; r += E;
    gr.conv_w = r; r += 4 * E;
    gr.conv_b = r;
    return gr;
}

// Images per group, and the group count, for k requested groups.
void bwd_group_shape(const Geom& g, int k, int64_t* per, int* n) {
    *per = (g.B + k - 1) / k;
    *n = (int)((g.B + *per - 1) / *per);
}

// Bytes of a workspace for k groups: a 256-byte header (the call's status
// word), one backward workspace per group sized for its largest group, then
// the groups' records.
size_t bwd_grouped_bytes(const Geom& g, int k) {
    int64_t per;
    int n;
    bwd_group_shape(g, k, &per, &n);
    Geom gp = g;
    gp.B = per;
    const size_t sub = align256(bwd_workspace_layout(gp, nullptr, nullptr));
    return kBwdHeaderBytes + (size_t)n * sub + align256((size_t)(n * bwd_record_floats(g)) * sizeof(float));
}

// Groups a call runs as: FASTVIM_TUNING_BWD_GROUPS when set (1: none), else,
// for batches of at least 16 images of at least 2^20 cells x channels
// (2048^2 FastVim-T has 6.3 M), the measured best at 2048^2, B = 128: 4
// groups (4.43 -> 4.13 ms with saved pooled tokens, 4.99 -> 4.66 ms
// pooling x again), 2 with the LayerNorm (whose first pass needs the
// forward scans, recomputed per group: 4.82 -> 4.64 ms) and none with the
// Conv1D on load (5.09 ms alone, 5.17 in 2 groups); else none.
int bwd_groups(const Geom& g, uint32_t flags) {
    const int set = (int)((g.tuning >> 20) & 0x3fu);
    int k = set ? set : 1;
    if (!set) {
        const int64_t cells = (g.masked ? g.K : g.h * g.w) * g.E;
        if (cells >= (int64_t(1) << 20) && g.B >= 16)
            k = (flags & FASTVIM_FLAG_POST_NORM) ? 2 : (flags & FASTVIM_FLAG_CONV) ? 1 : 4;
    }
    if (k > g.B) k = (int)g.B;
    return k < 1 ? 1 : k;
}

// Workspace bytes of a backward call: enough for its layer in one group and
// in every grouping the tuning word may ask for.
size_t bwd_total_bytes(const Geom& g) {
    size_t need = bwd_workspace_layout(g, nullptr, nullptr);
    for (int k = 2; k <= kMaxBwdGroups && k <= g.B; ++k) {
        const size_t b = bwd_grouped_bytes(g, k);
        if (b > need) need = b;
    }
    return need;
}

// The second stream of grouped calls on the stream's device: default
// priority, non-blocking, created on first use and kept until the process
// ends.  Calls on one device share it (their mid phases then queue).
int side_stream(hipStream_t s, hipStream_t* out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static hipStream_t tab[kMaxDevices] = {};
    int cur = -1, dev = -1;
    if (hipGetDevice(&cur) != hipSuccess) return FASTVIM_ERR_HIP;
    dev = cur;
    if (s && hipStreamGetDevice(s, &dev) != hipSuccess) return FASTVIM_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FASTVIM_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(mu);
    if (!tab[dev]) {
        if (dev != cur && hipSetDevice(dev) != hipSuccess) return FASTVIM_ERR_HIP;
        const hipError_t e = hipStreamCreateWithFlags(&tab[dev], hipStreamNonBlocking);
        if (dev != cur) (void)hipSetDevice(cur);
        if (e != hipSuccess) {
            tab[dev] = nullptr;
            return FASTVIM_ERR_HIP;
        }
    }
    *out = tab[dev];
    return FASTVIM_OK;
}

// Events of one grouped call, destroyed when it returns (HIP releases an
// event that is still pending once it completes).
struct CallEvents {
    hipEvent_t ev[2 * kMaxBwdGroups + 1] = {};
    int n = 0;
    int make(int count) {
        for (; n < count; ++n)
            if (hipEventCreateWithFlags(&ev[n], hipEventDisableTiming) != hipSuccess) return FASTVIM_ERR_HIP;
        return FASTVIM_OK;
    }
    ~CallEvents() {
        for (int i = 0; i < n; ++i) (void)hipEventDestroy(ev[i]);
    }
};

int run_bwd_grouped(const Geom& g, int k, const void* x, const void* z, const void* dout, const fastvim_params& p,
                    const int32_t* idx, void* dx, void* dz, const fastvim_grads& gr, void* base, hipStream_t s) {
    int64_t per;
    int n;
    bwd_group_shape(g, k, &per, &n);
    Geom gp = g;
    gp.B = per;
    const size_t sub = align256(bwd_workspace_layout(gp, nullptr, nullptr));
    char* c = static_cast<char*>(base);
    unsigned* header = reinterpret_cast<unsigned*>(c);
    float* records = reinterpret_cast<float*>(c + kBwdHeaderBytes + (size_t)n * sub);
    const int64_t rf = bwd_record_floats(g);
    const size_t img = io_span(g) / (size_t)g.B;  // bytes of one image of x (z, dout, dx, dz)
    const int64_t idx_img = g.masked ? g.K : 0;
    hipStream_t side = nullptr;
    int st = side_stream(s, &side);
    if (st) return st;
    CallEvents evs;
    if ((st = evs.make(2 * n + 1))) return st;
    hipEvent_t* front_done = evs.ev;
    hipEvent_t* mid_done = evs.ev + n;
    hipEvent_t start = evs.ev[2 * n];
    Workspace hdr{};
    hdr.sync = header;
    if (launch_zero_sync(hdr, kBwdStatusWords, s) != hipSuccess) return FASTVIM_ERR_HIP;
    // the side stream starts behind everything the caller queued before
    if (hipEventRecord(start, s) != hipSuccess || hipStreamWaitEvent(side, start, 0) != hipSuccess)
        return FASTVIM_ERR_HIP;
    struct Group {
        Geom g;
        BwdWorkspace ws;
        fastvim_grads rec;
        size_t off;
    } grp[kMaxBwdGroups];
    for (int i = 0; i < n; ++i) {
        Group& q = grp[i];
        q.g = g;
        q.g.B = (i + 1) * per <= g.B ? per : g.B - i * per;
        bwd_workspace_layout(q.g, c + kBwdHeaderBytes + (size_t)i * sub, &q.ws);
        q.ws.fwd.sync = header;  // one status word for the call
        if (p.saved_u) {
            q.ws.fwd.u = p.saved_u + (size_t)(i * per) * (size_t)(g.T * g.E);
            q.ws.u_saved = true;
        }
        q.rec = bwd_record(g, records + i * rf);
        q.off = (size_t)(i * per) * img;
    }
    auto at = [](const void* ptr, size_t off) { return static_cast<const char*>(ptr) + off; };
    auto atw = [](void* ptr, size_t off) { return static_cast<char*>(ptr) + off; };
    for (int i = 0; i < n; ++i) {
        const Group& q = grp[i];
        const int32_t* qi = g.masked ? idx + (size_t)(i * per) * (size_t)idx_img : nullptr;
        if ((st = bwd_front(q.g, at(x, q.off), at(z, q.off), at(dout, q.off), p, qi, atw(dx, q.off),
                            atw(dz, q.off), q.rec, q.ws, s)))
            return st;
        if (hipEventRecord(front_done[i], s) != hipSuccess || hipStreamWaitEvent(side, front_done[i], 0) != hipSuccess)
            return FASTVIM_ERR_HIP;
        if ((st = bwd_mid(q.g, p, q.rec, q.ws, side))) return st;
        if (hipEventRecord(mid_done[i], side) != hipSuccess) return FASTVIM_ERR_HIP;
    }
    for (int i = 0; i < n; ++i) {
        const Group& q = grp[i];
        if (hipStreamWaitEvent(s, mid_done[i], 0) != hipSuccess) return FASTVIM_ERR_HIP;
        if ((st = bwd_back(q.g, at(x, q.off), at(z, q.off), at(dout, q.off), p, atw(dx, q.off), atw(dz, q.off),
                           q.rec, q.ws, s)))
            return st;
    }
    // the groups' records, added in group order into the caller's gradients
    const fastvim_grads r0 = bwd_record(g, records);
    const int64_t E = g.E;
    ColsumBatch b1{}, b2{};
    const fastvim_dir_grads* rd[2] = {&r0.fwd, &r0.bwd};
    const fastvim_dir_grads* od[2] = {&gr.fwd, &gr.bwd};
    for (int d = 0; d < 2; ++d) {
        b1.seg[b1.n++] = ColsumSeg{rd[d]->x_proj_w, n, g.NX * E, rf, od[d]->x_proj_w, nullptr, 0};
        b1.seg[b1.n++] = ColsumSeg{rd[d]->dt_proj_w, n, E * g.R, rf, od[d]->dt_proj_w, nullptr, 0};
        b1.seg[b1.n++] = ColsumSeg{rd[d]->dt_proj_b, n, E, rf, od[d]->dt_proj_b, nullptr, 0};
        b1.seg[b1.n++] = ColsumSeg{rd[d]->A_log, n, E * 16, rf, od[d]->A_log, nullptr, 0};
    }
    b2.seg[b2.n++] = ColsumSeg{r0.fwd.D, n, E, rf, gr.fwd.D, gr.bwd.D, 0};
    if (p.flags & FASTVIM_FLAG_POST_NORM) {
        b2.seg[b2.n++] = ColsumSeg{r0.ln_weight, n, E, rf, gr.ln_weight, nullptr, 0};
        b2.seg[b2.n++] = ColsumSeg{r0.ln_bias, n, E, rf, gr.ln_bias, nullptr, 0};
    }
    if (p.flags & FASTVIM_FLAG_CONV) {
        b2.seg[b2.n++] = ColsumSeg{r0.conv_w, n, 4 * E, rf, gr.conv_w, nullptr, 0};
        b2.seg[b2.n++] = ColsumSeg{r0.conv_b, n, E, rf, gr.conv_b, nullptr, 0};
    }
    if (launch_colsum_batch(b1, s) != hipSuccess || launch_colsum_batch(b2, s) != hipSuccess)
        return FASTVIM_ERR_HIP;
    return FASTVIM_OK;
}

// Whether the conv's adjoint fits in the regions before du of every image
// group's workspace (bwd_back's scratch when it replaces the norm's second
// pass).
bool conv_adjoint_fits_front(const Geom& g, uint32_t flags) {
    int64_t per;
    int n;
    bwd_group_shape(g, bwd_groups(g, flags), &per, &n);
    for (const int64_t b : {per, g.B - (n - 1) * per}) {
        Geom gp = g;
        gp.B = b;
        int64_t front = 0;
        bwd_workspace_layout(gp, nullptr, nullptr, &front);
        if (!conv_adjoint_fits(gp, front)) return false;
    }
    return true;
}

// Whether a backward call writes x_conv out first (conv_written).  A dense
// pooled layer with the LayerNorm computes x_conv where its first pass reads
// x, and its conv's adjoint replaces the norm's second pass (bwd_back) when
// the adjoint fits beside du; tiny layers write it out.
bool conv_written_bwd(const Geom& g, uint32_t flags) {
    if (!conv_written(g, flags)) return false;
    return g.masked || !g.pooled || !conv_adjoint_fits_front(g, flags);
}

// A backward call on its workspace at base (bwd_total_bytes(g) bytes).
int run_bwd(const Geom& g, const void* x, const void* z, const void* dout, const fastvim_params& p,
            const int32_t* idx, void* dx, void* dz, const fastvim_grads& gr, void* base, hipStream_t s) {
    if (conv_written_bwd(g, p.flags)) {
        // x_conv into dz (the passes below read each cell's x before they
        // write its dz), the layer's backward pass on it, which leaves
        // dL/dx_conv in dx, then the conv's adjoint in place on dx, its scratch
        // the workspace the layer's pass no longer needs
        fastvim_params q = p;
        q.flags &= ~FASTVIM_FLAG_CONV;
        if (launch_conv_seq(g, x, p, dz, s) != hipSuccess) return FASTVIM_ERR_HIP;
        const int st = run_bwd(g, dz, z, dout, q, idx, dx, dz, gr, base, s);
        if (st) return st;
        float* scratch = reinterpret_cast<float*>(static_cast<char*>(base) + kBwdHeaderBytes);
        const int64_t floats = (int64_t)((bwd_total_bytes(g) - kBwdHeaderBytes) / 4);
        return launch_conv_adjoint(g, x, dx, p, scratch, floats, gr.conv_w, gr.conv_b, s) == hipSuccess
                   ? FASTVIM_OK
                   : FASTVIM_ERR_HIP;
    }
    const int k = bwd_groups(g, p.flags);
    if (k > 1) return run_bwd_grouped(g, k, x, z, dout, p, idx, dx, dz, gr, base, s);
    BwdWorkspace ws;
    bind_bwd_workspace(g, p, base, &ws);
    if (launch_zero_sync(ws.fwd, kBwdStatusWords, s) != hipSuccess) return FASTVIM_ERR_HIP;
    int st = bwd_front(g, x, z, dout, p, idx, dx, dz, gr, ws, s);
    if (!st) st = bwd_mid(g, p, gr, ws, s);
    if (!st) st = bwd_back(g, x, z, dout, p, dx, dz, gr, ws, s);
    return st;
}

// Destinations of fastvim_ssm_fwd_stages (each NULL to skip).
struct StageDst {
    float* u;
    float* s_f;
    float* s_b;
    int32_t* rows;
};

// The stage destinations of a validated call: present only where the layer
// has them, 4-byte aligned, clear of x, z, out, saved_u and each other.
int check_stage_dst(const Geom& g, const StageDst& d, const void* x, const void* z, const void* out,
                    const fastvim_params& prm) {
    if ((d.u && !g.pooled) || (d.rows && !g.masked)) return FASTVIM_ERR_ARG;
    const size_t bte = (size_t)(g.B * g.T * g.E) * sizeof(float);
    const Span dsts[4] = {{d.u, bte}, {d.s_f, bte}, {d.s_b, bte}, {d.rows, (size_t)(g.B * g.K) * sizeof(int32_t)}};
    const size_t io = io_span(g);
    const Span others[4] = {{x, io}, {z, io}, {out, io}, {prm.saved_u, prm.saved_u ? bte : 0}};
    for (int i = 0; i < 4; ++i) {
        if (dsts[i].p && !aligned(dsts[i].p, 4)) return FASTVIM_ERR_ALIGN;
        for (const Span& o : others)
            if (overlap(dsts[i].p, dsts[i].n, o.p, o.n)) return FASTVIM_ERR_OVERLAP;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(dsts[i].p, dsts[i].n, dsts[j].p, dsts[j].n)) return FASTVIM_ERR_OVERLAP;
        if (prm.workspace && overlap(dsts[i].p, dsts[i].n, prm.workspace, workspace_layout(g, nullptr, nullptr)))
            return FASTVIM_ERR_OVERLAP;
    }
    return FASTVIM_OK;
}

// The scan and output stages as one launch (scan_out.hip), for the short
// pooled layers it supports: by the tuning word's bits 26-27, else for masked
// layers and images of at most 1024 tokens.
bool scan_out_chosen(const Geom& g, uint32_t flags) {
    if (!scan_out_supported(g, flags)) return false;
    const uint32_t set = (g.tuning >> 26) & 3u;
    if (set) return set == 2u;
    return g.masked || g.h * g.w <= 1024;
}

// The layer on a bound workspace: counters cleared, then the single launch or
// the stage kernels (the scan and output stages of short layers as one).
int run_fwd(const Geom& g, const void* x, const void* z, const fastvim_params& prm, const int32_t* idx, void* out,
            const Workspace& ws, hipStream_t s) {
    const bool norm = (prm.flags & FASTVIM_FLAG_POST_NORM) != 0;
    const bool local = (prm.flags & FASTVIM_FLAG_LOCAL_BWD) != 0;
    const bool conv = (prm.flags & FASTVIM_FLAG_CONV) != 0;
    // the single launch (with the Conv1D computed on load where it takes it:
    // dense COLS layers)
    const bool single = (prm.flags & FASTVIM_FLAG_FUSED)
                            ? fused_supported(g, norm, local, conv)
                            : !(prm.flags & FASTVIM_FLAG_STAGED) && fused_preferred(g, norm, local, conv);
    if (!single && conv_written(g, prm.flags)) {
        // x_conv into out, then the layer on it: every stage reads a cell's x
        // before the output stage writes that cell
        if (launch_conv_seq(g, x, prm, out, s) != hipSuccess) return FASTVIM_ERR_HIP;
        fastvim_params q = prm;
        q.flags &= ~FASTVIM_FLAG_CONV;
        return run_fwd(g, out, z, q, idx, out, ws, s);
    }
    if (launch_zero_sync(ws, sync_words(g), s) != hipSuccess) return FASTVIM_ERR_HIP;
    const fastvim_params q = effective_params(prm);
    if (single) return launch_fused(g, x, z, q, ws, out, s) == hipSuccess ? FASTVIM_OK : FASTVIM_ERR_HIP;
    const bool scan_out = scan_out_chosen(g, q.flags);
    // masked layers: mask rows and pooling as one launch where the layer fits it
    const bool mask_pool = !(q.flags & FASTVIM_FLAG_CONV) && mask_pool_supported(g);
    for (int stage = FASTVIM_STAGE_ROWS; stage <= FASTVIM_STAGE_EPILOGUE; ++stage) {
        if (mask_pool && stage == FASTVIM_STAGE_ROWS) {
            unsigned* status = (q.flags & FASTVIM_FLAG_CHECK_IDX) ? ws.sync + 1 : nullptr;
            if (launch_mask_pool(g, idx, x, ws, status, s) != hipSuccess) return FASTVIM_ERR_HIP;
            stage = FASTVIM_STAGE_POOL;  // done too
            continue;
        }
        if (scan_out && stage == FASTVIM_STAGE_SCAN)
            return launch_scan_out(g, x, z, q, ws, out, s) == hipSuccess ? FASTVIM_OK : FASTVIM_ERR_HIP;
        const int st = run_stage(stage, g, x, z, q, idx, out, ws, s);
        if (st) return st;
    }
    return FASTVIM_OK;
}

// fastvim_ssm_fwd and fastvim_ssm_fwd_stages (dst != NULL): validate, bind or
// take the workspace, run, copy the stages out, give the scratch back.
int fwd_entry(const void* x, const void* z, const fastvim_params* params, const fastvim_dims* dims, int axis,
              const int32_t* idx, void* out, hipStream_t s, const StageDst* dst) {
    Geom g;
    bool empty = false;
    int st = validate(x, z, params, dims, axis, idx, out, &g, &empty);
    if (st) return st;
    if (dst && (st = check_stage_dst(g, *dst, x, z, out, *params))) return st;
    if (empty) return FASTVIM_OK;
    Workspace ws;
    StreamScratch scratch;
    if (params->workspace) {
        if ((st = bind_workspace(g, x, z, *params, out, &ws))) return st;
    } else {
        void* base = nullptr;
        if ((st = scratch.take(workspace_layout(g, nullptr, nullptr), s, &base))) return st;
        workspace_layout(g, base, &ws);
        if (params->saved_u) ws.u = params->saved_u;
    }
    st = run_fwd(g, x, z, *params, idx, out, ws, s);
    if (st == FASTVIM_OK && dst) {
        const size_t bte = (size_t)(g.B * g.T * g.E) * sizeof(float);
        const struct {
            void* to;
            const void* from;
            size_t n;
        } copies[4] = {{dst->u, ws.u, bte}, {dst->s_f, ws.s_f, bte}, {dst->s_b, ws.s_b, bte},
                       {dst->rows, ws.rows, (size_t)(g.B * g.K) * sizeof(int32_t)}};
        for (const auto& c : copies)
            if (c.to && hipMemcpyAsync(c.to, c.from, c.n, hipMemcpyDeviceToDevice, s) != hipSuccess) {
                st = FASTVIM_ERR_HIP;
                break;
            }
    }
    return scratch.give_back(st);
}

}  // namespace

int fwd_on_scratch(const void* x, const void* z, const fastvim_params* params, const fastvim_dims* dims, int axis,
                   const int32_t* idx, void* out, hipStream_t s, int (*scratch)(void**), size_t cap) {
    Geom g;
    bool empty = false;
    int st = validate(x, z, params, dims, axis, idx, out, &g, &empty);
    if (st || empty) return st;
    if (workspace_layout(g, nullptr, nullptr) > cap) return FASTVIM_ERR_SCRATCH;
    void* base = nullptr;
    if ((st = scratch(&base))) return st;
    Workspace ws;
    workspace_layout(g, base, &ws);
    if (params->saved_u) ws.u = params->saved_u;
    return run_fwd(g, x, z, *params, idx, out, ws, s);
}

size_t workspace_layout(const Geom& g, void* base, Workspace* ws) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t bte = (size_t)(g.B * g.T * g.E) * sizeof(float);
    const size_t o_sync = take((size_t)sync_words(g) * sizeof(unsigned));  // first: the status word at byte 4
    const size_t o_u = g.pooled ? take(bte) : 0;
    const size_t o_x = take((size_t)(g.B * g.T * 2 * g.NX) * sizeof(float));
    const size_t o_sf = take(bte);
    const size_t o_sb = take(bte);
    const size_t o_rows = g.masked ? take((size_t)(g.B * g.K) * sizeof(int32_t)) : 0;
    const size_t o_bad = g.masked ? take((size_t)g.B * sizeof(int32_t)) : 0;
    if (base && ws) {
        char* c = static_cast<char*>(base);
        ws->u = g.pooled ? reinterpret_cast<float*>(c + o_u) : nullptr;
        ws->xdbl = reinterpret_cast<float*>(c + o_x);
        ws->s_f = reinterpret_cast<float*>(c + o_sf);
        ws->s_b = reinterpret_cast<float*>(c + o_sb);
        ws->rows = g.masked ? reinterpret_cast<int32_t*>(c + o_rows) : nullptr;
        ws->bad = g.masked ? reinterpret_cast<int32_t*>(c + o_bad) : nullptr;
        ws->sync = reinterpret_cast<unsigned*>(c + o_sync);
    }
    return off;
}

size_t bwd_workspace_layout(const Geom& g, void* base, BwdWorkspace* ws, int64_t* front_floats) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const int64_t B = g.B, T = g.T, E = g.E, NX = g.NX, R = g.R, M = g.B * g.T;
    const int64_t G = (E + kBwdCh - 1) / kBwdCh, S = bwd_rmax(R) + 32;
    const int64_t MC = (M + kBwdTokChunk - 1) / kBwdTokChunk;
    const size_t bte = (size_t)(M * E) * sizeof(float);
    const size_t o_hdr = take(kBwdStatusWords * sizeof(unsigned));  // first: the status word at byte 4
    const size_t o_u = take(bte);
    const size_t o_x = take((size_t)(M * 2 * NX) * sizeof(float));
    const size_t o_sf = take(bte), o_sb = take(bte);
    const size_t o_rows = g.masked ? take((size_t)(B * g.K) * sizeof(int32_t)) : 0;
    const size_t o_bad = g.masked ? take((size_t)B * sizeof(int32_t)) : 0;
    const int64_t ND = bwd_dd_parts(g);
    const size_t o_gs = take(bte), o_dDp = take((size_t)(ND * E) * sizeof(float));
    const size_t o_duf = take(bte), o_dub = take(bte), o_du = take(bte);
    const size_t o_dvp = take((size_t)(2 * B * G * T * S) * sizeof(float));
    const size_t o_ck = take((size_t)(2 * B * G * bwd_nchk(g) * 256 * 4) * sizeof(float));
    const size_t o_dv = take((size_t)(M * 2 * NX) * sizeof(float));
    const size_t o_dAp = take((size_t)(2 * B * E * 16) * sizeof(float));
    const size_t o_dWdtp = take((size_t)(2 * B * E * R) * sizeof(float));
    const size_t o_dbp = take((size_t)(2 * B * E) * sizeof(float));
    const size_t o_dWxp = take((size_t)(MC * 2 * NX * E) * sizeof(float));
    auto stage1 = [](int64_t rows, int64_t cols) {
        return rows > kColRowsPerBlock ? (rows + kColRowsPerBlock - 1) / kColRowsPerBlock * cols : int64_t(0);
    };
    int64_t tmpf = 1;
    // (the local backward scan sums twice the rows of the per-image and per-chunk partials)
    // (the Conv1D's second pass leaves bwd_conv_parts(g) rows of 6 E partials
    // in the checkpoint region, which holds at least 16384 B ceil(E / 64) >=
    // 256 B E floats against at most 32 B * 6 E)
    for (int64_t v : {stage1(ND, E), stage1(M, E), stage1(2 * B, E * 16), stage1(2 * B, E * R), stage1(2 * B, E),
                      stage1(2 * MC, NX * E), stage1(bwd_conv_parts(g), 4 * E)})
        tmpf = v > tmpf ? v : tmpf;
    const size_t o_tmp = take((size_t)tmpf * sizeof(float));
    if (front_floats) *front_floats = (int64_t)((o_du - o_u) / sizeof(float));
    if (base && ws) {
        char* c = static_cast<char*>(base);
        auto f = [&](size_t o) { return reinterpret_cast<float*>(c + o); };
        ws->fwd.u = f(o_u);
        ws->front = f(o_u);
        ws->fwd.xdbl = f(o_x);
        ws->fwd.s_f = f(o_sf);
        ws->fwd.s_b = f(o_sb);
        ws->fwd.rows = g.masked ? reinterpret_cast<int32_t*>(c + o_rows) : nullptr;
        ws->fwd.bad = g.masked ? reinterpret_cast<int32_t*>(c + o_bad) : nullptr;
        ws->fwd.sync = reinterpret_cast<unsigned*>(c + o_hdr);
        ws->gs = f(o_gs);
        ws->dDp = f(o_dDp);
        ws->du_f = f(o_duf);
        ws->du_b = f(o_dub);
        ws->du = f(o_du);
        ws->dvp = f(o_dvp);
        ws->ckpt = f(o_ck);
        ws->dv = f(o_dv);
        ws->dAp = f(o_dAp);
        ws->dWdtp = f(o_dWdtp);
        ws->dbp = f(o_dbp);
        ws->dWxp = f(o_dWxp);
        ws->tmp = f(o_tmp);
        ws->G = G;
        ws->S = S;
        ws->MC = MC;
        ws->tmp_floats = tmpf;
        ws->nchk = bwd_nchk(g);
        ws->u_saved = false;
    }
    return off;
}

}  // namespace fastvim

using namespace fastvim;

extern "C" {

size_t fastvim_ssm_workspace_bytes(const fastvim_dims* dims, int pool_axis) {
    Geom g;
    if (resolve_geom(dims, pool_axis, &g) != FASTVIM_OK) return 0;
    return workspace_layout(g, nullptr, nullptr);
}

int fastvim_ssm_fwd(const void* x, const void* z, const fastvim_params* params, const fastvim_dims* dims,
                    int pool_axis, const int32_t* mask_idx, void* out, void* stream) {
    return fwd_entry(x, z, params, dims, pool_axis, mask_idx, out, static_cast<hipStream_t>(stream), nullptr);
}

int fastvim_ssm_fwd_stages(const void* x, const void* z, const fastvim_params* params, const fastvim_dims* dims,
                           int pool_axis, const int32_t* mask_idx, void* out, void* stream, float* u_out,
                           float* s_f_out, float* s_b_out, int32_t* row_of_token) {
    const StageDst dst{u_out, s_f_out, s_b_out, row_of_token};
    return fwd_entry(x, z, params, dims, pool_axis, mask_idx, out, static_cast<hipStream_t>(stream), &dst);
}

int fastvim_ssm_stage(int stage, const void* x, const void* z, const fastvim_params* params,
                      const fastvim_dims* dims, int pool_axis, const int32_t* mask_idx, void* out, void* stream) {
    if (stage < FASTVIM_STAGE_ROWS || stage > FASTVIM_STAGE_EPILOGUE) return FASTVIM_ERR_ARG;
    Geom g;
    Workspace ws;
    bool empty = false;
    int st = validate(x, z, params, dims, pool_axis, mask_idx, out, &g, &empty);
    if (st || empty) return st;
    if (conv_written(g, params->flags)) return FASTVIM_ERR_UNSUPPORTED;  // its conv is a step of its own
    if ((st = bind_workspace(g, x, z, *params, out, &ws))) return st;
    return run_stage(stage, g, x, z, effective_params(*params), mask_idx, out, ws, static_cast<hipStream_t>(stream));
}

size_t fastvim_ssm_export_bytes(const fastvim_dims* dims, int pool_axis, int what) {
    Geom g;
    if (resolve_geom(dims, pool_axis, &g) != FASTVIM_OK) return 0;
    return export_bytes(g, what);
}

int fastvim_ssm_export(const fastvim_params* params, const fastvim_dims* dims, int pool_axis, int what, void* dst,
                       size_t dst_bytes, void* stream) {
    if (!params || !dims) return FASTVIM_ERR_NULL;
    Geom g;
    int st = resolve_geom(dims, pool_axis, &g);
    if (st) return st;
    const size_t n = export_bytes(g, what);
    if (n == 0) return g.B == 0 && what >= FASTVIM_EXPORT_U && what <= FASTVIM_EXPORT_STATUS ? FASTVIM_OK
                                                                                             : FASTVIM_ERR_ARG;
    if (!dst) return FASTVIM_ERR_NULL;
    if (!params->workspace) return FASTVIM_ERR_WORKSPACE;
    if (dst_bytes < n) return FASTVIM_ERR_DIMS;
    if (params->workspace_bytes < workspace_layout(g, nullptr, nullptr)) return FASTVIM_ERR_WORKSPACE;
    Workspace ws;
    workspace_layout(g, params->workspace, &ws);
    const void* src = nullptr;
    switch (what) {
        case FASTVIM_EXPORT_U: src = params->saved_u ? params->saved_u : ws.u; break;
        case FASTVIM_EXPORT_XDBL: src = ws.xdbl; break;
        case FASTVIM_EXPORT_S_FWD: src = ws.s_f; break;
        case FASTVIM_EXPORT_S_BWD: src = ws.s_b; break;
        case FASTVIM_EXPORT_ROWS: src = ws.rows; break;
        case FASTVIM_EXPORT_BAD_TOKENS: src = ws.bad; break;
        default: src = ws.sync + 1; break;
    }
    hipError_t e = hipMemcpyAsync(dst, src, n, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? FASTVIM_OK : FASTVIM_ERR_HIP;
}

size_t fastvim_ssm_bwd_workspace_bytes(const fastvim_dims* dims, int pool_axis) {
    Geom g;
    if (resolve_geom(dims, pool_axis, &g) != FASTVIM_OK || !bwd_supported(g)) return 0;
    return bwd_total_bytes(g);
}

int fastvim_ssm_bwd(const void* x, const void* z, const void* dout, const fastvim_params* params,
                    const fastvim_dims* dims, int pool_axis, const int32_t* mask_idx, void* dx, void* dz,
                    const fastvim_grads* grads, void* stream) {
    Geom g;
    bool empty = false;
    int st = validate_bwd(x, z, dout, params, dims, pool_axis, mask_idx, dx, dz, grads, &g, &empty);
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (empty) {  // no tokens: every gradient is zero
        const int64_t n[5] = {g.NX * g.E, g.E * g.R, g.E, g.E * g.N, g.E};
        for (const fastvim_dir_grads* gd : {&grads->fwd, &grads->bwd}) {
            float* ps[5] = {gd->x_proj_w, gd->dt_proj_w, gd->dt_proj_b, gd->A_log, gd->D};
            for (int i = 0; i < 5; ++i)
                if (launch_fill_zero(ps[i], n[i], s) != hipSuccess) return FASTVIM_ERR_HIP;
        }
        if ((params->flags & FASTVIM_FLAG_POST_NORM) &&
            (launch_fill_zero(grads->ln_weight, g.E, s) != hipSuccess ||
             launch_fill_zero(grads->ln_bias, g.E, s) != hipSuccess))
            return FASTVIM_ERR_HIP;
        if ((params->flags & FASTVIM_FLAG_CONV) &&
            (launch_fill_zero(grads->conv_w, g.E * FASTVIM_CONV_TAPS, s) != hipSuccess ||
             launch_fill_zero(grads->conv_b, g.E, s) != hipSuccess))
            return FASTVIM_ERR_HIP;
        return FASTVIM_OK;
    }
    StreamScratch scratch;
    void* base = params->workspace;
    if (!base && (st = scratch.take(bwd_total_bytes(g), s, &base))) return st;
    st = run_bwd(g, x, z, dout, effective_params(*params), mask_idx, dx, dz, *grads, base, s);
    return scratch.give_back(st);
}

int fastvim_get_device_error(const fastvim_params* params, void* stream) {
    if (!params) return FASTVIM_ERR_NULL;
    if (!params->workspace || params->workspace_bytes < 2 * sizeof(unsigned)) return FASTVIM_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    unsigned word = 0;
    const unsigned* src = static_cast<const unsigned*>(params->workspace) + 1;
    if (hipMemcpyAsync(&word, src, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return FASTVIM_ERR_HIP;
    if (word & kStatusWaitGaveUp) return FASTVIM_ERR_DEVICE_WAIT;
    if (word & kStatusBadIndex) return FASTVIM_ERR_BAD_INDEX;
    return FASTVIM_OK;
}

int fastvim_calib_copy(void* dst, const void* src, size_t bytes, void* stream) {
    if (bytes == 0) return FASTVIM_OK;
    if (!dst || !src) return FASTVIM_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src) | bytes) & 15) return FASTVIM_ERR_ALIGN;
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst), s0 = reinterpret_cast<uintptr_t>(src);
    if (d0 < s0 + bytes && s0 < d0 + bytes) return FASTVIM_ERR_OVERLAP;
    return launch_calib_copy(dst, src, bytes, static_cast<hipStream_t>(stream)) == hipSuccess ? FASTVIM_OK
                                                                                               : FASTVIM_ERR_HIP;
}

const char* fastvim_status_string(int status) {
    switch (status) {
        case FASTVIM_OK: return "ok";
        case FASTVIM_ERR_NULL: return "a required pointer is NULL";
        case FASTVIM_ERR_DIMS: return "a size is out of range or inconsistent";
        case FASTVIM_ERR_UNSUPPORTED: return "shape not supported by this build (N != 16, R > 64, E > 4096 or E not a multiple of the vector width, h*w*E >= 2^31, masked grid > 16384 cells)";
        case FASTVIM_ERR_ALIGN: return "misaligned pointer (x, z, out, x_proj_w need 16 bytes, workspace 256, others 4)";
        case FASTVIM_ERR_OVERLAP: return "out overlaps x or z, or the workspace overlaps an input or output";
        case FASTVIM_ERR_WORKSPACE: return "workspace smaller than fastvim_ssm_workspace_bytes, or NULL where the call needs the caller's";
        case FASTVIM_ERR_HIP: return "HIP reported an error while enqueuing work or allocating stream-ordered scratch";
        case FASTVIM_ERR_ARG: return "bad enum, stage or export id, unknown or conflicting flags or tuning bits, or mask_idx given for a dense layer";
        case FASTVIM_ERR_BAD_INDEX: return "the device found an invalid mask index (out of range or repeated)";
        case FASTVIM_ERR_DEVICE_WAIT: return "a wait inside the single launch gave up; its outputs are invalid";
        case FASTVIM_ERR_SCRATCH: return "the layer needs more scratch than the fixed buffer of fastvim_ssm_fwd_noalloc holds (FASTVIM_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

int fastvim_abi_version(void) { return FASTVIM_ABI_VERSION; }

}  // extern "C"
