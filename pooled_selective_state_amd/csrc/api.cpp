// Host side of the C ABI: argument validation, workspace layout, stage
// dispatch and intermediate-result export.  Every check runs on the host
// before anything is enqueued, so an argument error launches nothing.
#include <cmath>
#include <cstdint>
#include <cstring>

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
    return na && nb && pa < pb + nb && pb < pa + na;
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

// FASTVIM_FLAG_POOL_SCALE: a finite factor, pooled layers only, into g.
int apply_pool_scale(const fastvim_params& p, Geom* g) {
    if (!(p.flags & FASTVIM_FLAG_POOL_SCALE)) return FASTVIM_OK;
    if (!g->pooled || !std::isfinite(p.pool_scale)) return FASTVIM_ERR_ARG;
    g->pool_scale = p.pool_scale;
    return FASTVIM_OK;
}

// Full validation of a layer call.  *empty is set for B == 0.
int validate(const void* x, const void* z, const fastvim_params* prm, const fastvim_dims* d, int axis,
             const int32_t* idx, const void* out, Geom* g, Workspace* ws, bool* empty) {
    if (!prm) return FASTVIM_ERR_NULL;
    const uint32_t paths = FASTVIM_FLAG_STAGED | FASTVIM_FLAG_FUSED;
    const uint32_t options =
        FASTVIM_FLAG_POST_NORM | FASTVIM_FLAG_CONV | FASTVIM_FLAG_LOCAL_BWD | FASTVIM_FLAG_POOL_SCALE;
    if ((prm->flags & ~(paths | options)) || (prm->flags & paths) == paths) return FASTVIM_ERR_ARG;
    int st = resolve_geom(d, axis, g);
    if (st) return st;
    if ((st = apply_pool_scale(*prm, g))) return st;
    if ((prm->flags & FASTVIM_FLAG_CONV) &&
        (!g->pooled || g->masked || (prm->flags & FASTVIM_FLAG_POST_NORM)))
        return FASTVIM_ERR_UNSUPPORTED;
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
    if (!prm->workspace) return FASTVIM_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(z, 16) || !aligned(out, 16) || !aligned(prm->workspace, 256) ||
        (idx && !aligned(idx, 4)))
        return FASTVIM_ERR_ALIGN;
    const size_t need = workspace_layout(*g, nullptr, nullptr);
    if (prm->workspace_bytes < need) return FASTVIM_ERR_WORKSPACE;
    const size_t io_bytes =
        (size_t)(g->B * (g->masked ? g->K : g->h * g->w) * g->E) * (g->io == FASTVIM_F32 ? 4 : 2);
    if (overlap(out, io_bytes, x, io_bytes) || overlap(out, io_bytes, z, io_bytes)) return FASTVIM_ERR_OVERLAP;
    const void* w = prm->workspace;
    if (overlap(w, need, x, io_bytes) || overlap(w, need, z, io_bytes) || overlap(w, need, out, io_bytes))
        return FASTVIM_ERR_OVERLAP;
    if (prm->saved_u) {
        const void* su = prm->saved_u;
        const size_t ub = (size_t)(g->B * g->T * g->E) * sizeof(float);
        if (!aligned(su, 16)) return FASTVIM_ERR_ALIGN;
        if (overlap(su, ub, x, io_bytes) || overlap(su, ub, z, io_bytes) || overlap(su, ub, out, io_bytes) ||
            overlap(su, ub, w, need))
            return FASTVIM_ERR_OVERLAP;
    }
    workspace_layout(*g, prm->workspace, ws);
    if (prm->saved_u) ws->u = prm->saved_u;
    return FASTVIM_OK;
}

int run_stage(int stage, const Geom& g, const void* x, const void* z, const fastvim_params& p,
              const int32_t* idx, void* out, const Workspace& ws, hipStream_t st) {
    hipError_t e = hipSuccess;
    switch (stage) {
        case FASTVIM_STAGE_ROWS:
            if (g.masked) e = launch_mask_rows(g, idx, ws, st);
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
// at most kBwdTMax steps; with the post-SSM norm, E <= 2048 (bwd_norm.hip).
bool bwd_supported(const Geom& g) { return g.pooled && g.T <= kBwdTMax; }

struct Span {
    const void* p;
    size_t n;
};

// Full validation of a backward call.  *empty is set for B == 0.
int validate_bwd(const void* x, const void* z, const void* dout, const fastvim_params* prm, const fastvim_dims* d,
                 int axis, const int32_t* idx, const void* dx, const void* dz, const fastvim_grads* gr, Geom* g,
                 BwdWorkspace* ws, bool* empty) {
    if (!prm) return FASTVIM_ERR_NULL;
    const uint32_t unsupported = FASTVIM_FLAG_FUSED;
    const uint32_t options = FASTVIM_FLAG_STAGED | FASTVIM_FLAG_POST_NORM | FASTVIM_FLAG_POOL_SCALE |
                             FASTVIM_FLAG_LOCAL_BWD | FASTVIM_FLAG_CONV;
    if (prm->flags & ~(options | unsupported)) return FASTVIM_ERR_ARG;
    if (prm->flags & unsupported) return FASTVIM_ERR_UNSUPPORTED;
    const bool norm = (prm->flags & FASTVIM_FLAG_POST_NORM) != 0;
    const bool conv = (prm->flags & FASTVIM_FLAG_CONV) != 0;
    int st = resolve_geom(d, axis, g);
    if (st) return st;
    if ((st = apply_pool_scale(*prm, g))) return st;
    if (!bwd_supported(*g) || (norm && !bwd_norm_supported(*g))) return FASTVIM_ERR_UNSUPPORTED;
    if (conv && (g->masked || norm)) return FASTVIM_ERR_UNSUPPORTED;  // as the forward call
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
    Span gs[12];
    for (int k = 0; k < 2; ++k) {
        const float* ps[5] = {gd[k]->x_proj_w, gd[k]->dt_proj_w, gd[k]->dt_proj_b, gd[k]->A_log, gd[k]->D};
        for (int i = 0; i < 5; ++i) {
            if (!ps[i]) return FASTVIM_ERR_NULL;
            if (!aligned(ps[i], 4)) return FASTVIM_ERR_ALIGN;
            gs[5 * k + i] = Span{ps[i], gsz[i] * sizeof(float)};
        }
    }
    const int ngs = norm || conv ? 12 : 10;
    if (norm) {
        gs[10] = Span{gr->ln_weight, (size_t)g->E * sizeof(float)};
        gs[11] = Span{gr->ln_bias, (size_t)g->E * sizeof(float)};
    } else if (conv) {
        gs[10] = Span{gr->conv_w, (size_t)(g->E * FASTVIM_CONV_TAPS) * sizeof(float)};
        gs[11] = Span{gr->conv_b, (size_t)g->E * sizeof(float)};
    }
    for (int i = 0; i < ngs; ++i)
        for (int j = i + 1; j < ngs; ++j)
            if (overlap(gs[i].p, gs[i].n, gs[j].p, gs[j].n)) return FASTVIM_ERR_OVERLAP;
    *empty = g->B == 0;
    if (*empty) return FASTVIM_OK;
    if (!x || !z || !dout || !dx || !dz || (g->masked && !idx)) return FASTVIM_ERR_NULL;
    const fastvim_params eff = effective_params(*prm);
    if ((st = check_dir(eff.fwd)) || (st = check_dir(eff.bwd))) return st;
    if (!prm->workspace) return FASTVIM_ERR_WORKSPACE;
    if (!aligned(x, 16) || !aligned(z, 16) || !aligned(dout, 16) || !aligned(dx, 16) || !aligned(dz, 16) ||
        !aligned(prm->workspace, 256) || (idx && !aligned(idx, 4)))
        return FASTVIM_ERR_ALIGN;
    const size_t need = bwd_workspace_layout(*g, nullptr, nullptr);
    if (prm->workspace_bytes < need) return FASTVIM_ERR_WORKSPACE;
    const size_t io = (size_t)(g->B * (g->masked ? g->K : g->h * g->w) * g->E) * (g->io == FASTVIM_F32 ? 4 : 2);
    // outputs (dx, dz, the workspace and every gradient) overlap neither each
    // other nor an input; parameters count as inputs
    Span ins[16] = {{x, io}, {z, io}, {dout, io}};
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
    } else if (conv) {
        ins[nin++] = Span{prm->conv_w, (size_t)(g->E * FASTVIM_CONV_TAPS) * sizeof(float)};
        ins[nin++] = Span{prm->conv_b, (size_t)g->E * sizeof(float)};
    }
    Span outs[15] = {{dx, io}, {dz, io}, {prm->workspace, need}};
    const int nout = 3 + ngs;
    for (int i = 0; i < ngs; ++i) outs[3 + i] = gs[i];
    for (int i = 0; i < nout; ++i) {
        for (int j = 0; j < nin; ++j)
            if (overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return FASTVIM_ERR_OVERLAP;
        for (int j = i + 1; j < nout; ++j)
            if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return FASTVIM_ERR_OVERLAP;
    }
    bwd_workspace_layout(*g, prm->workspace, ws);
    if (prm->saved_u) {
        ws->fwd.u = prm->saved_u;
        ws->u_saved = true;
    }
    return FASTVIM_OK;
}

int run_bwd(const Geom& g, const void* x, const void* z, const void* dout, const fastvim_params& p,
            const int32_t* idx, void* dx, void* dz, const fastvim_grads& gr, const BwdWorkspace& ws, hipStream_t s) {
    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t r) {
        if (e == hipSuccess) e = r;
        return e == hipSuccess;
    };
    const bool norm = (p.flags & FASTVIM_FLAG_POST_NORM) != 0;
    const bool local = (p.flags & FASTVIM_FLAG_LOCAL_BWD) != 0;  // p holds the effective parameters
    const bool conv = (p.flags & FASTVIM_FLAG_CONV) != 0;
    if (g.masked && !ok(launch_mask_rows(g, idx, ws.fwd, s))) return FASTVIM_ERR_HIP;
    if (norm) {
        // the norm's adjoint needs y, hence both scans' outputs: recompute the
        // forward stages first, then the first pass with the norm, whose
        // per-(b, t) partials of dD, d ln_w and d ln_b (in du, du_f, du_b) are
        // summed before the scan adjoint overwrites those buffers
        if ((!ws.u_saved && !ok(launch_pool(g, x, ws.fwd, s))) || !ok(launch_proj(g, x, p, ws.fwd, s)) ||
            !ok(launch_scan(g, x, p, ws.fwd, s)) || !ok(launch_bwd_norm_pass1(g, x, z, dout, p, ws, dx, dz, s)))
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
    BwdScanArgs a{ws.fwd.xdbl, ws.fwd.u, ws.gs, p.fwd, p.bwd, ws.fwd.s_f, ws.fwd.s_b, ws.du_f, ws.du_b, ws.dvp,
                  ws.ckpt, ws.dAp, ws.dWdtp, ws.dbp, g.B, g.T, g.E, (int)g.R, (int)g.NX, (int)ws.G, local};
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
    if (!ok(launch_colsum_batch(batch, s))) return FASTVIM_ERR_HIP;
    if (norm) return ok(launch_bwd_norm_pass2(g, p, ws, dx, dz, s)) ? FASTVIM_OK : FASTVIM_ERR_HIP;
    if (conv) {
        // second pass through the conv; its partial rows go to the checkpoint
        // region (free once the scan adjoint has run; large enough: see
        // bwd_workspace_layout)
        const int64_t np = bwd_conv_parts(g);
        const int64_t ckpt_floats = 2 * g.B * ws.G * (kBwdTMax / 16) * 256 * 4;
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

}  // namespace

size_t workspace_layout(const Geom& g, void* base, Workspace* ws) {
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align256(off + bytes);
        return o;
    };
    const size_t bte = (size_t)(g.B * g.T * g.E) * sizeof(float);
    const size_t o_u = g.pooled ? take(bte) : 0;
    const size_t o_x = take((size_t)(g.B * g.T * 2 * g.NX) * sizeof(float));
    const size_t o_sf = take(bte);
    const size_t o_sb = take(bte);
    const size_t o_rows = g.masked ? take((size_t)(g.B * g.K) * sizeof(int32_t)) : 0;
    const size_t o_bad = g.masked ? take((size_t)g.B * sizeof(int32_t)) : 0;
    const size_t o_sync = take((size_t)sync_words(g) * sizeof(unsigned));
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

size_t bwd_workspace_layout(const Geom& g, void* base, BwdWorkspace* ws) {
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
    const size_t o_u = take(bte);
    const size_t o_x = take((size_t)(M * 2 * NX) * sizeof(float));
    const size_t o_sf = take(bte), o_sb = take(bte);
    const size_t o_rows = g.masked ? take((size_t)(B * g.K) * sizeof(int32_t)) : 0;
    const size_t o_bad = g.masked ? take((size_t)B * sizeof(int32_t)) : 0;
    const int64_t ND = bwd_dd_parts(g);
    const size_t o_gs = take(bte), o_dDp = take((size_t)(ND * E) * sizeof(float));
    const size_t o_duf = take(bte), o_dub = take(bte), o_du = take(bte);
    const size_t o_dvp = take((size_t)(2 * B * G * T * S) * sizeof(float));
    const size_t o_ck = take((size_t)(2 * B * G * (kBwdTMax / 16) * 256 * 4) * sizeof(float));
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
    if (base && ws) {
        char* c = static_cast<char*>(base);
        auto f = [&](size_t o) { return reinterpret_cast<float*>(c + o); };
        ws->fwd.u = f(o_u);
        ws->fwd.xdbl = f(o_x);
        ws->fwd.s_f = f(o_sf);
        ws->fwd.s_b = f(o_sb);
        ws->fwd.rows = g.masked ? reinterpret_cast<int32_t*>(c + o_rows) : nullptr;
        ws->fwd.bad = g.masked ? reinterpret_cast<int32_t*>(c + o_bad) : nullptr;
        ws->fwd.sync = nullptr;
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
    Geom g;
    Workspace ws;
    bool empty = false;
    int st = validate(x, z, params, dims, pool_axis, mask_idx, out, &g, &ws, &empty);
    if (st || empty) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_zero_sync(ws, sync_words(g), s) != hipSuccess) return FASTVIM_ERR_HIP;
    const fastvim_params q = effective_params(*params);
    const bool norm = (params->flags & FASTVIM_FLAG_POST_NORM) != 0;
    const bool local = (params->flags & FASTVIM_FLAG_LOCAL_BWD) != 0;
    const bool single = !(params->flags & FASTVIM_FLAG_CONV) &&
                        ((params->flags & FASTVIM_FLAG_FUSED)
                             ? fused_supported(g, norm, local)
                             : !(params->flags & FASTVIM_FLAG_STAGED) && fused_preferred(g, norm, local));
    if (single) return launch_fused(g, x, z, q, ws, out, s) == hipSuccess ? FASTVIM_OK : FASTVIM_ERR_HIP;
    for (int stage = FASTVIM_STAGE_ROWS; stage <= FASTVIM_STAGE_EPILOGUE; ++stage) {
        st = run_stage(stage, g, x, z, q, mask_idx, out, ws, s);
        if (st) return st;
    }
    return FASTVIM_OK;
}

int fastvim_ssm_stage(int stage, const void* x, const void* z, const fastvim_params* params,
                      const fastvim_dims* dims, int pool_axis, const int32_t* mask_idx, void* out, void* stream) {
    if (stage < FASTVIM_STAGE_ROWS || stage > FASTVIM_STAGE_EPILOGUE) return FASTVIM_ERR_ARG;
    Geom g;
    Workspace ws;
    bool empty = false;
    int st = validate(x, z, params, dims, pool_axis, mask_idx, out, &g, &ws, &empty);
    if (st || empty) return st;
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
    if (!dst || !params->workspace) return FASTVIM_ERR_NULL;
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
    return bwd_workspace_layout(g, nullptr, nullptr);
}

int fastvim_ssm_bwd(const void* x, const void* z, const void* dout, const fastvim_params* params,
                    const fastvim_dims* dims, int pool_axis, const int32_t* mask_idx, void* dx, void* dz,
                    const fastvim_grads* grads, void* stream) {
    Geom g;
    BwdWorkspace ws;
    bool empty = false;
    const int st = validate_bwd(x, z, dout, params, dims, pool_axis, mask_idx, dx, dz, grads, &g, &ws, &empty);
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
    return run_bwd(g, x, z, dout, effective_params(*params), mask_idx, dx, dz, *grads, ws, s);
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
        case FASTVIM_ERR_WORKSPACE: return "workspace missing or smaller than fastvim_ssm_workspace_bytes";
        case FASTVIM_ERR_HIP: return "HIP reported an error while enqueuing work";
        case FASTVIM_ERR_ARG: return "bad enum, stage or export id, unknown or conflicting flags, or mask_idx given for a dense layer";
        default: return "unknown status";
    }
}

int fastvim_abi_version(void) { return FASTVIM_ABI_VERSION; }

}  // extern "C"
