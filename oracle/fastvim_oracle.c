/*
 * fastvim_oracle.c -- plain, slow, fp64 CPU oracle of the pooled bidirectional
 * selective-scan layer of FastVim (Fast Vision Mamba, arXiv 2502.00594).
 *
 * TEST INFRASTRUCTURE ONLY.  The library built from this file is loaded by the
 * test-suite, by the smoke check and by the benchmark's CPU-baseline leg, and
 * by nothing else.  The GPU product path never links, loads or calls it, and
 * this file shares no code, header, table or constant with the GPU path.
 *
 * Every stage is written as its plain definition, in fp64, with sequential
 * loops; the only parallelism is an OpenMP loop over independent images.
 * Inputs arrive as fp32 (bf16 inputs are widened to fp32 by the caller, which
 * is exact) and are widened to double before any arithmetic.
 *
 * Sources (cited by page and section; no line numbers):
 *   [FastVim summary]  gptget.net page on arXiv 2502.00594 (Chinese summary),
 *                      sections "方法详解" (method details, six bullets),
 *                      "术语表" (glossary) and "技术贡献".
 *   [Pith review]      pith.science verdict on 2502.00594, JSON fields
 *                      "key_machinery", "core_discovery", "minor_comments",
 *                      "referee_report" (major comments: the MAE experiments).
 *   [Vim article]      ijyty.com/news/106204, section 2.1, vim_block sketch.
 *   [SF-Mamba article] glsqs.com/news/422358, section 二 (batch folding with
 *                      periodic state reset).
 *   [LBMamba article]  pswp.cn page on LBMamba, 论文创新点 1-2 (the local
 *                      backward scan inside the forward scan).
 *
 * Readings of points the pages leave open:
 *   - x_proj output is split [delta_lowrank (R) | B (N) | C (N)];
 *   - s_delta(x) is the low-rank map W_dt * delta_lowrank plus a bias;
 *   - A = -exp(A_log) (negative real, so the recurrence is stable);
 *   - B enters as Delta * B_t * u_t (Euler), A as exp(Delta * A) (ZOH);
 *   - the skip D*x is added after the repeat, on the full-resolution x, with
 *     one D per direction (the layer adds (D_fwd + D_bwd) * x);
 *   - the two directions are summed, then gated by silu(z);
 *   - optionally a post-SSM LayerNorm over the channels of each token sits
 *     between the skip and the gate (population variance, eps inside the
 *     root, per-channel scale and shift);
 *   - initial state is zero; no state is output;
 *   - the producer Conv1D is depthwise, causal, with its taps along the
 *     oriented grid's sequence and SiLU after it; the layer's x is its output;
 *   - the local backward scan runs on the forward direction's inputs, its
 *     state reset at the top of every window of L steps aligned at t = 0;
 *   - the MAE recipe's pooling factor multiplies the pooled tokens only.
 * The backward pass is the chain rule through these definitions, one adjoint
 * per forward step; it is pinned by central differences of the forward
 * functions, not by a second derivation.
 *
 * Layouts (all row-major, last index fastest):
 *   dense x, z, out   (B, h, w, E)            masked x, z, out   (B, K, E)
 *   u                 (B, T, E)               v (x_proj output)  (B, T, NX), NX = R + 2N
 *   delta             (B, T, E)               s_fwd, s_bwd       (B, T, E)
 *   x_proj_w (NX, E)  dt_proj_w (E, R)  dt_proj_b (E)  A_log (E, N)  D (E)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Pooling axes.  COLS: mean over w, scan over the h rows.  ROWS: the
 * transposed grid, mean over h, scan over the w columns.  NONE_*: no pooling,
 * the scan runs over all h*w tokens in row-major (t = i*w + j) or column-major
 * (t = j*h + i) order. */
enum { FVO_COLS = 0, FVO_ROWS = 1, FVO_NONE_ROWMAJOR = 2, FVO_NONE_COLMAJOR = 3 };

typedef struct {
    const float *x_proj_w;  /* (R + 2N, E) */
    const float *dt_proj_w; /* (E, R) */
    const float *dt_proj_b; /* (E) */
    const float *A_log;     /* (E, N) */
    const float *D;         /* (E) */
} fvo_dir;

int fvo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls' image-parallel loops (timing only; the
 * results do not depend on it: images are independent). */
void fvo_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Scan length T and pooled-axis length P for a dense grid. */
static void seq_shape(int axis, int64_t h, int64_t w, int64_t *T, int64_t *P)
{
    switch (axis) {
    case FVO_COLS: *T = h; *P = w; break;
    case FVO_ROWS: *T = w; *P = h; break;
    default: *T = h * w; *P = 1; break;
    }
}

/* Position t along the scan of grid cell (i, j). */
static int64_t seq_pos(int axis, int64_t h, int64_t w, int64_t i, int64_t j)
{
    switch (axis) {
    case FVO_COLS: return i;
    case FVO_ROWS: return j;
    case FVO_NONE_ROWMAJOR: return i * w + j;
    default: return j * h + i;
    }
}

/*
 * O1, dense pooling.  [FastVim summary, 方法详解 bullets 1-2; 术语表 "Mean
 * Pooling"]: after the Conv1D the (B, h, w, D) grid is averaged, without
 * parameters, along one spatial axis, giving (B, h, 1, D).  The transposed
 * grid of the next block pools the other axis [FastVim summary, 方法详解
 * bullet 5].  With no pooling u is x itself, read in scan order.
 *   u[b, t, e] = (1/P) * sum_{cells (i,j) with seq_pos(i,j) = t} x[b, i, j, e]
 */
static void pool_dense_any(const float *x, const double *xd, int64_t B, int64_t h, int64_t w, int64_t E,
                           int axis, double *u);

int fvo_pool_dense(const float *x, int64_t B, int64_t h, int64_t w, int64_t E, int axis, double *u)
{
    if (axis < 0 || axis > 3) return -2;
    pool_dense_any(x, NULL, B, h, w, E, axis, u);
    return 0;
}

/* The same, reading x from xd (double) when xd is given. */
static void pool_dense_any(const float *x, const double *xd, int64_t B, int64_t h, int64_t w, int64_t E,
                           int axis, double *u)
{
    int64_t T, P;
    seq_shape(axis, h, w, &T, &P);
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        double *ub = u + b * T * E;
        for (int64_t k = 0; k < T * E; ++k) ub[k] = 0.0;
        for (int64_t i = 0; i < h; ++i)
            for (int64_t j = 0; j < w; ++j) {
                const int64_t t = seq_pos(axis, h, w, i, j);
                const int64_t c = ((b * h + i) * w + j) * E;
                for (int64_t e = 0; e < E; ++e) ub[t * E + e] += xd ? xd[c + e] : (double)x[c + e];
            }
        for (int64_t k = 0; k < T * E; ++k) ub[k] /= (double)P;
    }
}

/*
 * Producer side: depthwise causal Conv1D and SiLU on the token sequence of
 * the oriented grid.  [FastVim summary, 方法详解 bullets 1-2: the grid is
 * pooled after the Conv1D; Vim article 2.1: conv1d then the SSM, per
 * direction in Vim, one shared x here.]  The sequence is the flattened
 * oriented grid, the scan order of the unpooled layer: row-major
 * (r = i*w + j) for COLS and NONE_ROWMAJOR, column-major (r = j*h + i) for ROWS
 * and NONE_COLMAJOR.  With KC taps per channel (the oldest first):
 *   xc[b, cell(r), e] = silu(conv_b[e] + sum_{k<KC} conv_w[e, k] x[b, cell(r - KC + 1 + k), e])
 * where positions before the start of the sequence contribute zero.
 * xc has x's (B, h, w, E) layout.
 */
int fvo_conv_silu(const float *x, int64_t B, int64_t h, int64_t w, int64_t E, int axis, const float *conv_w,
                  const float *conv_b, int64_t KC, double *xc)
{
    if (axis < 0 || axis > 3) return -2;
    const int colmajor = axis == FVO_ROWS || axis == FVO_NONE_COLMAJOR;
    const int64_t n = h * w;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b)
        for (int64_t r = 0; r < n; ++r) {
            const int64_t cell = colmajor ? (r % h) * w + r / h : r;
            for (int64_t e = 0; e < E; ++e) {
                double acc = (double)conv_b[e];
                for (int64_t k = 0; k < KC; ++k) {
                    const int64_t rr = r - KC + 1 + k;
                    if (rr < 0) continue;
                    const int64_t cc = colmajor ? (rr % h) * w + rr / h : rr;
                    acc += (double)conv_w[e * KC + k] * (double)x[(b * n + cc) * E + e];
                }
                xc[(b * n + cell) * E + e] = acc / (1.0 + exp(-acc));
            }
        }
    return 0;
}

/*
 * Masked rows.  [FastVim summary, 方法详解 bullet 6; 技术贡献]: FastMaskVim
 * works on the kept tokens' sparse indices into the h*w grid.  A kept token
 * with flat index q = i*w + j belongs to scan row i (COLS) or to column j
 * (ROWS).  Returns -3 for an index outside [0, h*w) or a repeated index.
 */
int fvo_mask_rows(const int32_t *idx, int64_t B, int64_t K, int64_t h, int64_t w, int axis, int32_t *rows)
{
    if (axis != FVO_COLS && axis != FVO_ROWS) return -2;
    int bad = 0;
    unsigned char *seen = (unsigned char *)malloc((size_t)(h * w));
    if (!seen) return -9;
    for (int64_t b = 0; b < B; ++b) {
        memset(seen, 0, (size_t)(h * w));
        for (int64_t k = 0; k < K; ++k) {
            const int64_t q = idx[b * K + k];
            if (q < 0 || q >= h * w || seen[q]) { bad = 1; rows[b * K + k] = -1; continue; }
            seen[q] = 1;
            rows[b * K + k] = (int32_t)(axis == FVO_COLS ? q / w : q % w);
        }
    }
    free(seen);
    return bad ? -3 : 0;
}

/*
 * O1, masked pooling.  [FastVim summary, 方法详解 bullet 6]: the kept tokens
 * of a row are summed and normalised by the fixed row length P (w for COLS,
 * h for ROWS), not by how many tokens of that row were kept.  A row with no
 * kept token pools to zero and is still scanned.
 *   u[b, t, e] = (1/P) * sum_{k : rows[b,k] = t} x[b, k, e]
 */
static void pool_masked_any(const float *x, const double *xd, const int32_t *rows, int64_t B, int64_t K,
                            int64_t T, int64_t P, int64_t E, double *u);

int fvo_pool_masked(const float *x, const int32_t *rows, int64_t B, int64_t K, int64_t T, int64_t P,
                    int64_t E, double *u)
{
    pool_masked_any(x, NULL, rows, B, K, T, P, E, u);
    return 0;
}

/* The same, reading the kept tokens from xd (double) when xd is given. */
static void pool_masked_any(const float *x, const double *xd, const int32_t *rows, int64_t B, int64_t K,
                            int64_t T, int64_t P, int64_t E, double *u)
{
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        double *ub = u + b * T * E;
        for (int64_t k = 0; k < T * E; ++k) ub[k] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t t = rows[b * K + k];
            if (t < 0 || t >= T) continue;
            const int64_t c = (b * K + k) * E;
            for (int64_t e = 0; e < E; ++e) ub[t * E + e] += xd ? xd[c + e] : (double)x[c + e];
        }
        for (int64_t k = 0; k < T * E; ++k) ub[k] /= (double)P;
    }
}

/*
 * The producer Conv1D of a masked layer runs along the sequence of kept
 * tokens as they are given, k = 0 .. K-1: FastMaskVim's block sees only the
 * kept tokens (the MAE encoder drops the masked ones), and the Conv1D is a
 * sequence operation of that block [FastVim summary, 方法详解 bullets 1-2
 * and 6].  In fvo_conv_silu's terms that sequence is a K x 1 grid in row-major
 * order.
 */
static void conv_silu_masked(const float *x, int64_t B, int64_t K, int64_t E, const float *conv_w,
                             const float *conv_b, int64_t KC, double *xc)
{
    fvo_conv_silu(x, B, K, 1, E, FVO_COLS, conv_w, conv_b, KC, xc);
}

/*
 * O2, input-dependent projection.  [FastVim summary, 方法详解 bullet 3]:
 * Linear_N produces the input-dependent B and C (and the low-rank input of
 * Delta) from each pooled token.
 *   v[m, o] = sum_e x_proj_w[o, e] * u[m, e],   o in [0, R + 2N)
 */
void fvo_xproj(const double *u, int64_t M, int64_t E, const float *x_proj_w, int64_t NX, double *v)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t o = 0; o < NX; ++o) {
            double acc = 0.0;
            for (int64_t e = 0; e < E; ++e) acc += (double)x_proj_w[o * E + e] * u[m * E + e];
            v[m * NX + o] = acc;
        }
}

/* softplus(q) = log(1 + e^q), written in the overflow-free form. */
static double softplus(double q) { return (q > 0.0 ? q : 0.0) + log1p(exp(-fabs(q))); }

/*
 * O3, step size.  [FastVim summary, 方法详解 bullet 3]: Delta =
 * softplus(Parameter + s_Delta(x)); s_Delta is the low-rank map W_dt * v[0:R]
 * and the Parameter is the bias dt_proj_b.
 *   delta[m, e] = softplus(sum_r dt_proj_w[e, r] * v[m, r] + dt_proj_b[e])
 */
void fvo_delta(const double *v, int64_t M, int64_t NX, int64_t R, const float *dt_proj_w,
               const float *dt_proj_b, int64_t E, double *delta)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t e = 0; e < E; ++e) {
            double q = (double)dt_proj_b[e];
            for (int64_t r = 0; r < R; ++r) q += (double)dt_proj_w[e * R + r] * v[m * NX + r];
            delta[m * E + e] = softplus(q);
        }
}

/*
 * O4 + O5, discretisation and selective scan.  [FastVim summary, 术语表
 * "State Space Model": h_t = A h_{t-1} + B x_t, y_t = C h_t (+ D x_t, added
 * in the output stage); 方法详解 bullets 3-4: zero-order-hold discretisation,
 * then the forward and the backward selective scans over the pooled
 * sequence.]  Per image b and channel e, with A[e,n] = -exp(A_log[e,n]):
 *   H_n <- exp(delta_t * A[e,n]) * H_n + delta_t * B_t[n] * u_t      (H_{-1} = 0)
 *   s_t  = sum_n C_t[n] * H_n
 * B_t = v[t, R + n], C_t = v[t, R + N + n].  The backward scan visits
 * t = T-1 ... 0.  If reset is given, reset[t] != 0 drops the carried state at
 * step t (the decay is set to zero there), as in [SF-Mamba article, 二,
 * periodic state reset].
 */
void fvo_scan(const double *u, const double *delta, const double *v, int64_t B, int64_t T, int64_t E,
              int64_t N, int64_t R, int64_t NX, const float *A_log, int reverse,
              const unsigned char *reset, double *s)
{
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < B; ++b) {
        double *H = (double *)malloc((size_t)N * sizeof(double));
        for (int64_t e = 0; e < E; ++e) {
            for (int64_t n = 0; n < N; ++n) H[n] = 0.0;
            for (int64_t step = 0; step < T; ++step) {
                const int64_t t = reverse ? T - 1 - step : step;
                const int64_t m = b * T + t;
                const double d = delta[m * E + e];
                const double ut = u[m * E + e];
                const double *vt = v + m * NX;
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double A = -exp((double)A_log[e * N + n]);
                    const double a = (reset && reset[t]) ? 0.0 : exp(d * A);
                    H[n] = a * H[n] + d * vt[R + n] * ut;
                    acc += vt[R + N + n] * H[n];
                }
                s[m * E + e] = acc;
            }
        }
        free(H);
    }
}

/* silu(q) = q * sigmoid(q) */
static double silu(double q) { return q / (1.0 + exp(-q)); }

/* Stage outputs of one direction, all optional (NULL = not wanted). */
typedef struct {
    double *v;     /* (B, T, NX) */
    double *delta; /* (B, T, E)  */
    double *s;     /* (B, T, E)  */
} fvo_dir_out;

static int run_direction(const double *u, int64_t B, int64_t T, int64_t E, int64_t N, int64_t R,
                         const fvo_dir *p, int reverse, const unsigned char *reset, fvo_dir_out *o, double *s_out)
{
    const int64_t NX = R + 2 * N, M = B * T;
    double *v = o && o->v ? o->v : (double *)malloc((size_t)(M * NX) * sizeof(double));
    double *dl = o && o->delta ? o->delta : (double *)malloc((size_t)(M * E) * sizeof(double));
    if (!v || !dl) return -9;
    fvo_xproj(u, M, E, p->x_proj_w, NX, v);
    fvo_delta(v, M, NX, R, p->dt_proj_w, p->dt_proj_b, E, dl);
    fvo_scan(u, dl, v, B, T, E, N, R, NX, p->A_log, reverse, reset, s_out);
    if (!(o && o->v)) free(v);
    if (!(o && o->delta)) free(dl);
    return 0;
}

/*
 * The whole layer.  [FastVim summary, 方法详解 bullets 2-5; Pith review,
 * "key_machinery": the pooled scan output is repeated back to the full token
 * count before the D*x skip; Vim article 2.1: the two directions are summed
 * and gated by z.]
 *   out[b, cell, e] = (s_fwd[b, t(cell), e] + s_bwd[b, t(cell), e]
 *                      + (D_fwd[e] + D_bwd[e]) * x[b, cell, e]) * silu(z[b, cell, e])
 * cell is a grid cell (i, j) (dense) or a kept token k (masked, idx != NULL,
 * axis COLS or ROWS only).  Returns 0, or -2 bad axis, -3 bad mask index,
 * -9 out of memory.  Optional stage outputs: u_out (B,T,E), rows_out (B,K),
 * fwd / bwd (v, delta, s).
 */
/*
 * Output of one token (channels e < E): the repeated scan outputs of its scan
 * position plus the skip,
 *   y[e] = s_fwd[e] + s_bwd[e] + (D_fwd[e] + D_bwd[e]) x[e]
 * (FastVim summary, 方法详解 bullet 5: repeat, then the skip connection; Vim
 * article 2.1: the two directions summed), optionally the post-SSM LayerNorm
 * over the channels (FastVim summary, 方法详解 bullet 5, which puts a
 * LayerNorm after the skip connection; Pith review: the post-SSM LayerNorm
 * taken from VMamba, applied to the SSM output before the gate),
 *   y[e] <- (y[e] - mean) / sqrt(var + eps) * ln_w[e] + ln_b[e],
 *   mean = sum_e y[e] / E,  var = sum_e (y[e] - mean)^2 / E,
 * and finally the gate, out[e] = y[e] * silu(z[e]).  y is caller scratch.
 */
static void output_token(const double *sf, const double *sb, const float *x, const double *xd, const float *z,
                         const fvo_dir *pf, const fvo_dir *pb, int64_t E, const float *ln_w, const float *ln_b,
                         double ln_eps, double *y, double *out)
{
    for (int64_t e = 0; e < E; ++e) {
        const double skip = ((double)pf->D[e] + (double)pb->D[e]) * (xd ? xd[e] : (double)x[e]);
        y[e] = sf[e] + sb[e] + skip;
    }
    if (ln_w) {
        double mean = 0.0, var = 0.0;
        for (int64_t e = 0; e < E; ++e) mean += y[e];
        mean /= (double)E;
        for (int64_t e = 0; e < E; ++e) {
            const double d = y[e] - mean;
            var += d * d;
        }
        var /= (double)E;
        const double r = 1.0 / sqrt(var + ln_eps);
        for (int64_t e = 0; e < E; ++e) y[e] = (y[e] - mean) * r * (double)ln_w[e] + (double)ln_b[e];
    }
    for (int64_t e = 0; e < E; ++e) out[e] = y[e] * silu((double)z[e]);
}

/* ln_w == NULL: no post-SSM LayerNorm.  conv_w == NULL: x is the layer's
 * input itself; else x is the Conv1D's input and the layer runs on
 * fvo_conv_silu(x) (masked layers: on conv_silu_masked(x), the conv along the
 * kept tokens in their given order).
 *
 * local_window = L > 0: the local backward scan of LBMamba [LBMamba article,
 * 论文创新点 1-2: a light backward scan inside the forward selective scan, run
 * within subsequences, in place of the global backward scan].  The backward
 * output s_bwd is then the scan over t descending with the forward
 * direction's projection, step size and decay (the same inputs the forward
 * scan holds), whose state starts from zero at the top of every window of L
 * steps, windows aligned at t = 0: a reset at every t with t mod L = L - 1.
 * Of the backward parameters only D is used, in the skip.
 *
 * pool_scale multiplies the pooled tokens u (1 for the layer as defined): the
 * constant factor the MAE transfer recipe applies when pooling during
 * fine-tuning and linear probing, 0.25 there [Pith review, referee_report,
 * major comment on the MAE experiments].  Only u is scaled; the skip reads
 * the full-resolution x as before. */
int fvo_layer(const float *x, const float *z, const fvo_dir *pf, const fvo_dir *pb, int64_t B, int64_t h,
              int64_t w, int64_t E, int64_t N, int64_t R, int64_t K, int axis, const int32_t *idx,
              double *out, double *u_out, int32_t *rows_out, fvo_dir_out *fwd, fvo_dir_out *bwd,
              const float *ln_w, const float *ln_b, double ln_eps, const float *conv_w, const float *conv_b,
              int64_t conv_k, int64_t local_window, double pool_scale)
{
    int64_t T, P;
    const int masked = idx != NULL;
    if (axis < 0 || axis > 3 || (masked && axis > FVO_ROWS)) return -2;
    seq_shape(axis, h, w, &T, &P);
    const int64_t M = B * T, ntok = masked ? B * K : B * h * w;

    double *u = u_out ? u_out : (double *)malloc((size_t)(M * E) * sizeof(double));
    double *sf = fwd && fwd->s ? fwd->s : (double *)malloc((size_t)(M * E) * sizeof(double));
    double *sb = bwd && bwd->s ? bwd->s : (double *)malloc((size_t)(M * E) * sizeof(double));
    double *xc = conv_w ? (double *)malloc((size_t)(ntok * E) * sizeof(double)) : NULL;
    unsigned char *reset = NULL;
    int32_t *rows = NULL;
    int rc = 0;
    if (!u || !sf || !sb || (conv_w && !xc)) { rc = -9; goto done; }
    if (conv_w && masked) conv_silu_masked(x, B, K, E, conv_w, conv_b, conv_k, xc);
    else if (conv_w) fvo_conv_silu(x, B, h, w, E, axis, conv_w, conv_b, conv_k, xc);

    if (masked) {
        rows = rows_out ? rows_out : (int32_t *)malloc((size_t)(B * K) * sizeof(int32_t));
        if (!rows) { rc = -9; goto done; }
        rc = fvo_mask_rows(idx, B, K, h, w, axis, rows);
        if (rc) goto done;
        pool_masked_any(x, xc, rows, B, K, T, P, E, u);
    } else {
        pool_dense_any(x, xc, B, h, w, E, axis, u);
    }
    for (int64_t i = 0; i < M * E; ++i) u[i] *= pool_scale;

    rc = run_direction(u, B, T, E, N, R, pf, 0, NULL, fwd, sf);
    if (rc) goto done;
    if (local_window > 0) {
        const fvo_dir pl = {pf->x_proj_w, pf->dt_proj_w, pf->dt_proj_b, pf->A_log, pb->D};
        reset = (unsigned char *)malloc((size_t)T);
        if (!reset) { rc = -9; goto done; }
        for (int64_t t = 0; t < T; ++t) reset[t] = (unsigned char)(t % local_window == local_window - 1);
        rc = run_direction(u, B, T, E, N, R, &pl, 1, reset, bwd, sb);
    } else {
        rc = run_direction(u, B, T, E, N, R, pb, 1, NULL, bwd, sb);
    }
    if (rc) goto done;

    if (masked) {
#pragma omp parallel for schedule(static)
        for (int64_t b = 0; b < B; ++b) {
            double *y = (double *)malloc((size_t)E * sizeof(double));
            for (int64_t k = 0; y && k < K; ++k) {
                const int64_t t = rows[b * K + k], c = (b * K + k) * E;
                output_token(sf + (b * T + t) * E, sb + (b * T + t) * E, x + c, xc ? xc + c : NULL, z + c, pf, pb,
                             E, ln_w, ln_b, ln_eps, y, out + c);
            }
            free(y);
        }
    } else {
#pragma omp parallel for schedule(static)
        for (int64_t b = 0; b < B; ++b) {
            double *y = (double *)malloc((size_t)E * sizeof(double));
            for (int64_t i = 0; y && i < h; ++i)
                for (int64_t j = 0; j < w; ++j) {
                    const int64_t t = seq_pos(axis, h, w, i, j), c = ((b * h + i) * w + j) * E;
                    output_token(sf + (b * T + t) * E, sb + (b * T + t) * E, x + c, xc ? xc + c : NULL, z + c, pf,
                                 pb, E, ln_w, ln_b, ln_eps, y, out + c);
                }
            free(y);
        }
    }

done:
    free(xc);
    free(reset);
    if (!u_out) free(u);
    if (!(fwd && fwd->s)) free(sf);
    if (!(bwd && bwd->s)) free(sb);
    if (masked && !rows_out) free(rows);
    return rc;
}

/* ------------------------------------------------------------------------
 * Backward pass: the gradient of a scalar loss L = sum(dout * out) with
 * respect to x, z and every parameter of both directions, written as the
 * chain rule taken through the forward steps in reverse order, one step at a
 * time.  Each function below is the adjoint of one forward step above; the
 * training workload the gradients serve is the one the FastVim summary page
 * (实验结果: ImageNet training and MAE pre-training) trains.
 * ------------------------------------------------------------------------ */

/* Gradients of one direction's parameters (all shaped like the parameters). */
typedef struct {
    double *x_proj_w;  /* (NX, E) */
    double *dt_proj_w; /* (E, R)  */
    double *dt_proj_b; /* (E)     */
    double *A_log;     /* (E, N)  */
    double *D;         /* (E)     */
} fvo_dir_grad;

/* Optional intermediate adjoints (NULL = not wanted). */
typedef struct {
    double *gs;    /* (B, T, E)  dL/ds, the same for both directions      */
    double *du;    /* (B, T, E)  dL/du, both directions, scan and x_proj  */
    double *dv_f;  /* (B, T, NX) dL/dv of the forward direction           */
    double *dv_b;  /* (B, T, NX) dL/dv of the backward direction          */
} fvo_bwd_stages;

static double sigmoid(double q) { return 1.0 / (1.0 + exp(-q)); }

/* Pre-activation of the step size, q[m, e] = sum_r dt_proj_w[e, r] v[m, r] + dt_proj_b[e]. */
static void dt_preact(const double *v, int64_t M, int64_t NX, int64_t R, const float *dt_proj_w,
                      const float *dt_proj_b, int64_t E, double *q)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t e = 0; e < E; ++e) {
            double acc = (double)dt_proj_b[e];
            for (int64_t r = 0; r < R; ++r) acc += (double)dt_proj_w[e * R + r] * v[m * NX + r];
            q[m * E + e] = acc;
        }
}

/*
 * Adjoint of the output of one token (no LayerNorm).  With
 * y = s_fwd + s_bwd + (D_fwd + D_bwd) x and out = y silu(z):
 *   g       = dL/dy = dout silu(z)                  (also dL/ds of both scans)
 *   dz      = dout y silu'(z),  silu'(q) = sigmoid(q) (1 + q (1 - sigmoid(q)))
 *   dx_skip = g (D_fwd + D_bwd)
 *   dD     += g x          (the same for D_fwd and D_bwd)
 * xd, when given, is the layer's x in double (the Conv1D's output) in place of x.
 */
static void output_token_adjoint(const double *sf, const double *sb, const float *x, const double *xd,
                                 const float *z, const float *dout, const fvo_dir *pf, const fvo_dir *pb, int64_t E,
                                 double *g, double *dz, double *dx_skip, double *dD)
{
    for (int64_t e = 0; e < E; ++e) {
        const double Ds = (double)pf->D[e] + (double)pb->D[e];
        const double xe = xd ? xd[e] : (double)x[e], ze = (double)z[e], de = (double)dout[e];
        const double y = sf[e] + sb[e] + Ds * xe;
        const double sg = sigmoid(ze);
        g[e] = de * silu(ze);
        dz[e] = de * y * sg * (1.0 + ze * (1.0 - sg));
        dx_skip[e] = g[e] * Ds;
        dD[e] += g[e] * xe;
    }
}

/*
 * Adjoint of the output of one token with the post-SSM LayerNorm (the output
 * of output_token with ln_w set; FastVim summary page, section 方法详解,
 * bullet 5).  With y = s_fwd + s_bwd + (D_fwd + D_bwd) x, its mean and
 * population variance over the token's E channels, r = 1 / sqrt(var + eps),
 * n = (y - mean) r, o = n ln_w + ln_b and out = o silu(z):
 *   dz       = dout o silu'(z)
 *   dln_w   += dout silu(z) n,   dln_b += dout silu(z)
 *   dn       = dout silu(z) ln_w
 *   g = dL/dy = r (dn - mean(dn) - n mean(dn n))     (also dL/ds of both scans)
 *   dx_skip  = g (D_fwd + D_bwd),   dD += g x
 * ny is caller scratch of E doubles; xd as in output_token_adjoint.
 */
static void output_token_adjoint_ln(const double *sf, const double *sb, const float *x, const double *xd,
                                    const float *z,
                                    const float *dout, const fvo_dir *pf, const fvo_dir *pb, int64_t E,
                                    const float *ln_w, const float *ln_b, double ln_eps, double *ny, double *g,
                                    double *dz, double *dx_skip, double *dD, double *dln_w, double *dln_b)
{
    double mean = 0.0, var = 0.0;
    for (int64_t e = 0; e < E; ++e) {
        const double Ds = (double)pf->D[e] + (double)pb->D[e], xe = xd ? xd[e] : (double)x[e];
        ny[e] = sf[e] + sb[e] + Ds * xe;
        mean += ny[e];
    }
    mean /= (double)E;
    for (int64_t e = 0; e < E; ++e) {
        const double d = ny[e] - mean;
        var += d * d;
    }
    const double r = 1.0 / sqrt(var / (double)E + ln_eps);
    double m1 = 0.0, m2 = 0.0;
    for (int64_t e = 0; e < E; ++e) {
        ny[e] = (ny[e] - mean) * r;
        const double ze = (double)z[e], de = (double)dout[e], sg = sigmoid(ze);
        const double o = (double)ln_b[e] + ny[e] * (double)ln_w[e];
        const double go = de * silu(ze);
        dz[e] = de * o * sg * (1.0 + ze * (1.0 - sg));
        dln_w[e] += go * ny[e];
        dln_b[e] += go;
        g[e] = go * (double)ln_w[e];  /* dn, for now */
        m1 += g[e];
        m2 += g[e] * ny[e];
    }
    m1 /= (double)E;
    m2 /= (double)E;
    for (int64_t e = 0; e < E; ++e) {
        const double Ds = (double)pf->D[e] + (double)pb->D[e];
        g[e] = r * (g[e] - m1 - ny[e] * m2);
        dx_skip[e] = g[e] * Ds;
        const double xe = xd ? xd[e] : (double)x[e];
        dD[e] += g[e] * xe;
    }
}

/*
 * Adjoint of one selective scan (the recurrence of fvo_scan).  With k the
 * scan step (t = k forward, t = T-1-k backward), a_k[n] = exp(delta_k A[n]),
 * H_k = a_k H_{k-1} + delta_k B_k u_k and s_k = sum_n C_k[n] H_k[n], the state
 * adjoint lambda_k = dL/dH_k runs backwards in k:
 *   lambda_k[n] = C_k[n] gs_k + a_{k+1}[n] lambda_{k+1}[n]      (lambda_T = 0)
 * and gives
 *   ddelta_k   = sum_n lambda_k[n] (A[n] a_k[n] H_{k-1}[n] + B_k[n] u_k)
 *   du_k      += sum_n lambda_k[n] delta_k B_k[n]
 *   dB_k[n]   += lambda_k[n] delta_k u_k         (summed over channels e)
 *   dC_k[n]   += gs_k H_k[n]                     (summed over channels e)
 *   dA[e, n]  += lambda_k[n] a_k[n] delta_k H_{k-1}[n]
 * dB and dC land in dv[m, R + n] and dv[m, R + N + n].  The states of the
 * forward sweep are kept whole (T*N doubles per channel).  reset (per time t,
 * or NULL) as in fvo_scan: a step with reset[t] set has the decay a_k = 0, so
 * no state and no adjoint cross it, and its decay terms vanish.
 */
static int scan_adjoint(const double *u, const double *delta, const double *v, const double *gs, int64_t B,
                        int64_t T, int64_t E, int64_t N, int64_t R, int64_t NX, const float *A_log, int reverse,
                        const unsigned char *reset, double *du, double *ddelta, double *dv, double *dA)
{
    double *Hs = (double *)malloc((size_t)(T * N) * sizeof(double));
    double *lam = (double *)malloc((size_t)N * sizeof(double));
    double *carry = (double *)malloc((size_t)N * sizeof(double));
    if (!Hs || !lam || !carry) { free(Hs); free(lam); free(carry); return -9; }
    for (int64_t b = 0; b < B; ++b)
        for (int64_t e = 0; e < E; ++e) {
            /* forward sweep, keeping every state */
            for (int64_t k = 0; k < T; ++k) {
                const int64_t t = reverse ? T - 1 - k : k, m = b * T + t;
                for (int64_t n = 0; n < N; ++n) {
                    const double A = -exp((double)A_log[e * N + n]);
                    const double prev = k > 0 ? Hs[(k - 1) * N + n] : 0.0;
                    const double a = (reset && reset[t]) ? 0.0 : exp(delta[m * E + e] * A);
                    Hs[k * N + n] = a * prev + delta[m * E + e] * v[m * NX + R + n] * u[m * E + e];
                }
            }
            /* reverse sweep */
            for (int64_t n = 0; n < N; ++n) carry[n] = 0.0;
            for (int64_t k = T - 1; k >= 0; --k) {
                const int64_t t = reverse ? T - 1 - k : k, m = b * T + t;
                const double d = delta[m * E + e], ut = u[m * E + e], g = gs[m * E + e];
                double dd = 0.0, duk = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double A = -exp((double)A_log[e * N + n]);
                    const double a = reset && reset[t] ? 0.0 : exp(A * d);
                    const double Bn = v[m * NX + R + n], Cn = v[m * NX + R + N + n];
                    const double prev = k > 0 ? Hs[(k - 1) * N + n] : 0.0;
                    lam[n] = Cn * g + carry[n];
                    dd += lam[n] * (A * a * prev + Bn * ut);
                    duk += lam[n] * d * Bn;
                    dv[m * NX + R + n] += lam[n] * d * ut;
                    dv[m * NX + R + N + n] += g * Hs[k * N + n];
                    dA[e * N + n] += lam[n] * a * d * prev;
                    carry[n] = a * lam[n];
                }
                ddelta[m * E + e] = dd;
                du[m * E + e] += duk;
            }
        }
    free(Hs); free(lam); free(carry);
    return 0;
}

/*
 * Adjoint of the step size, delta = softplus(q) with q = W_dt v[0:R] + b_dt:
 *   dq = ddelta sigmoid(q);  db_dt[e] += dq;  dW_dt[e, r] += dq v[m, r];
 *   dv[m, r] += sum_e W_dt[e, r] dq.
 */
static void step_size_adjoint(const double *q, const double *ddelta, const double *v, int64_t M, int64_t NX,
                              int64_t R, int64_t E, const float *dt_proj_w, double *dWdt, double *dbdt, double *dv)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t e = 0; e < E; ++e) {
            const double dq = ddelta[m * E + e] * sigmoid(q[m * E + e]);
            dbdt[e] += dq;
            for (int64_t r = 0; r < R; ++r) {
                dWdt[e * R + r] += dq * v[m * NX + r];
                dv[m * NX + r] += (double)dt_proj_w[e * R + r] * dq;
            }
        }
}

/* Adjoint of v = W_x u:  dW_x[o, e] += dv[m, o] u[m, e];  du[m, e] += sum_o W_x[o, e] dv[m, o]. */
static void xproj_adjoint(const double *u, const double *dv, int64_t M, int64_t NX, int64_t E,
                          const float *x_proj_w, double *dWx, double *du)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t o = 0; o < NX; ++o)
            for (int64_t e = 0; e < E; ++e) {
                dWx[o * E + e] += dv[m * NX + o] * u[m * E + e];
                du[m * E + e] += (double)x_proj_w[o * E + e] * dv[m * NX + o];
            }
}

/*
 * Adjoint of fvo_conv_silu (the producer Conv1D + SiLU on the oriented grid's
 * sequence).  With a[r] the pre-activation of position r and gxc = dL/dxc:
 *   da[r]          = gxc[r] silu'(a[r])
 *   d conv_b[e]    = sum_r da[r, e]
 *   d conv_w[e, k] = sum_r da[r, e] x[r - KC + 1 + k, e]
 *   dx[r', e]      = sum_k conv_w[e, k] da[r' + KC - 1 - k, e]   (positions inside the sequence)
 * dx, dcw (E, KC) and dcb (E) are overwritten.
 */
static void conv_silu_adjoint(const float *x, const double *gxc, int64_t B, int64_t h, int64_t w, int64_t E,
                              int axis, const float *conv_w, const float *conv_b, int64_t KC, double *dx,
                              double *dcw, double *dcb)
{
    const int colmajor = axis == FVO_NONE_COLMAJOR || axis == FVO_ROWS;
    const int64_t n = h * w;
    for (int64_t i = 0; i < B * n * E; ++i) dx[i] = 0.0;
    for (int64_t i = 0; i < E * KC; ++i) dcw[i] = 0.0;
    for (int64_t e = 0; e < E; ++e) dcb[e] = 0.0;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t r = 0; r < n; ++r) {
            const int64_t cell = colmajor ? (r % h) * w + r / h : r;
            for (int64_t e = 0; e < E; ++e) {
                double a = (double)conv_b[e];
                for (int64_t k = 0; k < KC; ++k) {
                    const int64_t rr = r + k - (KC - 1);
                    if (rr < 0) continue;
                    const int64_t cc = colmajor ? (rr % h) * w + rr / h : rr;
                    a += (double)conv_w[e * KC + k] * (double)x[(b * n + cc) * E + e];
                }
                const double sg = sigmoid(a);
                const double da = gxc[(b * n + cell) * E + e] * sg * (1.0 + a * (1.0 - sg));
                dcb[e] += da;
                for (int64_t k = 0; k < KC; ++k) {
                    const int64_t rr = r + k - (KC - 1);
                    if (rr < 0) continue;
                    const int64_t cc = colmajor ? (rr % h) * w + rr / h : rr;
                    dcw[e * KC + k] += da * (double)x[(b * n + cc) * E + e];
                    dx[(b * n + cc) * E + e] += (double)conv_w[e * KC + k] * da;
                }
            }
        }
}

/*
 * The whole backward pass.  Inputs as fvo_layer plus dout (shaped like x).
 * Outputs dx, dz (shaped like x) and the gradients of both directions'
 * parameters (overwritten).  ln_w == NULL: no LayerNorm; otherwise the layer
 * has the post-SSM LayerNorm (ln_w, ln_b, ln_eps) and its weight and bias
 * gradients go to dln_w, dln_b (E each, overwritten).  pool_scale as in
 * fvo_layer.  The pool's adjoint spreads du of a scan position over its
 * cells: dx[b, cell, e] = dx_skip + pool_scale du[b, t(cell), e] / P (P = 1
 * unpooled; the fixed row length for masked tokens).  local_window = L > 0:
 * the layer of fvo_layer with LBMamba's local backward scan, which runs on
 * the forward direction's x_proj, dt_proj and A_log with a reset at every t
 * with t mod L = L - 1; the gradients of those shared parameters are the sums
 * of both scans' contributions and go to the forward direction's gradients,
 * while the backward direction's x_proj_w, dt_proj_w, dt_proj_b and A_log
 * gradients are zero (the layer does not read them) and its D gradient is dD
 * as usual.  conv_w != NULL: x is the Conv1D's input as in
 * fvo_layer; the layer's adjoint with respect to its x (the Conv1D's output)
 * goes through conv_silu_adjoint into dx, and the conv's weight and bias
 * gradients into dconv_w (E, conv_k) and dconv_b (E).  Returns 0, -2,
 * -3 or -9 as fvo_layer.
 */
int fvo_layer_bwd(const float *x, const float *z, const float *dout, const fvo_dir *pf, const fvo_dir *pb,
                  int64_t B, int64_t h, int64_t w, int64_t E, int64_t N, int64_t R, int64_t K, int axis,
                  const int32_t *idx, double *dx, double *dz, fvo_dir_grad *gf, fvo_dir_grad *gb,
                  fvo_bwd_stages *st, const float *ln_w, const float *ln_b, double ln_eps, double *dln_w,
                  double *dln_b, double pool_scale, int64_t local_window, const float *conv_w,
                  const float *conv_b, int64_t conv_k, double *dconv_w, double *dconv_b)
{
    int64_t T, P;
    const int masked = idx != NULL;
    if (axis < 0 || axis > 3 || (masked && axis > FVO_ROWS)) return -2;
    seq_shape(axis, h, w, &T, &P);
    const int64_t NX = R + 2 * N, M = B * T, ntok = masked ? B * K : B * h * w;
    const size_t me = (size_t)(M * E) * sizeof(double), mx = (size_t)(M * NX) * sizeof(double);
    fvo_dir pl = *pf; /* the local scan: the forward set with the backward D */
    pl.D = pb->D;
    const fvo_dir *pd[2] = {pf, local_window > 0 ? &pl : pb};
    fvo_dir_grad *gd[2] = {gf, gb};
    unsigned char *reset = NULL;
    int rc = 0;

    double *u = (double *)malloc(me), *gs = (double *)calloc((size_t)(M * E), sizeof(double));
    double *du = (double *)calloc((size_t)(M * E), sizeof(double)), *dd = (double *)malloc(me);
    double *g = (double *)malloc((size_t)E * sizeof(double)), *ny = (double *)malloc((size_t)E * sizeof(double));
    double *dxs = (double *)malloc((size_t)(ntok * E) * sizeof(double));
    double *dD = (double *)calloc((size_t)E, sizeof(double));
    double *xc = conv_w ? (double *)malloc((size_t)(ntok * E) * sizeof(double)) : NULL;
    double *dxc = conv_w ? (double *)malloc((size_t)(ntok * E) * sizeof(double)) : NULL;
    double *v[2], *q[2], *dl[2], *s[2], *dv[2];
    int32_t *rows = masked ? (int32_t *)malloc((size_t)(B * K) * sizeof(int32_t)) : NULL;
    for (int d = 0; d < 2; ++d) {
        v[d] = (double *)malloc(mx); q[d] = (double *)malloc(me); dl[d] = (double *)malloc(me);
        s[d] = (double *)malloc(me); dv[d] = (double *)calloc((size_t)(M * NX), sizeof(double));
    }
    if (!u || !gs || !du || !dd || !g || !ny || !dxs || !dD || (masked && !rows) || (conv_w && (!xc || !dxc))) {
        rc = -9;
        goto done;
    }
    if (conv_w && masked) conv_silu_masked(x, B, K, E, conv_w, conv_b, conv_k, xc);
    else if (conv_w) fvo_conv_silu(x, B, h, w, E, axis, conv_w, conv_b, conv_k, xc);
    if (ln_w)
        for (int64_t e = 0; e < E; ++e) dln_w[e] = dln_b[e] = 0.0;
    for (int d = 0; d < 2; ++d)
        if (!v[d] || !q[d] || !dl[d] || !s[d] || !dv[d]) { rc = -9; goto done; }
    if (local_window > 0) {
        reset = (unsigned char *)malloc((size_t)T);
        if (!reset) { rc = -9; goto done; }
        for (int64_t t = 0; t < T; ++t) reset[t] = (unsigned char)((t + 1) % local_window == 0);
    }

    /* forward recomputation: pooled input, per-direction v, q, delta, s */
    if (masked) {
        rc = fvo_mask_rows(idx, B, K, h, w, axis, rows);
        if (rc) goto done;
        pool_masked_any(x, xc, rows, B, K, T, P, E, u);
    } else {
        pool_dense_any(x, xc, B, h, w, E, axis, u);
    }
    for (int64_t i = 0; i < M * E; ++i) u[i] *= pool_scale;
    for (int d = 0; d < 2; ++d) {
        fvo_xproj(u, M, E, pd[d]->x_proj_w, NX, v[d]);
        dt_preact(v[d], M, NX, R, pd[d]->dt_proj_w, pd[d]->dt_proj_b, E, q[d]);
        for (int64_t i = 0; i < M * E; ++i) dl[d][i] = softplus(q[d][i]);
        fvo_scan(u, dl[d], v[d], B, T, E, N, R, NX, pd[d]->A_log, d, d == 1 ? reset : NULL, s[d]);
    }

    /* adjoint of the output (gate, skip, repeat): dz, the skip part of dx, dD and gs */
    for (int64_t b = 0; b < B; ++b) {
        const int64_t ncell = masked ? K : h * w;
        for (int64_t c = 0; c < ncell; ++c) {
            int64_t t;
            if (masked) t = rows[b * K + c];
            else t = seq_pos(axis, h, w, c / w, c % w);
            const int64_t off = (b * ncell + c) * E, mt = (b * T + t) * E;
            const double *xco = xc ? xc + off : NULL;
            if (ln_w)
                output_token_adjoint_ln(s[0] + mt, s[1] + mt, x + off, xco, z + off, dout + off, pf, pb, E, ln_w,
                                        ln_b, ln_eps, ny, g, dz + off, dxs + off, dD, dln_w, dln_b);
            else
                output_token_adjoint(s[0] + mt, s[1] + mt, x + off, xco, z + off, dout + off, pf, pb, E, g,
                                     dz + off, dxs + off, dD);
            for (int64_t e = 0; e < E; ++e) gs[mt + e] += g[e];
        }
    }

    /* adjoints of both directions: scan, step size, x_proj */
    for (int d = 0; d < 2; ++d) {
        fvo_dir_grad *o = gd[d];
        for (int64_t i = 0; i < NX * E; ++i) o->x_proj_w[i] = 0.0;
        for (int64_t i = 0; i < E * R; ++i) o->dt_proj_w[i] = 0.0;
        for (int64_t i = 0; i < E * N; ++i) o->A_log[i] = 0.0;
        for (int64_t e = 0; e < E; ++e) o->dt_proj_b[e] = 0.0;
        rc = scan_adjoint(u, dl[d], v[d], gs, B, T, E, N, R, NX, pd[d]->A_log, d, d == 1 ? reset : NULL, du, dd,
                          dv[d], o->A_log);
        if (rc) goto done;
        /* dA -> dA_log: A = -exp(A_log), so dA/dA_log = A */
        for (int64_t i = 0; i < E * N; ++i) o->A_log[i] *= -exp((double)pd[d]->A_log[i]);
        step_size_adjoint(q[d], dd, v[d], M, NX, R, E, pd[d]->dt_proj_w, o->dt_proj_w, o->dt_proj_b, dv[d]);
        xproj_adjoint(u, dv[d], M, NX, E, pd[d]->x_proj_w, o->x_proj_w, du);
        for (int64_t e = 0; e < E; ++e) o->D[e] = dD[e];
    }
    if (local_window > 0) {
        /* the local scan's parameters are the forward direction's: add its
         * contributions there; the backward set's unused gradients are zero */
        for (int64_t i = 0; i < NX * E; ++i) { gf->x_proj_w[i] += gb->x_proj_w[i]; gb->x_proj_w[i] = 0.0; }
        for (int64_t i = 0; i < E * R; ++i) { gf->dt_proj_w[i] += gb->dt_proj_w[i]; gb->dt_proj_w[i] = 0.0; }
        for (int64_t i = 0; i < E * N; ++i) { gf->A_log[i] += gb->A_log[i]; gb->A_log[i] = 0.0; }
        for (int64_t e = 0; e < E; ++e) { gf->dt_proj_b[e] += gb->dt_proj_b[e]; gb->dt_proj_b[e] = 0.0; }
    }

    /* adjoint of the pool */
    for (int64_t b = 0; b < B; ++b) {
        const int64_t ncell = masked ? K : h * w;
        for (int64_t c = 0; c < ncell; ++c) {
            int64_t t;
            if (masked) t = rows[b * K + c];
            else t = seq_pos(axis, h, w, c / w, c % w);
            const int64_t off = (b * ncell + c) * E, mt = (b * T + t) * E;
            for (int64_t e = 0; e < E; ++e) dx[off + e] = dxs[off + e] + du[mt + e] * pool_scale / (double)P;
        }
    }
    if (conv_w) {
        /* dx holds dL/d(the conv's output): take it through the conv */
        memcpy(dxc, dx, (size_t)(ntok * E) * sizeof(double));
        if (masked) /* along the kept-token sequence, as conv_silu_masked */
            conv_silu_adjoint(x, dxc, B, K, 1, E, FVO_COLS, conv_w, conv_b, conv_k, dx, dconv_w, dconv_b);
        else
            conv_silu_adjoint(x, dxc, B, h, w, E, axis, conv_w, conv_b, conv_k, dx, dconv_w, dconv_b);
    }

    if (st) {
        if (st->gs) memcpy(st->gs, gs, me);
        if (st->du) memcpy(st->du, du, me);
        if (st->dv_f) memcpy(st->dv_f, dv[0], mx);
        if (st->dv_b) memcpy(st->dv_b, dv[1], mx);
    }

done:
    free(u); free(gs); free(du); free(dd); free(g); free(ny); free(dxs); free(dD); free(rows); free(reset);
    free(xc); free(dxc);
    for (int d = 0; d < 2; ++d) { free(v[d]); free(q[d]); free(dl[d]); free(s[d]); free(dv[d]); }
    return rc;
}
