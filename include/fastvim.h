/*
 * fastvim.h -- C ABI of the MI355X (gfx950) pooled bidirectional
 * selective-scan layer of FastVim (Fast Vision Mamba, arXiv 2502.00594).
 *
 * What one call computes (FastVim summary page, gptget.net, section 方法详解,
 * bullets 1-6; Pith review of 2502.00594, field "key_machinery"; Vim article,
 * ijyty.com, section 2.1):
 *
 *   1. mean-pool the post-Conv1D token grid x (B, h, w, E) along one spatial
 *      axis: COLS averages over w and scans the h rows, ROWS (the transposed
 *      grid of the next block) averages over h and scans the w columns:
 *          u[b, t, e] = (1/P) * sum_p x[b, (t, p), e]
 *   2. per direction d in {fwd, bwd}: v = x_proj_w^d u split as
 *      [delta_lowrank (R) | B_t (N) | C_t (N)], and the step size
 *          Delta[b, t, e] = softplus(dt_proj_w^d[e, :] . delta_lowrank + dt_proj_b^d[e])
 *   3. zero-order-hold decay and selective scan, forward over t = 0..T-1 and
 *      backward over t = T-1..0, with A^d = -exp(A_log^d) and H = 0 at start:
 *          H[e, n] <- exp(Delta * A^d[e, n]) * H[e, n] + Delta * B_t[n] * u[b, t, e]
 *          s^d[b, t, e] = sum_n C_t[n] * H[e, n]
 *   4. repeat back over the pooled axis, add the skip, sum the directions and
 *      gate:
 *          out[b, i, j, e] = (s^fwd[b, t, e] + s^bwd[b, t, e]
 *                             + (D^fwd[e] + D^bwd[e]) * x[b, i, j, e]) * silu(z[b, i, j, e])
 *      with t = i (COLS) or t = j (ROWS).  Every output is written once.
 *
 * Masked (FastMaskVim, same page, bullet 6): x, z and out hold only the K kept
 * tokens of each image, (B, K, E), and mask_idx (B, K) gives each kept
 * token's flat index q = i*w + j into the h x w grid.  A row sums its kept
 * tokens and divides by the fixed row length P (w for COLS, h for ROWS); an
 * empty row pools to zero and is still scanned; out[b, k] uses the scan
 * output of the token's own row.
 *
 * Unpooled (FASTVIM_POOL_NONE_*): the same layer with no pooling, the scan
 * running over all T = h*w tokens in row-major (t = i*w + j) or column-major
 * (t = j*h + i) order.  It exists to measure what pooling saves.
 *
 * Conventions for every entry point:
 *   - device pointers (x, z, out, mask_idx, parameters, workspace) are HIP
 *     device memory owned by the caller; the library keeps no pointer after a
 *     call returns and holds no memory between calls.  A layer call given a
 *     NULL workspace takes its scratch from the stream-ordered allocator
 *     instead (hipMallocAsync before its kernels, hipFreeAsync after them,
 *     both on the call's stream);
 *   - stream is a hipStream_t passed as void* (NULL = the legacy default
 *     stream); work is only enqueued on it, nothing synchronises the host;
 *   - the return value is FASTVIM_OK (0) or a negative fastvim_status; on an
 *     argument error nothing has been launched.  No exception crosses the ABI;
 *   - calls that share a workspace must not overlap in time (the workspace
 *     holds the pooled tokens, projections and scan outputs of a call).
 */
#ifndef FASTVIM_H
#define FASTVIM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FASTVIM_ABI_VERSION 13

typedef enum fastvim_status {
    FASTVIM_OK = 0,
    FASTVIM_ERR_NULL = -1,        /* a required pointer is NULL */
    FASTVIM_ERR_DIMS = -2,        /* a size is out of range or inconsistent */
    FASTVIM_ERR_UNSUPPORTED = -3, /* valid shape this build does not run (N != 16, R > 64, E > 4096, E % vec,
                                     an image of 2^31 elements or more) */
    FASTVIM_ERR_ALIGN = -4,       /* x, z, out, x_proj_w not 16-byte aligned; workspace not 256-byte; others not 4-byte */
    FASTVIM_ERR_OVERLAP = -5,     /* out overlaps x or z, or the workspace overlaps an input or output */
    FASTVIM_ERR_WORKSPACE = -6,   /* workspace smaller than fastvim_ssm_workspace_bytes, or NULL where a
                                     call needs the caller's (stages, exports, device errors) */
    FASTVIM_ERR_HIP = -7,         /* a HIP launch, copy or stream-ordered allocation reported an error */
    FASTVIM_ERR_ARG = -8,         /* bad enum value, stage id or export id, or mask_idx given with K = 0 */
    /* reported by fastvim_get_device_error only, for the last call that ran
     * its kernels with the workspace: */
    FASTVIM_ERR_BAD_INDEX = -9,   /* FASTVIM_FLAG_CHECK_IDX found an invalid mask index */
    FASTVIM_ERR_DEVICE_WAIT = -10, /* a wait inside the single launch gave up; its outputs are invalid */
    FASTVIM_ERR_SCRATCH = -11     /* fastvim_ssm_fwd_noalloc: the layer needs more than
                                     FASTVIM_NOALLOC_SCRATCH_BYTES of scratch */
} fastvim_status;

/* Element type of x, z and out.  Parameters are always fp32; all arithmetic
 * (pooled sums, projections, scan state, epilogue) is fp32.  bf16 outputs are
 * rounded to nearest even. */
typedef enum fastvim_dtype { FASTVIM_F32 = 0, FASTVIM_BF16 = 1 } fastvim_dtype;

typedef enum fastvim_pool_axis {
    FASTVIM_POOL_COLS = 0,          /* mean over w, scan over h (T = h, P = w) */
    FASTVIM_POOL_ROWS = 1,          /* mean over h, scan over w (T = w, P = h): the transposed grid */
    FASTVIM_POOL_NONE_ROWMAJOR = 2, /* no pooling, T = h*w, t = i*w + j */
    FASTVIM_POOL_NONE_COLMAJOR = 3  /* no pooling, T = h*w, t = j*h + i */
} fastvim_pool_axis;

/* Problem sizes.  B images of an h x w token grid with E channels (d_inner),
 * state size N, dt rank R.  K > 0 selects the masked layer with K kept tokens
 * per image (then mask_idx is required and pool_axis must be COLS or ROWS);
 * K = 0 is the dense layer.  B = 0 is a valid empty call (returns FASTVIM_OK,
 * launches nothing).  Limits of this build: N = 16, 1 <= R <= 64,
 * E <= 4096 and E % 4 == 0 (fp32) or E % 8 == 0 (bf16); masked grids
 * h*w <= 16384; unpooled T = h*w <= 2^31 - 1. */
typedef struct fastvim_dims {
    int64_t B, h, w, E, N, R, K;
    int32_t io_dtype; /* fastvim_dtype */
    int32_t reserved; /* set to 0 */
} fastvim_dims;

/* One scan direction's parameters, all fp32, contiguous, row-major device
 * memory, 4-byte aligned (x_proj_w 16-byte aligned):
 *   x_proj_w (R + 2N, E): rows [0, R) give the low-rank step input, rows
 *                         [R, R+N) give B_t, rows [R+N, R+2N) give C_t;
 *   dt_proj_w (E, R), dt_proj_b (E), A_log (E, N) with A = -exp(A_log), D (E). */
typedef struct fastvim_dir_params {
    const float *x_proj_w;
    const float *dt_proj_w;
    const float *dt_proj_b;
    const float *A_log;
    const float *D;
} fastvim_dir_params;

typedef struct fastvim_params {
    fastvim_dir_params fwd; /* forward scan (t ascending) */
    fastvim_dir_params bwd; /* backward scan (t descending) */
    void *workspace;        /* device scratch, >= fastvim_ssm_workspace_bytes, 256-byte aligned, or NULL
                               (fastvim_ssm_fwd, fastvim_ssm_fwd_stages and fastvim_ssm_bwd then allocate
                               and free it on the call's stream) */
    size_t workspace_bytes;
    uint32_t flags;         /* FASTVIM_FLAG_* bits, else 0 */
    uint32_t tuning;        /* 0, or FASTVIM_TUNING_* fields (measurement and tests) */
    /* Post-SSM LayerNorm, used with FASTVIM_FLAG_POST_NORM only: per-channel
     * scale and shift (E) fp32, 16-byte aligned, and eps > 0. */
    const float *ln_weight;
    const float *ln_bias;
    float ln_eps;
    /* Factor on the pooled tokens, used with FASTVIM_FLAG_POOL_SCALE only
     * (the layer as defined has 1). */
    float pool_scale;
    /* Producer Conv1D, used with FASTVIM_FLAG_CONV only: depthwise taps
     * (E, FASTVIM_CONV_TAPS) fp32, oldest tap first, 16-byte aligned, and bias
     * (E) fp32. */
    const float *conv_w;
    const float *conv_b;
    /* Pooled tokens kept from the forward call for the backward call (as
     * training keeps a layer's activations), or NULL: pooled layers only,
     * (B, T, E) fp32, 16-byte aligned.  fastvim_ssm_fwd (and its stages) then
     * writes the pooled tokens u here instead of into the workspace, and
     * fastvim_ssm_bwd reads them from here instead of pooling x again, so its
     * first pass reads z and dout only.  The caller keeps the buffer between
     * the two calls and passes the same x, mask, pool axis and pool scale to
     * both; the library does not check that the contents match.  Errors: FASTVIM_ERR_ARG
     * (unpooled layer), FASTVIM_ERR_ALIGN, FASTVIM_ERR_OVERLAP (it overlaps
     * an input, an output or the workspace). */
    float *saved_u;
} fastvim_params;

/* params.flags bits.  By default a dense pooled layer (COLS or ROWS, no mask)
 * whose images hold at least 8 MiB of x each runs as one pipelined launch,
 * preceded by a one-block launch that resets its counters in the workspace;
 * every other layer runs as its stage kernels (the ones fastvim_ssm_stage
 * runs).  FASTVIM_FLAG_STAGED runs every layer as its stage kernels;
 * FASTVIM_FLAG_FUSED runs every dense pooled layer as the single launch,
 * whatever its size.  Both paths give the same results within rounding.
 * Setting both bits is FASTVIM_ERR_ARG.  The single launch pipelines images:
 * an image's scans start LS images after its pooling and its outputs LE
 * images after; both follow the image size (LE = 180 MB / bytes of x per
 * image, LS = max(3, LE / 4)), and params.tuning overrides them. */
#define FASTVIM_FLAG_STAGED 1u
#define FASTVIM_FLAG_FUSED 2u

/* params.tuning: measurement and test settings of the single launch, 0 for
 * the defaults.  Bits 0-7: LS (0 = automatic), bits 8-15: LE (0 =
 * automatic; raised to LS if smaller).  FASTVIM_TUNING_POLL1 makes every
 * wait inside the single launch give up after one poll, so that tests can
 * exercise the give-up path (the kernel then finishes with invalid outputs,
 * NaN in every output block that follows a failed wait, and
 * fastvim_get_device_error reports FASTVIM_ERR_DEVICE_WAIT).  Other bits,
 * except FASTVIM_TUNING_BWD_GROUPS and FASTVIM_TUNING_SCAN_OUT below:
 * FASTVIM_ERR_ARG. */
#define FASTVIM_TUNING_LS(n) ((uint32_t)(n) & 0xffu)
#define FASTVIM_TUNING_LE(n) (((uint32_t)(n) & 0xffu) << 8)
#define FASTVIM_TUNING_POLL1 (1u << 16)
/* Bits 20-25: image groups of fastvim_ssm_bwd (0 = automatic, 1 = none,
 * at most 32; see fastvim_ssm_bwd).  The forward calls ignore them, the
 * backward call takes no other tuning bits. */
#define FASTVIM_TUNING_BWD_GROUPS(n) (((uint32_t)(n) & 0x3fu) << 20)
/* Bits 26-27: how the stage kernels of a pooled layer with a scan of at most
 * 64 steps, without the post-SSM LayerNorm and without the Conv1D computed
 * on load, run their scan and output stages: 0 = automatic (one launch for
 * masked layers and for images of at most 1024 tokens, two launches
 * otherwise), 1 = two launches, 2 = one launch; 3 is FASTVIM_ERR_ARG.  The
 * results are the same either way, bit for bit. */
#define FASTVIM_TUNING_SCAN_OUT(n) (((uint32_t)(n) & 0x3u) << 26)

/* FASTVIM_FLAG_POST_NORM adds the post-SSM LayerNorm between the skip and the
 * gate (FastVim summary page, section 方法详解, bullet 5: LayerNorm after the
 * repeat and the skip connection; the Pith review on 2502.00594: the
 * post-SSM LayerNorm of VMamba, on the SSM output).  Per token, over its E
 * channels: y = s_fwd + s_bwd + (D_fwd + D_bwd) x,
 *   out = ((y - mean(y)) / sqrt(var(y) + ln_eps) * ln_weight + ln_bias) * silu(z)
 * with the population variance.  The single launch takes the norm for dense
 * pooled layers with E / V <= 128 (V = 4 for fp32, 8 for bf16 elements per 16
 * bytes): by default for COLS layers (the size rule above), with
 * FASTVIM_FLAG_FUSED for ROWS too; other layers run the norm in their stage
 * epilogue (FASTVIM_FLAG_FUSED then falls back to the stage kernels).
 * Errors: FASTVIM_ERR_NULL (ln_weight or ln_bias NULL), FASTVIM_ERR_ALIGN (not
 * 16-byte aligned), FASTVIM_ERR_ARG (ln_eps not > 0 or not finite). */
#define FASTVIM_FLAG_POST_NORM 4u

/* FASTVIM_FLAG_CONV fuses the producer side into the layer: x is the input of
 * the depthwise causal Conv1D + SiLU that makes the layer's x (FastVim summary
 * page, section 方法详解, bullets 1-2: the grid is pooled after the Conv1D;
 * Vim article, section 2.1: conv1d, then the SSM).  Along the oriented grid's
 * sequence r -- row-major r = i*w + j for COLS, column-major r = j*h + i for
 * ROWS (the transposed grid) -- with zeros before its start,
 *   x_conv[r, e] = silu(conv_b[e] + sum_{k<4} conv_w[e, k] * x[r - 3 + k, e])
 * and the layer runs on x_conv.  Dense pooled layers compute it where their
 * pool and output stages read x, so it is never written: the single launch
 * does so on both axes, with or without FASTVIM_FLAG_POST_NORM (and without
 * FASTVIM_FLAG_LOCAL_BWD), where it would run without the conv; the stage
 * kernels for the other dense layers without the norm.  Masked layers --
 * whose conv runs along the kept tokens in the order given, r = k --
 * unpooled layers and the remaining layers with FASTVIM_FLAG_POST_NORM (on
 * the stage kernels) get x_conv written once into out first (in the I/O
 * element type: bf16 layers round it to bf16), and the layer then runs on it,
 * by the path it would take without the conv; fastvim_ssm_stage returns
 * FASTVIM_ERR_UNSUPPORTED for them.
 * Errors: FASTVIM_ERR_NULL (conv_w or conv_b NULL), FASTVIM_ERR_ALIGN (conv_w
 * not 16-byte aligned, conv_b not 4-byte aligned). */
#define FASTVIM_FLAG_CONV 8u
#define FASTVIM_CONV_TAPS 4

/* FASTVIM_FLAG_LOCAL_BWD replaces the global backward scan by LBMamba's local
 * backward scan (LBMamba article, pswp.cn, 论文创新点 1-2: a light backward
 * scan run within subsequences inside the forward selective scan, on the
 * same inputs, instead of a second global scan).  s_bwd is then the scan
 * over t descending with the forward direction's projection, step size and
 * decay, its state starting from zero at the top of every window of
 * FASTVIM_LOCAL_WINDOW steps aligned at t = 0 (at every t with
 * t mod FASTVIM_LOCAL_WINDOW = FASTVIM_LOCAL_WINDOW - 1); the layer is
 *   out = (s_fwd + s_bwd + (D_fwd + D_bwd) x) silu(z)
 * as before.  Of params.bwd only D is read (the other four may be NULL); pass
 * D_bwd = 0 for a single skip.  Any pooled, masked or unpooled layer, and
 * combines with the other options.  Dense pooled layers take the single
 * launch under the same rules as without it (the size rule by default,
 * FASTVIM_FLAG_FUSED to force it), except with FASTVIM_FLAG_POST_NORM; other
 * layers run as stage kernels.  The backward pass takes it for pooled layers:
 * the gradients of the shared x_proj_w, dt_proj_w, dt_proj_b and A_log sum
 * both scans' contributions and go to grads->fwd, grads->bwd receives zeros
 * for those four (its buffers are still required) and dD as usual. */
#define FASTVIM_FLAG_LOCAL_BWD 16u
#define FASTVIM_LOCAL_WINDOW 16

/* FASTVIM_FLAG_POOL_SCALE multiplies the pooled tokens by params.pool_scale:
 * u = pool_scale * (row sum) / P, for the projections and the scans, while
 * the skip term reads x unscaled.  It is the constant the MAE transfer
 * recipe applies when pooling in fine-tuning and linear probing of a model
 * pre-trained on 75 %-masked inputs, 0.25 there (Pith review on 2502.00594,
 * referee report, major comments: the MAE experiments): with the fixed
 * normaliser P, pooled rows of a masked image are about a quarter of those of
 * a full one.  Pooled layers (dense or masked) and every option and path; the
 * backward pass takes it too (the pool's adjoint becomes pool_scale / P).
 * Errors: FASTVIM_ERR_ARG for an unpooled layer or a pool_scale that is not
 * finite. */
#define FASTVIM_FLAG_POOL_SCALE 32u

/* FASTVIM_FLAG_CHECK_IDX (masked layers) records, on the device, whether any
 * mask index was invalid (outside [0, h*w), or repeated within its image);
 * fastvim_get_device_error then reports FASTVIM_ERR_BAD_INDEX.  The check
 * itself always runs (an invalid index is never dereferenced, its tokens get
 * NaN, see fastvim_ssm_fwd); the flag adds the error report.  Forward and
 * backward calls; ignored for dense layers. */
#define FASTVIM_FLAG_CHECK_IDX 64u

/* Bytes of workspace a call with these sizes needs (0 if the sizes are
 * invalid).  Dense pooled layers need 4 * B * T * (3E + 2(R + 2N)) bytes plus
 * 4 * (2 + 2B) bytes of counters and alignment; unpooled layers hold the per-token projections and scan outputs
 * (at B = 128, h = w = 128, E = 384 about 7.2 GB).  The workspace begins
 * with the call's status word (see fastvim_get_device_error). */
size_t fastvim_ssm_workspace_bytes(const fastvim_dims *dims, int pool_axis);

/* The layer.  x, z, out: (B, h, w, E) dense or (B, K, E) masked, contiguous,
 * element type dims->io_dtype, 16-byte aligned; out must not overlap x or z.
 * mask_idx: (B, K) int32 flat grid indices (masked only, else NULL).  Every
 * index must lie in [0, h*w) and be unique within its image; a token whose
 * index breaks this gets NaN in every output channel (and is counted, see
 * FASTVIM_EXPORT_BAD_TOKENS), the other tokens of that image pool as if it
 * were absent.  Enqueues its kernels on stream and returns. */
int fastvim_ssm_fwd(const void *x, const void *z, const fastvim_params *params, const fastvim_dims *dims,
                    int pool_axis, const int32_t *mask_idx, void *out, void *stream);

/* The layer, as fastvim_ssm_fwd, also copying its intermediate results into
 * caller buffers in the same call (for stage-by-stage checks; works with a
 * NULL workspace too, the copies are enqueued before it is freed).  Each
 * destination is device memory, 4-byte aligned, or NULL to skip it:
 *   u_out        (B, T, E) fp32 pooled tokens (pooled layers only, else FASTVIM_ERR_ARG)
 *   s_f_out      (B, T, E) fp32 forward scan output
 *   s_b_out      (B, T, E) fp32 backward scan output
 *   row_of_token (B, K) int32 scan row (COLS) or column (ROWS) of each kept token,
 *                -1 for an invalid index (masked layers only, else FASTVIM_ERR_ARG)
 * A destination must not overlap x, z, out, the workspace or another
 * destination (FASTVIM_ERR_OVERLAP). */
int fastvim_ssm_fwd_stages(const void *x, const void *z, const fastvim_params *params, const fastvim_dims *dims,
                           int pool_axis, const int32_t *mask_idx, void *out, void *stream, float *u_out,
                           float *s_f_out, float *s_b_out, int32_t *row_of_token);

/* Errors found on the device by the last call that ran its kernels with
 * params->workspace (forward or backward): FASTVIM_ERR_DEVICE_WAIT if a wait
 * inside the single launch gave up (its outputs are then invalid; a broken
 * invariant, never expected), else FASTVIM_ERR_BAD_INDEX if that call had
 * FASTVIM_FLAG_CHECK_IDX and found an invalid mask index, else FASTVIM_OK.
 * Reads the status word at the start of the workspace: synchronises stream
 * (waits for the work enqueued on it).  FASTVIM_ERR_WORKSPACE for a NULL
 * workspace (a call that allocated its own keeps no status). */
int fastvim_get_device_error(const fastvim_params *params, void *stream);

/* The layer for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid device allocation.  The same
 * arguments and results as fastvim_ssm_fwd, except that params->workspace and
 * params->workspace_bytes are not read: the scratch is a fixed buffer of
 * FASTVIM_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held from
 * the library's first use on that GPU until the process ends.  The call
 * allocates nothing (no hipMalloc, hipMallocAsync or hipFree), also not on
 * its first call on a GPU, which only looks up that GPU's buffer.  Layers whose
 * fastvim_ssm_workspace_bytes exceeds the buffer get FASTVIM_ERR_SCRATCH
 * (every pooled layer of this build's workloads fits; unpooled layers of
 * large grids do not).  All calls on one GPU share its buffer, which keeps
 * the last call's intermediates: calls that overlap in time on one GPU
 * (different streams, different threads) race and give wrong results, so
 * the caller serialises them, e.g. on one stream.  Every counter the layer
 * needs zeroed is cleared by the call itself, by a kernel.  No export or
 * device-error read reaches this buffer. */
#define FASTVIM_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)
int fastvim_ssm_fwd_noalloc(const void *x, const void *z, const fastvim_params *params, const fastvim_dims *dims,
                            int pool_axis, const int32_t *mask_idx, void *out, void *stream);

/* The layer's stages, for timing and inspection.  fastvim_ssm_fwd runs
 * ROWS (masked only), POOL (pooled only), PROJ, SCAN and EPILOGUE in that
 * order; fastvim_ssm_stage runs one of them with the same arguments, reading
 * what earlier stages left in the workspace.  Running a stage before the
 * stages it depends on gives unspecified (but in-bounds) results. */
typedef enum fastvim_stage {
    FASTVIM_STAGE_ROWS = 0,     /* masked: validate mask_idx, row of every kept token */
    FASTVIM_STAGE_POOL = 1,     /* u = pooled tokens */
    FASTVIM_STAGE_PROJ = 2,     /* v = x_proj of u (both directions) */
    FASTVIM_STAGE_SCAN = 3,     /* step sizes, decays and both scans -> s_fwd, s_bwd */
    FASTVIM_STAGE_EPILOGUE = 4  /* repeat + skip + gate -> out */
} fastvim_stage;

int fastvim_ssm_stage(int stage, const void *x, const void *z, const fastvim_params *params,
                      const fastvim_dims *dims, int pool_axis, const int32_t *mask_idx, void *out,
                      void *stream);

/* Copy one intermediate result of the last call that used this workspace into
 * dst (device memory, dst_bytes large enough), enqueued on stream:
 *   U           (B, T, E)        fp32 pooled tokens (pooled layers only; from saved_u when given)
 *   XDBL        (B, T, 2, R+2N)  fp32 x_proj outputs, [.., 0, :] fwd, [.., 1, :] bwd
 *   S_FWD/S_BWD (B, T, E)        fp32 scan outputs of each direction
 *   ROWS        (B, K)           int32 row (COLS) or column (ROWS) of each kept token, -1 if invalid
 *   BAD_TOKENS  (B)              int32 number of invalid mask entries per image
 *   STATUS      (1)              uint32, 0 normally; bit 0 set if a wait inside the single-launch
 *                                kernel gave up after its bounded polling (results then invalid)
 * Returns FASTVIM_ERR_ARG for an export the layer does not have. */
typedef enum fastvim_export {
    FASTVIM_EXPORT_U = 0,
    FASTVIM_EXPORT_XDBL = 1,
    FASTVIM_EXPORT_S_FWD = 2,
    FASTVIM_EXPORT_S_BWD = 3,
    FASTVIM_EXPORT_ROWS = 4,
    FASTVIM_EXPORT_BAD_TOKENS = 5,
    FASTVIM_EXPORT_STATUS = 6
} fastvim_export;

int fastvim_ssm_export(const fastvim_params *params, const fastvim_dims *dims, int pool_axis, int what,
                       void *dst, size_t dst_bytes, void *stream);

/* Size in bytes of an export (0 if the layer does not have it). */
size_t fastvim_ssm_export_bytes(const fastvim_dims *dims, int pool_axis, int what);

/* ------------------------------------------------------------------ backward
 * Gradients of the layer, for training (FastVim summary page, section 实验结果:
 * the pooled layer is trained from scratch and in MAE pre-training).  For a
 * scalar loss L whose gradient with respect to out is dout, fastvim_ssm_bwd
 * computes dx = dL/dx, dz = dL/dz and dL/dparameter for both directions, by
 * the chain rule through the forward steps in reverse:
 *   g     = dout * silu(z)                          (dL/dy, y the pre-gate value)
 *   dz    = dout * y * sigmoid(z) * (1 + z * (1 - sigmoid(z)))
 *   gs    = g summed over the cells repeated from each scan position (the
 *           repeat's adjoint), the adjoint input of both scans
 *   each scan's adjoint, run backwards in time from the recomputed forward
 *           states, gives du and dL/d(delta_lowrank, B_t, C_t), d dt_proj_w,
 *           d dt_proj_b (through softplus) and d A_log (A = -exp(A_log))
 *   d x_proj_w = sum over pooled tokens of dL/dv u^T, du += x_proj_w^T dL/dv
 *   dD_fwd = dD_bwd = sum over all cells of g * x
 *   dx    = g * (D_fwd + D_bwd) + du[b, t(cell), :] / P   (the pool's adjoint)
 * The forward pass is recomputed inside the call (pooled tokens, projections,
 * states), so only x, z and dout are needed; with params->saved_u the pooled
 * tokens come from the forward call instead.  Two passes stream the grid: the
 * first reads x (unless saved_u is given), z and dout and pools u and gs; the
 * second reads x, z and dout again, writes dx and dz and sums dD.  Arithmetic
 * is fp32; every sum has a fixed order (no atomics), so results are
 * run-to-run identical.
 *
 * With FASTVIM_FLAG_POST_NORM (params->ln_weight, ln_bias, ln_eps as for the
 * forward call; FastVim summary page, section 方法详解, bullet 5) the adjoint
 * of the output goes through the LayerNorm: with y as above, its mean and
 * population variance over the token's E channels, r = 1 / sqrt(var + eps),
 * n = (y - mean) r and o = n ln_weight + ln_bias,
 *   dz    = dout * o * sigmoid(z) * (1 + z * (1 - sigmoid(z)))
 *   d ln_weight = sum over all cells of dout silu(z) n,  d ln_bias = sum of dout silu(z)
 *   dn    = dout silu(z) ln_weight,   g = r (dn - mean(dn) - n mean(dn n))
 * and g takes the place of dL/dy above.  Since g needs the scan outputs, the
 * call first recomputes the pooled tokens (unless saved_u is given), the
 * projections and both scans; its first pass then reads x, z and dout, writes
 * dz and leaves g in dx, which the second pass turns into dx (for bf16 I/O g
 * is rounded to bf16 there).  grads->ln_weight and ln_bias receive the norm's
 * gradients.
 *
 * With FASTVIM_FLAG_LOCAL_BWD the backward scan is LBMamba's local one (see
 * the flag): its adjoint runs within each window, on the forward direction's
 * parameters, and nothing carries across a window's reset.
 *
 * With FASTVIM_FLAG_CONV (params->conv_w, conv_b as for the forward call) x
 * is the Conv1D's input and dx its gradient: with a[r] the conv's
 * pre-activation at sequence position r, dxc the layer's gradient with
 * respect to the conv's output and da = dxc silu'(a),
 *   dx[r] = sum_k conv_w[k] da[r + 3 - k],  d conv_w[k] = sum_r da[r] x[r - 3 + k],
 *   d conv_b = sum_r da[r]
 * (per channel, along the oriented grid's sequence, or along the kept tokens
 * of a masked layer), written to grads->conv_w and conv_b.  Dense layers
 * without the LayerNorm: the first pass pools x_conv (unless saved_u is
 * given) and the second computes x_conv and da where it reads x, so neither
 * is written.  Dense layers with the LayerNorm: the pool and the norm's first
 * pass compute x_conv where they read x, and the conv's adjoint takes the
 * norm's second pass, forming dL/dx_conv from the norm's gradient as it
 * reads it, in place on dx (its scratch the workspace).  Masked layers (and
 * dense ones with the norm too small for that scratch): x_conv is written
 * into dz first, the layer's backward pass runs on it (reading each cell's
 * x_conv before writing its dz) and leaves dL/dx_conv in dx, and the conv's
 * adjoint then runs in place on dx, its scratch the workspace (bf16 layers
 * round x_conv and dL/dx_conv to bf16 there).
 *
 * Supported: pooled layers (COLS or ROWS, dense or masked) whose scan has at
 * most 720, 512, 384 or 288 steps at dt rank R <= 16, 32, 48 or 64 (the scan
 * adjoint holds the sequence's x_proj rows in one workgroup's LDS), within
 * the limits of the forward call, with or without
 * FASTVIM_FLAG_POST_NORM (then E <= 2048), FASTVIM_FLAG_POOL_SCALE,
 * FASTVIM_FLAG_LOCAL_BWD and FASTVIM_FLAG_CONV, in any combination;
 * FASTVIM_ERR_UNSUPPORTED for unpooled layers, longer scans, the LayerNorm
 * with E > 2048, the cases the forward call does not take, and
 * FASTVIM_FLAG_FUSED (0 and FASTVIM_FLAG_STAGED run the same kernels). */

/* Gradients of one direction's parameters: fp32 device buffers shaped like
 * the parameters, 4-byte aligned, overwritten by the call. */
typedef struct fastvim_dir_grads {
    float *x_proj_w;  /* (R + 2N, E) */
    float *dt_proj_w; /* (E, R) */
    float *dt_proj_b; /* (E) */
    float *A_log;     /* (E, N) */
    float *D;         /* (E) */
} fastvim_dir_grads;

typedef struct fastvim_grads {
    fastvim_dir_grads fwd, bwd;
    /* With FASTVIM_FLAG_POST_NORM: the LayerNorm's weight and bias gradients,
     * (E) fp32 each, 4-byte aligned, overwritten; ignored (may be NULL)
     * otherwise. */
    float *ln_weight;
    float *ln_bias;
    /* With FASTVIM_FLAG_CONV: the Conv1D's weight (E, FASTVIM_CONV_TAPS) and
     * bias (E) gradients, fp32, 4-byte aligned, overwritten; ignored (may be
     * NULL) otherwise. */
    float *conv_w;
    float *conv_b;
} fastvim_grads;

/* Bytes of workspace fastvim_ssm_bwd needs (0 if the sizes are invalid or
 * the backward pass does not support them): about 4 * B * T * (8E + 4(R + 2N))
 * plus per-image and per-chunk partial sums (at B = 128, h = w = 128, E = 384,
 * R = 12: about 530 MB, enough for every image grouping). */
size_t fastvim_ssm_bwd_workspace_bytes(const fastvim_dims *dims, int pool_axis);

/* The backward pass.  x, z, dout, dx, dz: like x of fastvim_ssm_fwd (same
 * shape, element type and 16-byte alignment); params as for the forward call,
 * its workspace at least fastvim_ssm_bwd_workspace_bytes (256-byte aligned);
 * mask_idx as for the forward call (a token with an invalid index gets NaN in
 * dx and dz and takes no part in the pooled sums).  dx, dz, the workspace and
 * the ten gradient buffers (and the LayerNorm's or the Conv1D's two) must
 * overlap neither each other nor any input or parameter (FASTVIM_ERR_OVERLAP).  B == 0 writes zero gradients.  Errors as
 * fastvim_ssm_fwd, plus FASTVIM_ERR_NULL for a NULL grads or gradient buffer.
 * Enqueues its kernels on stream and returns.
 *
 * Image groups.  A large call (by default: B >= 16 and h w E >= 2^20, or
 * K E >= 2^20 when masked: 4 groups, 2 with the LayerNorm (with or without
 * the Conv1D), none for dense layers with the Conv1D and without the norm;
 * params.tuning's FASTVIM_TUNING_BWD_GROUPS sets the count) runs in groups of ceil(B / groups) images: the first passes of all
 * groups, then their second passes, in order on stream, while each group's
 * scan adjoint and parameter sums run on a second stream of the library's
 * own (one per device, default priority, created on the first such call and
 * kept until the process ends) between events recorded on both streams, so
 * that they overlap the streaming passes.  Every piece of work the call
 * enqueues there comes after what stream held when the call was made, and
 * stream's own later work comes after all of it.  Parameter gradients are
 * the groups' sums added in group order: run-to-run identical for a given
 * grouping, equal to the ungrouped call's within rounding.  The workspace
 * size covers every grouping. */
int fastvim_ssm_bwd(const void *x, const void *z, const void *dout, const fastvim_params *params,
                    const fastvim_dims *dims, int pool_axis, const int32_t *mask_idx, void *dx, void *dz,
                    const fastvim_grads *grads, void *stream);

/* Measurement aid, not part of the layer: copy `bytes` bytes from src to dst
 * (device memory, both 16-byte aligned, bytes a multiple of 16, no overlap)
 * with a plain streaming kernel -- 16-byte nontemporal loads and stores, every
 * byte read once and written once.  Its rate is the device's practical
 * streaming ceiling, and its hardware byte counters (read bytes == written
 * bytes == `bytes`) calibrate those of the layer's kernels.  Enqueued on
 * stream; bytes == 0 launches nothing.  Errors: FASTVIM_ERR_NULL,
 * FASTVIM_ERR_ALIGN, FASTVIM_ERR_OVERLAP, FASTVIM_ERR_HIP. */
int fastvim_calib_copy(void *dst, const void *src, size_t bytes, void *stream);

/* Static text for a status code. */
const char *fastvim_status_string(int status);

/* FASTVIM_ABI_VERSION of the built library. */
int fastvim_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FASTVIM_H */
