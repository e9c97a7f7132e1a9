// Internal declarations shared by the HIP kernels and the host API of the
// gfx950 pooled selective-scan layer.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "fastvim.h"

namespace fastvim {

// ------------------------------------------------------------------ geometry
// Resolved sizes of one call.  T is the scan length, P the pooled-axis length
// (1 when unpooled), NX = R + 2N the width of one direction's x_proj output.
struct Geom {
    int64_t B, h, w, E, N, R, K, T, P, NX;
    int axis;     // fastvim_pool_axis
    bool masked;  // K > 0
    bool pooled;  // axis is COLS or ROWS
    int io;       // fastvim_dtype
    float pool_scale = 1.f;  // factor on the pooled tokens (FASTVIM_FLAG_POOL_SCALE)
    uint32_t tuning = 0;     // params.tuning (single-launch lags, poll limit)
};

// What a pooled row sum is multiplied by: pool_scale / P.
inline float pool_norm(const Geom& g) { return g.pool_scale / (float)g.P; }

// Workspace carve-up (every region 256-byte aligned).
struct Workspace {
    float* u;         // (B, T, E) pooled tokens; unused when unpooled
    float* xdbl;      // (B, T, 2, NX) x_proj outputs of both directions
    float* s_f;       // (B, T, E) forward scan output
    float* s_b;       // (B, T, E) backward scan output
    int32_t* rows;    // (B, K) masked: scan row of each kept token, -1 if invalid
    int32_t* bad;     // (B) masked: invalid mask entries per image
    unsigned* sync;   // (2 + 2B) ticket, status word, per-image progress counters; first in the
                      // workspace, so the status word sits at byte offset 4
};

// Words of the sync region: ticket, status, and two counters per image.
inline int64_t sync_words(const Geom& g) { return 2 + 2 * g.B; }

// Status word bits (sync[1]): a wait in the single launch gave up; an invalid
// mask index was found (FASTVIM_FLAG_CHECK_IDX).
constexpr unsigned kStatusWaitGaveUp = 1u;
constexpr unsigned kStatusBadIndex = 2u;

// Bytes needed; when base != nullptr also fills *ws.
size_t workspace_layout(const Geom& g, void* base, Workspace* ws);

// fastvim_ssm_fwd on a scratch region of cap bytes whose device address
// scratch() gives, asked only once every argument has passed validation
// (params->workspace is not read); FASTVIM_ERR_SCRATCH when the layer needs
// more than cap.  Enqueues no allocation.
int fwd_on_scratch(const void* x, const void* z, const fastvim_params* params, const fastvim_dims* dims, int axis,
                   const int32_t* idx, void* out, hipStream_t s, int (*scratch)(void**), size_t cap);

// Stage launchers (enqueue only; return the launch's hipError_t).
// status: NULL, or the status word that gets kStatusBadIndex when an index is invalid.
hipError_t launch_mask_rows(const Geom& g, const int32_t* idx, const Workspace& ws, unsigned* status,
                            hipStream_t st);
hipError_t launch_pool(const Geom& g, const void* x, const Workspace& ws, hipStream_t st);
// Masked layers: mask rows and pooling in one launch, one workgroup per image
// (pool.hip), for at most 1024 kept tokens per image.
bool mask_pool_supported(const Geom& g);
hipError_t launch_mask_pool(const Geom& g, const int32_t* idx, const void* x, const Workspace& ws,
                            unsigned* status, hipStream_t st);
hipError_t launch_proj(const Geom& g, const void* x, const fastvim_params& p, const Workspace& ws,
                       hipStream_t st);
hipError_t launch_scan(const Geom& g, const void* x, const fastvim_params& p, const Workspace& ws,
                       hipStream_t st);
hipError_t launch_epilogue(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                           const Workspace& ws, void* out, hipStream_t st);
hipError_t launch_conv_pool(const Geom& g, const void* x, const fastvim_params& p, const Workspace& ws,
                            hipStream_t st);
hipError_t launch_conv_epilogue(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                                const Workspace& ws, void* out, hipStream_t st);
// Scan and output stage in one launch (scan_out.hip): pooled layers with
// scans of at most 64 steps, without the LayerNorm or the Conv1D on load.
bool scan_out_supported(const Geom& g, uint32_t flags);
hipError_t launch_scan_out(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                           const Workspace& ws, void* out, hipStream_t st);
hipError_t launch_epilogue_norm(const Geom& g, const void* x, const void* z, const fastvim_params& p,
                                const Workspace& ws, void* out, hipStream_t st);
// Single-launch dense pooled layer (fused.hip).
// norm: with the post-SSM LayerNorm (FASTVIM_FLAG_POST_NORM); conv: with the
// producer Conv1D computed on load (FASTVIM_FLAG_CONV; COLS only).
bool fused_supported(const Geom& g, bool norm, bool local, bool conv);
bool fused_preferred(const Geom& g, bool norm, bool local, bool conv);  // the default path is the single launch
hipError_t launch_fused(const Geom& g, const void* x, const void* z, const fastvim_params& p, const Workspace& ws,
                        void* out, hipStream_t st);
hipError_t launch_zero_sync(const Workspace& ws, int64_t n, hipStream_t st);
hipError_t launch_calib_copy(void* dst, const void* src, size_t bytes, hipStream_t st);

// ------------------------------------------------------------ device helpers
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// I/O element traits: one 16-byte vector (raw) holds V elements.
struct IoF32 {
    using elem = float;
    using raw = f32x4;
    static constexpr int V = 4;
};
struct IoBf16 {
    using elem = uint16_t;
    using raw = u32x4;
    static constexpr int V = 8;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Two fp32 values to packed bf16 (the first in the low half) with gfx950's
// v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// 16-byte vector load / store of V I/O elements widened to fp32.
template <bool NT>
__device__ __forceinline__ void load_vec(const float* p, float (&v)[4]) {
    f32x4 t = NT ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p))
                 : *reinterpret_cast<const f32x4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
template <bool NT>
__device__ __forceinline__ void load_vec(const uint16_t* p, float (&v)[8]) {
    u32x4 t = NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p))
                 : *reinterpret_cast<const u32x4*>(p);
    v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xffff0000u);
    v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xffff0000u);
    v[4] = __uint_as_float(t.z << 16); v[5] = __uint_as_float(t.z & 0xffff0000u);
    v[6] = __uint_as_float(t.w << 16); v[7] = __uint_as_float(t.w & 0xffff0000u);
}
template <bool NT>
__device__ __forceinline__ void store_vec(float* p, const float (&v)[4]) {
    f32x4 t = {v[0], v[1], v[2], v[3]};
    if (NT) __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(p));
    else *reinterpret_cast<f32x4*>(p) = t;
}
template <bool NT>
__device__ __forceinline__ void store_vec(uint16_t* p, const float (&v)[8]) {
    u32x4 t;
    t.x = f32x2_to_bf16x2(v[0], v[1]);
    t.y = f32x2_to_bf16x2(v[2], v[3]);
    t.z = f32x2_to_bf16x2(v[4], v[5]);
    t.w = f32x2_to_bf16x2(v[6], v[7]);
    if (NT) __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = t;
}

// Raw 16-byte loads (kept narrow until used) and their widening.
template <bool NT>
__device__ __forceinline__ f32x4 load_raw(const float* p) {
    return NT ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p)) : *reinterpret_cast<const f32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ u32x4 load_raw(const uint16_t* p) {
    return NT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)) : *reinterpret_cast<const u32x4*>(p);
}
// Element k (0 <= k < V) of a raw vector, as fp32.
__device__ __forceinline__ float raw_at(const f32x4& r, int k) { return r[k]; }
__device__ __forceinline__ float raw_at(const u32x4& r, int k) {
    const uint32_t wd = r[k >> 1];
    return __uint_as_float((k & 1) ? (wd & 0xffff0000u) : (wd << 16));
}

// Scalar element load widened to fp32.
__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t* p) { return bf16_bits_to_f32(*p); }

// Offset (in tokens) of scan position t of image b's grid in unpooled order.
__device__ __forceinline__ int64_t unpooled_token(int axis, int64_t t, int64_t h, int64_t w) {
    if (axis == FASTVIM_POOL_NONE_ROWMAJOR) return t;
    const int64_t j = t / h, i = t - j * h;  // t = j*h + i
    return i * w + j;
}

}  // namespace fastvim
