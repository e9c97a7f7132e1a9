// Device helpers of the producer Conv1D + SiLU (depthwise, causal, 4 taps,
// oldest tap first), shared by the kernels that compute it where x is read
// (conv.hip) and those that write it out or take its adjoint (conv_seq.hip).
//   x_conv[r, e] = silu(conv_b[e] + sum_{k<4} conv_w[e, k] x[r - 3 + k, e])
// FastVim summary page (gptget.net, arXiv 2502.00594), section 方法详解,
// bullets 1-2; Vim article (ijyty.com) 2.1.
#pragma once

#include "fastvim_internal.h"

namespace fastvim {

constexpr int kTaps = FASTVIM_CONV_TAPS;

__device__ __forceinline__ float conv_silu_f(float q) { return q * __builtin_amdgcn_rcpf(1.f + __expf(-q)); }

// Channel weights of the lane's V channels: taps (oldest first) and bias.
template <int V>
struct ConvW {
    float w[V][kTaps], b[V];
};
template <int V>
__device__ __forceinline__ void load_conv_w(const float* cw, const float* cb, int64_t col, ConvW<V>& W) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(cw + (col + v) * kTaps);
        W.w[v][0] = t.x;
        W.w[v][1] = t.y;
        W.w[v][2] = t.z;
        W.w[v][3] = t.w;
        W.b[v] = cb[col + v];
    }
}

// x_conv for the lane's V channels from a window of raw vectors: the cell
// (cur) and its three predecessors (p1 the newest); a predecessor before the
// start of the sequence is a zero vector.
template <class IO>
__device__ __forceinline__ void conv_window(const typename IO::raw& p3, const typename IO::raw& p2,
                                            const typename IO::raw& p1, const typename IO::raw& cur,
                                            const ConvW<IO::V>& W, float (&xc)[IO::V]) {
    static_assert(kTaps == 4, "window of three predecessors");
#pragma unroll
    for (int v = 0; v < IO::V; ++v) {
        float a = fmaf(W.w[v][3], raw_at(cur, v), W.b[v]);
        a = fmaf(W.w[v][2], raw_at(p1, v), a);
        a = fmaf(W.w[v][1], raw_at(p2, v), a);
        a = fmaf(W.w[v][0], raw_at(p3, v), a);
        xc[v] = conv_silu_f(a);
    }
}

// Token index within the image of the k-th predecessor (k >= 1) of grid cell
// (i, j) in the oriented sequence, or -1 before the start of the sequence.
template <bool COLS>
__device__ __forceinline__ int pred_token(int i, int j, int k, int h, int w) {
    if (COLS) {
        const int r = i * w + j - k;
        return r;  // row-major: memory order; negative before the start
    }
    if (i >= k) return (i - k) * w + j;
    const int r = j * h + i - k;  // column-major position; may lie several columns back when h < k
    return r < 0 ? -1 : (r % h) * w + r / h;
}

// The three predecessors of cell (i, j) (p1 the newest), zero before the start.
template <class IO, bool COLS>
__device__ __forceinline__ void load_halo(const typename IO::elem* xb, int coff, int E, int i, int j, int h, int w,
                                          typename IO::raw& p3, typename IO::raw& p2, typename IO::raw& p1) {
    typename IO::raw r[3];
#pragma unroll
    for (int k = 1; k <= 3; ++k) {
        const int tok = pred_token<COLS>(i, j, k, h, w);
        r[k - 1] = typename IO::raw{};
        if (tok >= 0) r[k - 1] = load_raw<false>(xb + (coff + tok * E));
    }
    p1 = r[0];
    p2 = r[1];
    p3 = r[2];
}

// d silu(a) / da = sigmoid(a) (1 + a (1 - sigmoid(a))).
__device__ __forceinline__ float conv_silu_grad(float a) {
    const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-a));
    return sg * (1.f + a * (1.f - sg));
}

}  // namespace fastvim
