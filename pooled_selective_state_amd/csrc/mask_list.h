// Row lists of a masked layer's kept tokens, for the pooling kernels.
//
// FastMaskVim pools only the kept tokens of each scan row (FastVim summary
// page, section 方法详解, bullet 6: a kept token belongs to the row of its grid
// index).  A pooling workgroup for row t of image b first
// collects which of the image's kept tokens lie in row t, then loads them all
// at once, instead of testing the tokens one by one with a load in between.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fastvim {

constexpr int kMaxListWaves = 16;  // waves of a 1024-thread workgroup

// The kept tokens k in [k0, k0 + blockDim.x) of one image whose row is t, in
// increasing k, go to list[0 .. n) as k - k0; returns n (the same value in
// every thread).  rows_img: the image's (K) row ids, -1 for an invalid token.
// list holds blockDim.x ints, wave_cnt kMaxListWaves.  Every thread of the
// workgroup calls it (it holds barriers; the first one also ends every use of
// the previous call's list).
__device__ __forceinline__ int row_token_list(const int32_t* __restrict__ rows_img, int64_t K, int64_t t,
                                              int64_t k0, int* list, int* wave_cnt) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = (int)((blockDim.x + 63) >> 6);
    const int64_t k = k0 + tid;
    const bool hit = k < K && rows_img[k] == t;
    const unsigned long long m = __ballot(hit);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) wave_cnt[wave] = __popcll(m);
    __syncthreads();
    int off = 0, n = 0;
    for (int w = 0; w < nw; ++w) {
        const int cnt = wave_cnt[w];
        off += w < wave ? cnt : 0;
        n += cnt;
    }
    if (hit) list[off + before] = tid;
    __syncthreads();
    return n;
}

}  // namespace fastvim
