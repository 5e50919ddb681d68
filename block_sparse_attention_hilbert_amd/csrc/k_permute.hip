// Token reordering along the 3D Hilbert order (DFSAttn page, trick 1): a row
// gather (permute) or scatter (unpermute) of [B,H,N,d] bf16 tensors.
//
// HBM-bound copy: each thread moves 16 bytes; the d/8 threads of one token
// row read and write one contiguous row, so both sides are coalesced per row.
// Work items are ordered (bh, n, chunk) so a wavefront covers 4 (d = 128) or
// 8 (d = 64) whole rows.
#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void k_permute(const uint4* __restrict__ src,
                                                      uint4* __restrict__ dst,
                                                      const int32_t* __restrict__ perm,
                                                      int64_t BH, int N, int inverse) {
    constexpr int CH = D / 8;
    const int64_t total = BH * N * CH;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kThreads) {
        const int c = (int)(e % CH);
        const int64_t t = e / CH;
        const int n = (int)(t % N);
        const int64_t bh = t / N;
        const int p = clamp_token(perm[n], N);
        const int64_t from = inverse ? n : p;
        const int64_t to = inverse ? p : n;
        dst[(bh * N + to) * CH + c] = src[(bh * N + from) * CH + c];
    }
}

}  // namespace

sa_status launch_permute(const Geometry& g, const uint16_t* src, uint16_t* dst,
                         const int32_t* perm, bool inverse, hipStream_t stream) {
    const int64_t total = g.BH() * g.N * (g.d / 8);
    const int64_t want = ceil_div(total, kThreads);
    const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
    if (g.d == 128)
        hipLaunchKernelGGL(k_permute<128>, dim3(grid), dim3(kThreads), 0, stream,
                           (const uint4*)src, (uint4*)dst, perm, g.BH(), g.N, inverse ? 1 : 0);
    else
        hipLaunchKernelGGL(k_permute<64>, dim3(grid), dim3(kThreads), 0, stream,
                           (const uint4*)src, (uint4*)dst, perm, g.BH(), g.N, inverse ? 1 : 0);
    return hip_check(hipGetLastError(), "k_permute launch");
}

}  // namespace sa
