// Data-dependent block formation for gfx950 (SVOO page, section 2B: online
// bidirectional co-clustering; SVG-EAR page, section 2A: k-means and a
// permutation that makes every cluster contiguous).
//
// Per (batch, head) and per side (queries, keys):
//   k_chunk_assign  initial partition: C equal chunks of the token order
//   k_assign_mx (C <= 64), k_cent_prep + k_assign (larger C)
//                   every token to its best centroid: the largest
//                   x.c (co-clustering affinity) or x.c - |c|^2/2 (k-means),
//                   each dot product a sequential fp32 FMA chain over the
//                   channels, ties to the lower index -- the integer decision
//                   is taken in one fixed arithmetic
//   k_chunkmean, k_clmean (C <= 64)
//                   cluster means without sorting: the initial chunks' means
//                   from contiguous rows; in every round k_assign_mx leaves
//                   per-workgroup exact fp64 cluster sums and k_clmean adds
//                   them up (an empty cluster keeps its previous centroid)
//   k_hist, k_hist_scan, k_sort_scatter
//                   stable counting sort of the tokens by cluster (tiles of
//                   1024 tokens; LDS bitonic sort inside a tile): every round
//                   for C > 64, once at the end otherwise
//   k_segmean       cluster means from exact fp64 sums over the sorted order
//                   (rounds with C > 64, value means, tile partitions)
//   k_layout        the padded layout: each cluster takes whole blocks
//                   (its tokens in ascending order, then padding); per-block
//                   cluster and token count
//   k_gather_rows, k_scatter_rows
//                   tensors into / out of the padded layout
//   k_cselect, k_crow_count, k_crow_fill, k_block_comp
//                   cluster-level selection, its block-level CSR and the
//                   per-block compensation statistics
#include <math.h>

#include <algorithm>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kTok = 1024;          // tokens per sort tile (and threads of the sort kernels)
constexpr int kCmax = 1024;         // largest number of clusters

// ----------------------------------------------------------------------------
// initial partition
// ----------------------------------------------------------------------------
__global__ void k_chunk_assign(int32_t* __restrict__ assign, int N, int C) {
    const int64_t bh = blockIdx.y;
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= N) return;
    // chunk c holds tokens [floor(cN/C), floor((c+1)N/C))
    assign[bh * N + t] = (int32_t)((((int64_t)t + 1) * C + N - 1) / N - 1);
}

// ----------------------------------------------------------------------------
// assignment
// ----------------------------------------------------------------------------
constexpr int kAsgThreads = 256;
constexpr int kAsgIlp = 8;          // centroid chains a thread runs side by side

// Centroids of every head transposed to [D][Cp] (Cp = C rounded up to 8, the
// padding 0) and their decision bias: -|c|^2/2 = fl32(-0.5 * seqfma(c, c))
// for k-means, 0 for co-clustering, -inf for the padding (never chosen).
template <int D>
__global__ void k_cent_prep(const float* __restrict__ cent, float* __restrict__ centT,
                            float* __restrict__ bias, int C, int Cp, int kmeans) {
    const int64_t bh = blockIdx.y;
    const int e = blockIdx.x * blockDim.x + threadIdx.x;      // (d, c) of centT
    if (e < D * Cp) {
        const int d = e / Cp, c = e % Cp;
        centT[bh * (int64_t)D * Cp + e] = c < C ? cent[(bh * C + c) * (int64_t)D + d] : 0.f;
    }
    if (e < Cp) {
        float b = e < C ? 0.f : -INFINITY;
        if (kmeans && e < C) {
            const float* ce = cent + (bh * C + e) * (int64_t)D;
            float acc = 0.f;
            for (int d = 0; d < D; ++d) acc = __builtin_fmaf(ce[d], ce[d], acc);
            b = -0.5f * acc;
        }
        bias[bh * Cp + e] = b;
    }
}

// One thread per token, its row in registers as packed bf16 pairs.  The
// centroid values are the same for every lane, so they come through the
// scalar data path (wave-uniform loads of 8 consecutive floats of the
// transposed centroids) and enter each FMA as its scalar operand.  Each of the
// 8 interleaved chains is the sequential FMA over the channels in channel
// order; the score is the chain plus the bias, one fp32 add; strict > keeps
// the lowest index on ties.
template <int D>
__global__ __launch_bounds__(kAsgThreads) void k_assign(const uint16_t* __restrict__ X,
                                                        const float* __restrict__ centT,
                                                        const float* __restrict__ bias,
                                                        int32_t* __restrict__ assign, int N,
                                                        int Cp) {
    const int64_t bh = blockIdx.y;
    const int t = blockIdx.x * kAsgThreads + threadIdx.x;
    uint32_t xw[D / 2];
    {
        const int tt = t < N ? t : N - 1;
        const uint4* row = reinterpret_cast<const uint4*>(X + (bh * N + tt) * (int64_t)D);
#pragma unroll
        for (int q = 0; q < D / 8; ++q) {
            const uint4 v = row[q];
            xw[4 * q] = v.x;
            xw[4 * q + 1] = v.y;
            xw[4 * q + 2] = v.z;
            xw[4 * q + 3] = v.w;
        }
    }
    const float* ct = centT + bh * (int64_t)D * Cp;
    const float* bs = bias + bh * Cp;
    float best = -INFINITY;
    int arg = 0;
#pragma unroll 1
    for (int j = 0; j < Cp; j += kAsgIlp) {
        float acc[kAsgIlp];
#pragma unroll
        for (int k = 0; k < kAsgIlp; ++k) acc[k] = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const float xd = __uint_as_float((d & 1) ? (xw[d / 2] & 0xffff0000u) : (xw[d / 2] << 16));
            const float* c = ct + (int64_t)d * Cp + j;
#pragma unroll
            for (int k = 0; k < kAsgIlp; ++k) acc[k] = __builtin_fmaf(xd, c[k], acc[k]);
        }
#pragma unroll
        for (int k = 0; k < kAsgIlp; ++k) {
            const float s = acc[k] + bs[j + k];
            if (s > best) {
                best = s;
                arg = j + k;
            }
        }
    }
    if (t < N) assign[bh * N + t] = arg;
}

// ----------------------------------------------------------------------------
// assignment on the matrix cores with a certified filter (C <= 64)
//
// s~[c, t] = x_t . c on v_mfma_f32_32x32x16_bf16: x is bf16 (exact operand),
// the fp32 centroid is split into bf16 hi + lo; |s~ - seqfma| <= 2^-14.7
// sum_d |x_d c_d| (split remainder 2^-16, fp32 accumulation of 256 terms, the
// chain's own 128 roundings).  With B = 2^-12 (|x| |c| + |bias|), a
// centroid can win only if s~ + bias + B >= the token's best s~ + bias - B;
// those candidates (about one per token) get the exact decision arithmetic
// of k_assign, and the exact winner among them is the winner among all.
//
// A workgroup (16 waves; its LDS, which also holds the cluster sums below,
// fits one per CU) serves one head and many 32-token groups: it stages
// the head's centroids once (fp32 rows for the exact chains, the split hi / lo
// operands in the lane order of the matrix instruction, the decision bias and
// the bound terms per centroid), then each wave takes groups of 32 tokens
// (two lanes per token) in turn.  Each token's candidates are evaluated by its
// own two lanes in ascending index order.
// ----------------------------------------------------------------------------
typedef __bf16 amx_bf16x8 __attribute__((ext_vector_type(8)));
typedef float amx_f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 amx_bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kAmxC = 64;                  // centroid slots (C <= 64)
constexpr int kAmxWaves = 16;              // waves per workgroup
constexpr int kAmxWgTarget = 256;          // workgroups per launch, over all heads
constexpr float kAmxEps = 1.0f / 4096.0f;  // bound factor 2^-12
// added to both squared norms: it covers squares and products lost below the
// fp32 / bf16 normal range (flushed or underflowed), so that the bound holds
// for arbitrarily small tokens and centroids
constexpr float kAmxTiny = 0x1p-118f;

__device__ __forceinline__ uint16_t amx_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// the value of lane (l & 31) + 32 h, for both lanes l of a pair (h constant)
template <int HALF>
__device__ __forceinline__ float amx_pair_take(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(HALF == 0 ? r[0] : r[1]);
}

// Cluster sums without sorting.  A cluster mean is fl32(exact sum / n): fp64
// sums of bf16 values are exact while their significands span fewer than 53
// bits (the means' definition takes them as exact), so they may be formed in
// any order.  Each
// workgroup sums its tokens per cluster in LDS and writes one partial row per
// cluster it touched; k_clmean adds the partials of a head.
//
// Adds the rows of tokens tok0 .. tok0 + 31 (those below N) to their
// clusters' LDS sums; lane j < 32 holds the cluster of token tok0 + j.  Lane l
// takes channels D/64 l .. of every row; a run of tokens of one cluster is
// summed in registers and added to LDS when the cluster changes.
template <int D>
__device__ __forceinline__ void amx_accumulate(const uint16_t* __restrict__ Xh, int tok0, int N,
                                               int cl, double* ssum, int* scnt, int lane) {
    constexpr int CPL = D / 64;
    static_assert(CPL == 1 || CPL == 2, "D is 64 or 128");
    const int nt = min(32, N - tok0);
    uint32_t v[32];                        // channel 2l | 2l+1 (D = 128), or channel l in the high half
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const int64_t row = (int64_t)(tok0 + min(j, nt - 1)) * D;
        if constexpr (CPL == 2)
            v[j] = reinterpret_cast<const uint32_t*>(Xh + row)[lane];
        else
            v[j] = (uint32_t)Xh[row + lane] << 16;
    }
    auto flush = [&](int c, double a0, double a1, int run) {
        __hip_atomic_fetch_add(ssum + c * D + CPL * lane, a0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if constexpr (CPL == 2)
            __hip_atomic_fetch_add(ssum + c * D + 2 * lane + 1, a1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (lane == 0) __hip_atomic_fetch_add(scnt + c, run, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    int cur = __builtin_amdgcn_readlane(cl, 0);
    double a0 = 0.0, a1 = 0.0;
    int run = 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        if (j < nt) {
            const int c = __builtin_amdgcn_readlane(cl, j);
            if (c != cur) {
                flush(cur, a0, a1, run);
                cur = c;
                a0 = a1 = 0.0;
                run = 0;
            }
            if constexpr (CPL == 2) {
                a0 += (double)__uint_as_float(v[j] << 16);
                a1 += (double)__uint_as_float(v[j] & 0xffff0000u);
            } else {
                a0 += (double)__uint_as_float(v[j]);
            }
            ++run;
        }
    }
    flush(cur, a0, a1, run);
}

// zeroes the workgroup's LDS sums (before the first accumulation)
template <int D, int NT>
__device__ __forceinline__ void amx_sums_clear(double* ssum, int* scnt) {
    for (int p = threadIdx.x; p < kAmxC * D; p += NT) ssum[p] = 0.0;
    for (int p = threadIdx.x; p < kAmxC; p += NT) scnt[p] = 0;
}

// writes the workgroup's partial sums: the count of every slot, the row of
// every slot with tokens (k_clmean reads only those)
template <int D, int NT>
__device__ __forceinline__ void amx_sums_store(const double* ssum, const int* scnt,
                                               double* __restrict__ psum,
                                               int32_t* __restrict__ pcnt, int64_t part) {
    __syncthreads();
    for (int p = threadIdx.x; p < kAmxC * D; p += NT)
        if (scnt[p / D] > 0) psum[part * kAmxC * D + p] = ssum[p];
    for (int p = threadIdx.x; p < kAmxC; p += NT) pcnt[part * kAmxC + p] = scnt[p];
}

template <int D>
__global__ __launch_bounds__(64 * kAmxWaves) __attribute__((amdgpu_waves_per_eu(4))) void k_assign_mx(const uint16_t* __restrict__ X,
                                                              const float* __restrict__ cent,
                                                              int32_t* __restrict__ assign,
                                                              double* __restrict__ psum,
                                                              int32_t* __restrict__ pcnt, int N,
                                                              int C, int kmeans) {
    constexpr int ROW = D + 4;                     // floats per centroid row in LDS
    constexpr int NST = D / 16;                    // k-steps of the matrix instruction
    constexpr int NT = 64 * kAmxWaves;
    __shared__ __align__(16) float cs[kAmxC * ROW];     // the head's centroids (fp32)
    __shared__ uint4 aop[2][NST][2][64];                // A operands [tile][k-step][hi, lo][lane]
    __shared__ float sb[kAmxC];                         // decision bias
    __shared__ __align__(16) float sbl[kAmxC];          // bias - its bound share
    __shared__ __align__(16) float sbh[kAmxC];          // bias + its bound share
    __shared__ __align__(16) float sn[kAmxC];           // norm upper bound
    __shared__ double ssum[kAmxC * D];                  // cluster sums (fp64, exact)
    __shared__ int scnt[kAmxC];                         // cluster token counts
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int r32 = lane & 31, hf = lane >> 5;
    const int64_t bh = blockIdx.y;
    const int nct = (C + 31) / 32;                 // centroid tiles
    const uint16_t* Xh = X + bh * (int64_t)N * D;
    {
        const float* ch = cent + bh * (int64_t)C * D;
        for (int p = threadIdx.x; p < kAmxC * (D / 4); p += NT) {
            const int c = p / (D / 4), o = p % (D / 4);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < C) v = reinterpret_cast<const float4*>(ch + (int64_t)c * D)[o];
            *reinterpret_cast<float4*>(cs + c * ROW + 4 * o) = v;
        }
    }
    amx_sums_clear<D, NT>(ssum, scnt);
    __syncthreads();
    // A operand of lane l in tile ct, k-step st: centroid ct*32 + (l & 31),
    // channels 16 st + 8 (l >> 5) .. + 7, as bf16 hi and the bf16 of the rest
    for (int p = threadIdx.x; p < 2 * NST * 64; p += NT) {
        const int l = p & 63, st = (p >> 6) % NST, ct = p / (64 * NST);
        const float* cr = cs + (ct * 32 + (l & 31)) * ROW + 16 * st + 8 * (l >> 5);
        float v[8];
        *reinterpret_cast<float4*>(v) = *reinterpret_cast<const float4*>(cr);
        *reinterpret_cast<float4*>(v + 4) = *reinterpret_cast<const float4*>(cr + 4);
        uint32_t h[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint16_t h0 = amx_bf16(v[2 * e]), h1 = amx_bf16(v[2 * e + 1]);
            const uint16_t l0 = amx_bf16(v[2 * e] - __uint_as_float((uint32_t)h0 << 16));
            const uint16_t l1 = amx_bf16(v[2 * e + 1] - __uint_as_float((uint32_t)h1 << 16));
            h[e] = h0 | ((uint32_t)h1 << 16);
            lo[e] = l0 | ((uint32_t)l1 << 16);
        }
        aop[ct][st][0][l] = make_uint4(h[0], h[1], h[2], h[3]);
        aop[ct][st][1][l] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    if (threadIdx.x >= NT - kAmxC) {
        // decision bias, as k_cent_prep: fl32(-0.5 seqfma(c, c)) for k-means,
        // 0 for co-clustering, -inf for unused slots; a norm upper bound
        const int c = threadIdx.x - (NT - kAmxC);
        float acc = 0.f;
#pragma unroll 8
        for (int k = 0; k < D; ++k) acc = __builtin_fmaf(cs[c * ROW + k], cs[c * ROW + k], acc);
        const float b = c < C ? (kmeans ? -0.5f * acc : 0.f) : -INFINITY;
        sb[c] = b;
        sbl[c] = c < C ? b - kAmxEps * fabsf(b) : -INFINITY;
        sbh[c] = c < C ? b + kAmxEps * fabsf(b) : -INFINITY;
        sn[c] = sqrtf(acc + kAmxTiny) * (1.0f + 1.0f / 1024.0f);
    }
    __syncthreads();

    const int ngr = (N + 31) / 32;
    for (int g = blockIdx.x * kAmxWaves + wave; g < ngr; g += gridDim.x * kAmxWaves) {
        const int tok0 = g * 32;
        // B operand (x^T) of the group's 32 tokens: lane (r32, hf) holds
        // channels 16 st + 8 hf .. + 7 of token r32, for st = 0 .. NST - 1
        amx_bf16x8 xf[NST];
        {
            const int t = min(tok0 + r32, N - 1);
            const uint4* row = reinterpret_cast<const uint4*>(Xh + (int64_t)t * D);
#pragma unroll
            for (int st = 0; st < NST; ++st) xf[st] = __builtin_bit_cast(amx_bf16x8, row[2 * st + hf]);
        }
        amx_f32x16 acc[2] = {amx_f32x16{}, amx_f32x16{}};
#pragma unroll
        for (int st = 0; st < NST; ++st) {
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                if (ct >= nct) break;
                const amx_bf16x8 ah = __builtin_bit_cast(amx_bf16x8, aop[ct][st][0][lane]);
                const amx_bf16x8 al = __builtin_bit_cast(amx_bf16x8, aop[ct][st][1][lane]);
                acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xf[st], acc[ct], 0, 0, 0);
                acc[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xf[st], acc[ct], 0, 0, 0);
            }
        }
        // the token's norm bound (two-term dot products: only the bound reads
        // it, and the 2^-10 factor covers their rounding)
        float ss = 0.f;
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            const uint4 v = __builtin_bit_cast(uint4, xf[st]);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const amx_bf16x2 p = __builtin_bit_cast(amx_bf16x2, w[e]);
                ss = __builtin_amdgcn_fdot2_f32_bf16(p, p, ss, false);
            }
        }
        ss = amx_pair_take<0>(ss) + amx_pair_take<1>(ss);
        const float enx = kAmxEps * (sqrtf(ss + kAmxTiny) * (1.0f + 1.0f / 1024.0f));

        // element r of tile ct: centroid ct*32 + 8 (r / 4) + 4 hf + r % 4, token r32.
        // The token's best lower bound, then the mask of its candidates.
        float thr = -INFINITY;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            if (ct >= nct) break;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c0 = ct * 32 + 8 * q + 4 * hf;
                const float4 bl = *reinterpret_cast<const float4*>(sbl + c0);
                const float4 nn = *reinterpret_cast<const float4*>(sn + c0);
                thr = fmaxf(thr, __builtin_fmaf(-enx, nn.x, acc[ct][4 * q + 0] + bl.x));
                thr = fmaxf(thr, __builtin_fmaf(-enx, nn.y, acc[ct][4 * q + 1] + bl.y));
                thr = fmaxf(thr, __builtin_fmaf(-enx, nn.z, acc[ct][4 * q + 2] + bl.z));
                thr = fmaxf(thr, __builtin_fmaf(-enx, nn.w, acc[ct][4 * q + 3] + bl.w));
            }
        }
        thr = fmaxf(amx_pair_take<0>(thr), amx_pair_take<1>(thr));
        // unused slots have -inf bounds and never pass (thr is finite)
        uint32_t cm[2] = {0u, 0u};
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            if (ct >= nct) break;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c0 = ct * 32 + 8 * q + 4 * hf;
                const float4 bu = *reinterpret_cast<const float4*>(sbh + c0);
                const float4 nn = *reinterpret_cast<const float4*>(sn + c0);
                const float u[4] = {__builtin_fmaf(enx, nn.x, acc[ct][4 * q + 0] + bu.x),
                                    __builtin_fmaf(enx, nn.y, acc[ct][4 * q + 1] + bu.y),
                                    __builtin_fmaf(enx, nn.z, acc[ct][4 * q + 2] + bu.z),
                                    __builtin_fmaf(enx, nn.w, acc[ct][4 * q + 3] + bu.w)};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (u[e] >= thr) cm[ct] |= 1u << (8 * q + 4 * hf + e);
            }
        }
        // both lanes of the token take the union of their halves' masks
        uint64_t cand = 0;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const float m = __uint_as_float(cm[ct]);
            const uint32_t both = __float_as_uint(amx_pair_take<0>(m)) | __float_as_uint(amx_pair_take<1>(m));
            cand |= (uint64_t)both << (32 * ct);
        }

        // the token's channels as fp32 (exact)
        float xu[NST][8];
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            const uint4 v = __builtin_bit_cast(uint4, xf[st]);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xu[st][2 * e] = __uint_as_float(w[e] << 16);
                xu[st][2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
            }
        }

        // Exact decision arithmetic for the candidates, in ascending centroid
        // order: the token's two lanes run the chain over the channels in order,
        // 8 channels at a time, handing the partial sum across (lane hf = 0 holds
        // channel groups 0, 2, 4, ...; hf = 1 groups 1, 3, 5, ...).
        float best = -INFINITY;
        int arg = 0;
        for (;;) {
            const uint64_t any = __ballot(cand != 0);
            if (any == 0) break;
            const bool act = cand != 0;
            const int c = act ? __ffsll((long long)cand) - 1 : 0;
            if (act) cand &= cand - 1;
            const float* cr = cs + c * ROW + 8 * hf;
            float a = 0.f;
#pragma unroll
            for (int st = 0; st < NST; ++st) {
                const float4 c0 = *reinterpret_cast<const float4*>(cr + 16 * st);
                const float4 c1 = *reinterpret_cast<const float4*>(cr + 16 * st + 4);
                const float cc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
                // channels 16 st .. + 7 (lane hf = 0), then 16 st + 8 .. + 15 (hf = 1)
                float t = a;
                if (hf == 0) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) t = __builtin_fmaf(xu[st][e], cc[e], t);
                }
                a = amx_pair_take<0>(t);
                t = a;
                if (hf == 1) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) t = __builtin_fmaf(xu[st][e], cc[e], t);
                }
                a = amx_pair_take<1>(t);
            }
            if (act) {
                const float sc = a + sb[c];
                if (sc > best) {
                    best = sc;
                    arg = c;
                }
            }
        }
        const int t = tok0 + r32;
        if (hf == 0 && t < N) assign[bh * N + t] = arg;
        amx_accumulate<D>(Xh, tok0, N, arg, ssum, scnt, lane);
    }
    amx_sums_store<D, NT>(ssum, scnt, psum, pcnt, bh * gridDim.x + blockIdx.x);
}

// cluster means from the partial sums of G <= kAmxWgTarget workgroups per
// head; an empty cluster keeps its previous centroid
template <int D>
__global__ __launch_bounds__(D) void k_clmean(const double* __restrict__ psum,
                                              const int32_t* __restrict__ pcnt, int G,
                                              float* __restrict__ cent, int32_t* __restrict__ count,
                                              int C) {
    __shared__ int pc[kAmxWgTarget];
    const int c = blockIdx.x, tid = threadIdx.x;
    const int64_t p0 = (int64_t)blockIdx.y * G;
    for (int g = tid; g < G; g += D) pc[g] = pcnt[(p0 + g) * kAmxC + c];
    __syncthreads();
    int n = 0;
    for (int g = 0; g < G; ++g) n += pc[g];
    if (tid == 0) count[blockIdx.y * C + c] = n;
    if (n == 0) return;
    // eight partial rows in flight at a time (the sums are exact: any order)
    const double* col = psum + (p0 * kAmxC + c) * D + tid;
    double s = 0.0;
    int g = 0;
    for (; g + 8 <= G; g += 8) {
        double t[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) t[u] = pc[g + u] > 0 ? col[(int64_t)(g + u) * kAmxC * D] : 0.0;
#pragma unroll
        for (int u = 0; u < 8; ++u) s += t[u];
    }
    for (; g < G; ++g)
        if (pc[g] > 0) s += col[(int64_t)g * kAmxC * D];
    cent[((int64_t)blockIdx.y * C + c) * D + tid] = (float)(s / (double)n);
}

// ----------------------------------------------------------------------------
// stable counting sort by cluster
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kTok) void k_hist(const int32_t* __restrict__ assign,
                                               int32_t* __restrict__ tile_hist, int N, int C,
                                               int ntiles) {
    __shared__ int32_t h[kCmax];
    const int64_t bh = blockIdx.y;
    const int tile = blockIdx.x, tid = threadIdx.x;
    for (int c = tid; c < C; c += kTok) h[c] = 0;
    __syncthreads();
    const int t = tile * kTok + tid;
    if (t < N) atomicAdd(&h[assign[bh * N + t]], 1);
    __syncthreads();
    for (int c = tid; c < C; c += kTok) tile_hist[(bh * ntiles + tile) * C + c] = h[c];
}

// Per cluster: total count and start in the sorted order; per (tile, cluster):
// where the tile's tokens of that cluster go.
__global__ __launch_bounds__(kTok) void k_hist_scan(const int32_t* __restrict__ tile_hist,
                                                    int32_t* __restrict__ tile_off,
                                                    int32_t* __restrict__ count,
                                                    int32_t* __restrict__ cstart, int C,
                                                    int ntiles) {
    __shared__ int32_t wsum[kTok / 64];
    const int64_t bh = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int32_t* th = tile_hist + bh * ntiles * (int64_t)C;
    int32_t total = 0;
    if (tid < C)
        for (int t = 0; t < ntiles; ++t) total += th[(int64_t)t * C + tid];
    // exclusive scan of the totals over the clusters
    int32_t x = total;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < wid; ++w) before += wsum[w];
    const int32_t start = before + x - total;
    if (tid < C) {
        count[bh * C + tid] = total;
        cstart[bh * C + tid] = start;
        int32_t run = start;
        for (int t = 0; t < ntiles; ++t) {
            tile_off[(bh * ntiles + t) * (int64_t)C + tid] = run;
            run += th[(int64_t)t * C + tid];
        }
    }
}

__global__ __launch_bounds__(kTok) void k_sort_scatter(const int32_t* __restrict__ assign,
                                                       const int32_t* __restrict__ tile_off,
                                                       int32_t* __restrict__ sorted, int N, int C,
                                                       int ntiles) {
    __shared__ uint32_t key[kTok];
    const int64_t bh = blockIdx.y;
    const int tile = blockIdx.x, tid = threadIdx.x;
    const int t = tile * kTok + tid;
    key[tid] = t < N ? ((uint32_t)assign[bh * N + t] << 10) | (uint32_t)tid : 0xffffffffu;
    __syncthreads();
    for (int size = 2; size <= kTok; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (tid < kTok / 2) {
                const int lo = 2 * tid - (tid & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const uint32_t a = key[lo], b = key[hi];
                if ((a > b) == up) { key[lo] = b; key[hi] = a; }
            }
            __syncthreads();
        }
    }
    const uint32_t k = key[tid];
    if (k == 0xffffffffu) return;
    const uint32_t c = k >> 10;
    // first sorted position of cluster c in this tile (lower bound of c << 10)
    int lo = 0, hi = tid;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (key[mid] < (c << 10)) lo = mid + 1;
        else hi = mid;
    }
    const int rank = tid - lo;
    const int dst = tile_off[(bh * ntiles + tile) * (int64_t)C + c] + rank;
    sorted[bh * N + dst] = tile * kTok + (int)(k & 1023u);
}

// ----------------------------------------------------------------------------
// means and sizes of the initial partition: C equal chunks of the token order,
// chunk c = tokens [floor(c N / C), floor((c + 1) N / C)) (C <= N: none empty);
// exact fp64 sums of contiguous rows, one fp32 rounding
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_chunkmean(const uint16_t* __restrict__ X,
                                                   float* __restrict__ cent,
                                                   int32_t* __restrict__ count, int N, int C) {
    constexpr int CH = D / 8;                 // 16-byte chunks per row
    constexpr int ST = 256 / CH;              // token streams
    __shared__ double red[ST][D];
    const int c = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int s0 = (int)((int64_t)c * N / C), n = (int)((int64_t)(c + 1) * N / C) - s0;
    if (tid == 0) count[bh * C + c] = n;
    const int ch = tid % CH, st = tid / CH;
    const uint16_t* Xh = X + (bh * N + s0) * (int64_t)D + ch * 8;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto add = [&](uint4 v) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)__uint_as_float(w[e] << 16);
            acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xffff0000u);
        }
    };
    constexpr int U = 4;                      // rows in flight per thread
    int r = st;
    for (; r + (U - 1) * ST < n; r += U * ST) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const uint4*>(Xh + (int64_t)(r + u * ST) * D);
#pragma unroll
        for (int u = 0; u < U; ++u) add(v[u]);
    }
    for (; r < n; r += ST) add(*reinterpret_cast<const uint4*>(Xh + (int64_t)r * D));
#pragma unroll
    for (int e = 0; e < 8; ++e) red[st][ch * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        double sum = 0.0;
        for (int k = 0; k < ST; ++k) sum += red[k][tid];
        cent[(bh * C + c) * (int64_t)D + tid] = (float)(sum / (double)n);
    }
}

// ----------------------------------------------------------------------------
// cluster means (exact fp64 sums, one fp32 rounding); empty clusters untouched
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_segmean(const uint16_t* __restrict__ X,
                                                 const int32_t* __restrict__ sorted,
                                                 const int32_t* __restrict__ count,
                                                 const int32_t* __restrict__ cstart,
                                                 float* __restrict__ cent, int N, int C,
                                                 int zero_empty) {
    constexpr int CH = D / 8;                 // 16-byte chunks per row
    constexpr int ST = 256 / CH;              // token streams
    __shared__ double red[ST][D];
    const int c = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int n = count[bh * C + c];
    if (n == 0) {
        // an empty cluster keeps its previous centroid, or (no previous one:
        // an empty tile) gets zeros
        if (zero_empty && tid < D) cent[(bh * C + c) * (int64_t)D + tid] = 0.f;
        return;
    }
    const int s0 = cstart[bh * C + c];
    const int ch = tid % CH, st = tid / CH;
    const int32_t* srt = sorted + bh * N + s0;
    const uint16_t* Xh = X + bh * N * (int64_t)D + ch * 8;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto add = [&](uint4 v) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)__uint_as_float(w[e] << 16);
            acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xffff0000u);
        }
    };
    // the sums are exact, so the order of the additions is free: four rows in
    // flight per thread hide the index -> row load latency
    constexpr int U = 4;
    int r = st;
    for (; r + (U - 1) * ST < n; r += U * ST) {
        int tok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) tok[u] = srt[r + u * ST];
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const uint4*>(Xh + (int64_t)tok[u] * D);
#pragma unroll
        for (int u = 0; u < U; ++u) add(v[u]);
    }
    for (; r < n; r += ST) add(*reinterpret_cast<const uint4*>(Xh + (int64_t)srt[r] * D));
#pragma unroll
    for (int e = 0; e < 8; ++e) red[st][ch * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        double s = 0.0;
        for (int k = 0; k < ST; ++k) s += red[k][tid];
        cent[(bh * C + c) * (int64_t)D + tid] = (float)(s / (double)n);
    }
}

// ----------------------------------------------------------------------------
// cluster means from tensors already in the padded layout (a call that reuses
// the partition): cluster c's tokens are the first count[c] rows of its
// blocks, which start after the blocks of the clusters before it
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_cmean_padded(const uint16_t* __restrict__ Xp,
                                                      const int32_t* __restrict__ count,
                                                      float* __restrict__ cent, int64_t np, int C,
                                                      int block) {
    constexpr int CH = D / 8;
    constexpr int ST = 256 / CH;
    __shared__ double red[ST][D];
    __shared__ int32_t wpart[4];
    const int c = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int32_t* cnt = count + bh * C;
    int32_t part = 0;
    for (int k = tid; k < c; k += 256) part += (cnt[k] + block - 1) / block;
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) wpart[wid] = part;
    __syncthreads();
    const int64_t first = (int64_t)(wpart[0] + wpart[1] + wpart[2] + wpart[3]) * block;
    const int n = cnt[c];
    if (n == 0) return;
    const int ch = tid % CH, st = tid / CH;
    const uint16_t* src = Xp + (bh * np + first) * D + ch * 8;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int r = st; r < n; r += ST) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + (int64_t)r * D);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)__uint_as_float(w[e] << 16);
            acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[st][ch * 8 + e] = acc[e];
    __syncthreads();
    if (tid < D) {
        double s = 0.0;
        for (int k = 0; k < ST; ++k) s += red[k][tid];
        cent[(bh * C + c) * (int64_t)D + tid] = (float)(s / (double)n);
    }
}

// ----------------------------------------------------------------------------
// padded layout of one side
// ----------------------------------------------------------------------------
// One thread per padded slot (grid: slot tiles x heads); every slot and block
// entry is written exactly once.  Each workgroup first scans the clusters'
// block counts (C <= 1024, one per thread) for the first block of each.
__global__ __launch_bounds__(kTok) void k_layout(const int32_t* __restrict__ sorted,
                                                 const int32_t* __restrict__ count,
                                                 const int32_t* __restrict__ cstart,
                                                 int32_t* __restrict__ order,
                                                 int32_t* __restrict__ blk_cluster,
                                                 int32_t* __restrict__ blk_count, int N, int C,
                                                 int block, int nbp) {
    __shared__ int32_t bstart[kCmax], nblk_s[kCmax], cst[kCmax], cnt[kCmax];
    __shared__ int32_t wsum[kTok / 64];
    const int64_t bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int n = tid < C ? count[bh * C + tid] : 0;
    const int nblk = (n + block - 1) / block;
    int32_t x = nblk;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < wid; ++w) before += wsum[w];
    if (tid < C) {
        bstart[tid] = before + x - nblk;
        nblk_s[tid] = nblk;
        cst[tid] = cstart[bh * C + tid];
        cnt[tid] = n;
    }
    __syncthreads();
    const int64_t np = (int64_t)nbp * block;
    const int64_t p = (int64_t)blockIdx.x * kTok + tid;
    if (p >= np) return;
    const int j = (int)(p / block);
    // the cluster owning block j: the last c with bstart[c] <= j (an empty
    // cluster shares its start with the next one, which comes later)
    int lo = 0, hi = C - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (bstart[mid] <= j) lo = mid;
        else hi = mid - 1;
    }
    int tok = -1, bc = -1, bn = 0;
    if (j < bstart[lo] + nblk_s[lo]) {
        const int off = (int)(p - (int64_t)bstart[lo] * block);
        if (off < cnt[lo]) tok = sorted[bh * N + cst[lo] + off];
        bc = lo;
        const int rest = cnt[lo] - (j - bstart[lo]) * block;
        bn = rest < block ? rest : block;
    }
    order[bh * np + p] = tok;
    if (p % block == 0) {
        blk_cluster[bh * nbp + j] = bc;
        blk_count[bh * nbp + j] = bn;
    }
}

// ----------------------------------------------------------------------------
// into / out of the padded layout (16-byte pieces of rows)
// ----------------------------------------------------------------------------
template <int D>
__global__ void k_gather_rows(const uint16_t* __restrict__ src, const int32_t* __restrict__ order,
                              uint16_t* __restrict__ dst, int N, int64_t np) {
    constexpr int CH = D / 8;
    const int64_t bh = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= np * CH) return;
    const int64_t p = i / CH;
    const int ch = (int)(i % CH);
    const int tok = order[bh * np + p];
    uint4 v = make_uint4(0, 0, 0, 0);
    if (tok >= 0) v = *reinterpret_cast<const uint4*>(src + (bh * N + tok) * (int64_t)D + ch * 8);
    *reinterpret_cast<uint4*>(dst + (bh * np + p) * D + ch * 8) = v;
}

template <int D>
__global__ void k_scatter_rows(const uint16_t* __restrict__ src, const int32_t* __restrict__ order,
                               uint16_t* __restrict__ dst, const float* __restrict__ lse_src,
                               float* __restrict__ lse_dst, int N, int64_t np) {
    constexpr int CH = D / 8;
    const int64_t bh = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= np * CH) return;
    const int64_t p = i / CH;
    const int ch = (int)(i % CH);
    const int tok = order[bh * np + p];
    if (tok < 0) return;
    *reinterpret_cast<uint4*>(dst + (bh * N + tok) * (int64_t)D + ch * 8) =
        *reinterpret_cast<const uint4*>(src + (bh * np + p) * D + ch * 8);
    if (lse_src && ch == 0) lse_dst[bh * N + tok] = lse_src[bh * np + p];
}

// ----------------------------------------------------------------------------
// cluster-level selection
// ----------------------------------------------------------------------------
constexpr int kSelThreads = 256;

__device__ __forceinline__ uint32_t ordered_f32(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0) u = 0;                     // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct CSelArgs {
    const float* S;             // [BH][C][C]
    const int32_t* nk;          // [BH][C] key-cluster sizes
    const int64_t* budget;      // [H] token budget (TOPK)
    uint8_t* keep;              // [BH][C][C]
    int32_t C, Cpad, H, rule, diag;
    float mass;
    // tile mode with a SICS ticket: key tile j of head bh may be kept only if
    // coh[(bh * n_shapes + shape_idx[bh]) * C + j] >= ticket (else coh null)
    const double* coh;
    const int32_t* shape_idx;
    int32_t n_shapes;
    double ticket;
};

__global__ __launch_bounds__(kSelThreads) void k_cselect(CSelArgs a) {
    extern __shared__ unsigned char smem[];
    unsigned long long* key = reinterpret_cast<unsigned long long*>(smem);   // [Cpad]
    double* cum = reinterpret_cast<double*>(smem);                           // aliases key
    int32_t* ord = reinterpret_cast<int32_t*>(smem + (size_t)a.Cpad * 8);    // [Cpad]
    __shared__ int32_t s_live, s_cut;
    const int64_t row = blockIdx.x;                // bh * C + cq
    const int cq = (int)(row % a.C);
    const int64_t bh = row / a.C;
    const int h = (int)(bh % a.H);
    const int tid = threadIdx.x;
    const float* S = a.S + row * a.C;
    const int32_t* nk = a.nk + bh * a.C;
    if (tid == 0) { s_live = 0; s_cut = 0; }
    __syncthreads();
    const double* coh = nullptr;
    if (a.coh) {
        int sh = a.shape_idx[bh];
        sh = sh < 0 ? 0 : (sh >= a.n_shapes ? a.n_shapes - 1 : sh);
        coh = a.coh + (bh * a.n_shapes + sh) * a.C;
    }
    int live_local = 0;
    for (int j = tid; j < a.Cpad; j += kSelThreads) {
        // a live key cluster has tokens and, with a ticket, coherent keys
        const bool live = j < a.C && nk[j] > 0 && (!coh || coh[j] >= a.ticket);
        live_local += live;
        key[j] = live ? ((unsigned long long)(~ordered_f32(S[j])) << 32) | (uint32_t)j : ~0ull;
    }
    if (live_local) atomicAdd(&s_live, live_local);
    __syncthreads();
    for (int size = 2; size <= a.Cpad; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < a.Cpad / 2; t += kSelThreads) {
                const int lo = 2 * t - (t & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const unsigned long long x = key[lo], y = key[hi];
                if ((x > y) == up) { key[lo] = y; key[hi] = x; }
            }
            __syncthreads();
        }
    }
    const int live = s_live;
    for (int r = tid; r < live; r += kSelThreads) ord[r] = (int32_t)(key[r] & 0xffffffffu);
    __syncthreads();
    if (a.rule == SA_RULE_TOPK) {
        // the shortest rank prefix whose token count reaches the budget (all
        // of them if none does): counts in rank order to LDS, then one wave
        // scans them in 64 consecutive chunks (integer sums: exact in any order)
        int64_t* wc = reinterpret_cast<int64_t*>(smem);        // the keys are dead
        for (int r = tid; r < live; r += kSelThreads) wc[r] = nk[ord[r]];
        __syncthreads();
        if (tid < 64) {
            const int64_t budget = a.budget[h];
            const int per = (live + 63) / 64;
            const int r0 = min(tid * per, live), r1 = min(r0 + per, live);
            int64_t own = 0;
            for (int r = r0; r < r1; ++r) own += wc[r];
            // exclusive prefix of the chunk sums over the lanes
            int64_t incl = own;
            for (int off = 1; off < 64; off <<= 1) {
                const int64_t o = __shfl_up(incl, off, 64);
                if (tid >= off) incl += o;
            }
            int64_t run = incl - own;
            int m = live;
            for (int r = r0; r < r1; ++r) {
                run += wc[r];
                if (run >= budget) { m = r + 1; break; }
            }
            for (int off = 32; off > 0; off >>= 1) m = min(m, __shfl_xor(m, off, 64));
            if (tid == 0) s_cut = m;
        }
    } else {
        // weight n_b exp(S_b - S_max) in fp64, summed sequentially in rank order
        const double smax = live > 0 ? (double)S[ord[0]] : 0.0;
        for (int r = tid; r < live; r += kSelThreads)
            cum[r] = (double)nk[ord[r]] * exp((double)S[ord[r]] - smax);
        __syncthreads();
        if (tid == 0 && live > 0) {
            double run = 0.0;
            for (int r = 0; r < live; ++r) { run += cum[r]; cum[r] = run; }
            const double thr = (double)a.mass * cum[live - 1];
            int m = live;
            for (int r = 0; r < live; ++r)
                if (cum[r] >= thr) { m = r + 1; break; }
            s_cut = m;
        }
    }
    __syncthreads();
    const int m = s_cut;
    uint8_t* out = a.keep + row * a.C;
    for (int j = tid; j < a.C; j += kSelThreads) out[j] = 0;
    __syncthreads();
    for (int r = tid; r < m; r += kSelThreads) out[ord[r]] = 1;
    if (tid == 0 && a.diag && nk[cq] > 0) out[cq] = 1;
}

// token budgets of a chunk of heads, passed by value
constexpr int kBudgetChunk = 64;
struct BudgetChunk {
    int64_t v[kBudgetChunk];
};
__global__ void k_set_budget(int64_t* __restrict__ dst, BudgetChunk c, int n) {
    if ((int)threadIdx.x < n) dst[threadIdx.x] = c.v[threadIdx.x];
}

// blocks kept by every row of the padded layout (one wave per row)
__global__ __launch_bounds__(256) void k_crow_count(const uint8_t* __restrict__ keep,
                                                    const int32_t* __restrict__ nk,
                                                    const int32_t* __restrict__ q_blk,
                                                    int32_t* __restrict__ counts, int64_t rows,
                                                    int nbp, int C, int block) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;
    const int64_t bh = r / nbp;
    const int cq = q_blk[r];
    int32_t n = 0;
    if (cq >= 0) {
        const uint8_t* kr = keep + (bh * C + cq) * C;
        for (int c = lane; c < C; c += 64)
            if (kr[c]) n += (nk[bh * C + c] + block - 1) / block;
    }
    for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off, 64);
    if (lane == 0) counts[r] = n;
}

// one wave per row: the blocks of the kept key clusters, ascending
__global__ __launch_bounds__(256) void k_crow_fill(const uint8_t* __restrict__ keep,
                                                   const int32_t* __restrict__ nk,
                                                   const int32_t* __restrict__ q_blk,
                                                   const int32_t* __restrict__ row_ptr,
                                                   int32_t* __restrict__ col_idx, int64_t rows,
                                                   int nbp, int C, int block) {
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= rows) return;
    const int64_t bh = r / nbp;
    const int cq = q_blk[r];
    if (cq < 0) return;
    const uint8_t* kr = keep + (bh * C + cq) * C;
    int32_t bbase = 0;                 // first block of cluster c0 + lane (all clusters)
    int32_t obase = row_ptr[r];        // next output slot
    for (int c0 = 0; c0 < C; c0 += 64) {
        const int c = c0 + lane;
        const int nb_c = c < C ? (nk[bh * C + c] + block - 1) / block : 0;
        const int kept = (c < C && kr[c]) ? nb_c : 0;
        int32_t xb = nb_c, xk = kept;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t yb = __shfl_up(xb, off, 64), yk = __shfl_up(xk, off, 64);
            if (lane >= off) { xb += yb; xk += yk; }
        }
        const int32_t first = bbase + xb - nb_c;
        const int32_t out = obase + xk - kept;
        for (int k = 0; k < kept; ++k) col_idx[out + k] = first + k;
        bbase += __shfl(xb, 63, 64);
        obase += __shfl(xk, 63, 64);
    }
}

// compensation statistics per block: the cluster's centroid key and its value
// mean times the block's token count
template <int D>
__global__ void k_block_comp(const float* __restrict__ k_cent, const float* __restrict__ v_cent,
                             const int32_t* __restrict__ k_blk, const int32_t* __restrict__ k_cnt,
                             float* __restrict__ k_mean, float* __restrict__ v_sum, int nbp, int C) {
    const int j = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int d = threadIdx.x;
    const int c = k_blk[bh * nbp + j];
    const int n = k_cnt[bh * nbp + j];
    float km = 0.f, vs = 0.f;
    if (c >= 0 && n > 0) {
        km = k_cent[(bh * C + c) * (int64_t)D + d];
        vs = (float)n * v_cent[(bh * C + c) * (int64_t)D + d];
    }
    k_mean[(bh * nbp + j) * (int64_t)D + d] = km;
    v_sum[(bh * nbp + j) * (int64_t)D + d] = vs;
}

// ----------------------------------------------------------------------------
// host side
// ----------------------------------------------------------------------------
struct ClusterWs {
    size_t assign[2], sorted[2], hist, off, cstart[2], centT, bias, psum, pcnt, total;
};

inline int padded_c(int C) { return (C + kAsgIlp - 1) / kAsgIlp * kAsgIlp; }

// workgroups per head of k_assign_mx: about one per CU over all heads (its
// LDS holds one per CU), at least 16 token groups each, at most kAmxWgTarget
inline int amx_wg_per_head(const Geometry& g) {
    const int64_t groups = ceil_div(g.N, 32);
    const int64_t target = std::max<int64_t>(1, kAmxWgTarget / std::max<int64_t>(1, g.BH()));
    return (int)std::min<int64_t>({target, ceil_div(groups, kAmxWaves), (int64_t)kAmxWgTarget});
}

// the rounds form their means from unsorted partial sums (C <= 64)
inline bool fused_means(const sa_cluster_spec& cs) {
    return cs.mode != SA_CLUSTER_TILES && cs.n_clusters <= kAmxC;
}

ClusterWs cluster_ws(const Geometry& g, const sa_cluster_spec& cs) {
    const int C = cs.n_clusters;
    ClusterWs w{};
    const int64_t ntiles = ceil_div(g.N, kTok);
    size_t o = 0;
    for (int s = 0; s < 2; ++s) {
        w.assign[s] = o; o = align_up(o + (size_t)g.BH() * g.N * 4, 256);
        w.sorted[s] = o; o = align_up(o + (size_t)g.BH() * g.N * 4, 256);
        w.cstart[s] = o; o = align_up(o + (size_t)g.BH() * C * 4, 256);
    }
    w.hist = o; o = align_up(o + (size_t)g.BH() * ntiles * C * 4, 256);
    w.off = o; o = align_up(o + (size_t)g.BH() * ntiles * C * 4, 256);
    w.centT = o; o = align_up(o + (size_t)g.BH() * g.d * padded_c(C) * 4, 256);
    w.bias = o; o = align_up(o + (size_t)g.BH() * padded_c(C) * 4, 256);
    if (fused_means(cs)) {
        const size_t parts = (size_t)g.BH() * amx_wg_per_head(g);
        w.psum = o; o = align_up(o + parts * kAmxC * g.d * 8, 256);
        w.pcnt = o; o = align_up(o + parts * kAmxC * 4, 256);
    }
    w.total = o;
    return w;
}

template <int D>
sa_status segmean(const Geometry& g, int C, const uint16_t* X, const int32_t* sorted,
                  const int32_t* count, const int32_t* cstart, float* cent, hipStream_t st,
                  int zero_empty = 0) {
    hipLaunchKernelGGL((k_segmean<D>), dim3(C, (unsigned)g.BH()), dim3(256), 0, st, X, sorted,
                       count, cstart, cent, g.N, C, zero_empty);
    return hip_check(hipGetLastError(), "k_segmean launch");
}

// sorts side s by its assignment (sorted order, counts, cluster starts)
sa_status sort_side(const Geometry& g, int C, char* ws, const ClusterWs& w, int s, int32_t* count,
                    hipStream_t st) {
    const int ntiles = (int)ceil_div(g.N, kTok);
    const int32_t* assign = reinterpret_cast<const int32_t*>(ws + w.assign[s]);
    int32_t* sorted = reinterpret_cast<int32_t*>(ws + w.sorted[s]);
    int32_t* hist = reinterpret_cast<int32_t*>(ws + w.hist);
    int32_t* off = reinterpret_cast<int32_t*>(ws + w.off);
    int32_t* cstart = reinterpret_cast<int32_t*>(ws + w.cstart[s]);
    hipLaunchKernelGGL(k_hist, dim3(ntiles, (unsigned)g.BH()), dim3(kTok), 0, st, assign, hist, g.N,
                       C, ntiles);
    sa_status e = hip_check(hipGetLastError(), "k_hist launch");
    if (e != SA_OK) return e;
    hipLaunchKernelGGL(k_hist_scan, dim3((unsigned)g.BH()), dim3(kTok), 0, st, hist, off, count,
                       cstart, C, ntiles);
    if ((e = hip_check(hipGetLastError(), "k_hist_scan launch")) != SA_OK) return e;
    hipLaunchKernelGGL(k_sort_scatter, dim3(ntiles, (unsigned)g.BH()), dim3(kTok), 0, st, assign,
                       off, sorted, g.N, C, ntiles);
    return hip_check(hipGetLastError(), "k_sort_scatter launch");
}

// sorts side s by its assignment and refreshes its centroids
template <int D>
sa_status sort_and_mean(const Geometry& g, int C, char* ws, const ClusterWs& w, int s,
                        const uint16_t* X, int32_t* count, float* cent, hipStream_t st,
                        int zero_empty = 0) {
    sa_status e = sort_side(g, C, ws, w, s, count, st);
    if (e != SA_OK) return e;
    return segmean<D>(g, C, X, reinterpret_cast<const int32_t*>(ws + w.sorted[s]), count,
                      reinterpret_cast<const int32_t*>(ws + w.cstart[s]), cent, st, zero_empty);
}

// means of side s from the partial sums of the last assignment (C <= 64)
template <int D>
sa_status partial_means(const Geometry& g, int C, char* ws, const ClusterWs& w, int32_t* count,
                        float* cent, hipStream_t st) {
    hipLaunchKernelGGL((k_clmean<D>), dim3((unsigned)C, (unsigned)g.BH()), dim3(D), 0, st,
                       reinterpret_cast<const double*>(ws + w.psum),
                       reinterpret_cast<const int32_t*>(ws + w.pcnt), amx_wg_per_head(g), cent,
                       count, C);
    return hip_check(hipGetLastError(), "k_clmean launch");
}

// means and sizes of the initial chunk partition (no assignment needed)
template <int D>
sa_status chunk_means(const Geometry& g, int C, const uint16_t* X, int32_t* count, float* cent,
                      hipStream_t st) {
    hipLaunchKernelGGL((k_chunkmean<D>), dim3((unsigned)C, (unsigned)g.BH()), dim3(256), 0, st, X,
                       cent, count, g.N, C);
    return hip_check(hipGetLastError(), "k_chunkmean launch");
}

template <int D>
sa_status assign_side(const Geometry& g, int C, char* ws, const ClusterWs& w, int s,
                      const uint16_t* X, const float* cent, int kmeans, hipStream_t st) {
    int32_t* assign = reinterpret_cast<int32_t*>(ws + w.assign[s]);
    if (C <= kAmxC) {
        // about one workgroup per CU, spread over the heads; each stages its
        // head's centroids once, serves many token groups and leaves the
        // partial cluster sums of its tokens
        hipLaunchKernelGGL((k_assign_mx<D>), dim3((unsigned)amx_wg_per_head(g), (unsigned)g.BH()),
                           dim3(64 * kAmxWaves), 0, st, X, cent, assign,
                           reinterpret_cast<double*>(ws + w.psum),
                           reinterpret_cast<int32_t*>(ws + w.pcnt), g.N, C, kmeans);
        return hip_check(hipGetLastError(), "k_assign_mx launch");
    }
    float* centT = reinterpret_cast<float*>(ws + w.centT);
    float* bias = reinterpret_cast<float*>(ws + w.bias);
    const int Cp = padded_c(C);
    hipLaunchKernelGGL((k_cent_prep<D>), dim3((unsigned)ceil_div((int64_t)D * Cp, 256), (unsigned)g.BH()),
                       dim3(256), 0, st, cent, centT, bias, C, Cp, kmeans);
    sa_status e = hip_check(hipGetLastError(), "k_cent_prep launch");
    if (e != SA_OK) return e;
    hipLaunchKernelGGL((k_assign<D>), dim3((unsigned)ceil_div(g.N, kAsgThreads), (unsigned)g.BH()),
                       dim3(kAsgThreads), 0, st, X, centT, bias, assign, g.N, Cp);
    return hip_check(hipGetLastError(), "k_assign launch");
}

template <int D>
sa_status cluster_t(const Geometry& g, const sa_cluster_spec& cs, const uint16_t* Q,
                    const uint16_t* K, const uint16_t* V, ClusterOut o, char* ws, hipStream_t st) {
    const int C = cs.n_clusters;
    const ClusterWs w = cluster_ws(g, cs);
    const bool fused = fused_means(cs);
    sa_status e;
    if (cs.mode == SA_CLUSTER_TILES) {
        // the partition is geometric: the tiles of each head's chosen shape,
        // the same for queries and keys
        for (int s = 0; s < 2; ++s) {
            if ((e = launch_tile_assign(g, cs, reinterpret_cast<int32_t*>(ws + w.assign[s]), st)) != SA_OK)
                return e;
            if ((e = sort_and_mean<D>(g, C, ws, w, s, s ? K : Q, s ? o.k_count : o.q_count,
                                      s ? o.k_cent : o.q_cent, st, 1)) != SA_OK)
                return e;
        }
    }
    // initial partition of both sides and its centroids: C equal chunks of
    // the token order (with partial-sum means every round reassigns both
    // sides before anything reads an assignment, so none is written)
    for (int s = 0; s < 2 && cs.mode != SA_CLUSTER_TILES; ++s) {
        if (fused) {
            e = chunk_means<D>(g, C, s ? K : Q, s ? o.k_count : o.q_count, s ? o.k_cent : o.q_cent, st);
        } else {
            hipLaunchKernelGGL(k_chunk_assign, dim3((unsigned)ceil_div(g.N, 256), (unsigned)g.BH()),
                               dim3(256), 0, st, reinterpret_cast<int32_t*>(ws + w.assign[s]), g.N, C);
            if ((e = hip_check(hipGetLastError(), "k_chunk_assign launch")) != SA_OK) return e;
            e = sort_and_mean<D>(g, C, ws, w, s, s ? K : Q, s ? o.k_count : o.q_count,
                                 s ? o.k_cent : o.q_cent, st);
        }
        if (e != SA_OK) return e;
    }
    // a side's means after its assignment: from the partial sums the
    // assignment left (C <= 64), else by sorting
    auto means = [&](int s, const uint16_t* X, int32_t* count, float* cent) -> sa_status {
        return fused ? partial_means<D>(g, C, ws, w, count, cent, st)
                     : sort_and_mean<D>(g, C, ws, w, s, X, count, cent, st);
    };
    for (int it = 0; it < (cs.mode == SA_CLUSTER_TILES ? 0 : cs.iters); ++it) {
        if (cs.mode == SA_CLUSTER_COCLUSTER) {
            // keys by affinity to the query centroids, then queries by affinity
            // to the refreshed key centroids
            if ((e = assign_side<D>(g, C, ws, w, 1, K, o.q_cent, 0, st)) != SA_OK) return e;
            if ((e = means(1, K, o.k_count, o.k_cent)) != SA_OK) return e;
            if ((e = assign_side<D>(g, C, ws, w, 0, Q, o.k_cent, 0, st)) != SA_OK) return e;
            if ((e = means(0, Q, o.q_count, o.q_cent)) != SA_OK) return e;
        } else {
            for (int s = 0; s < 2; ++s) {
                const uint16_t* X = s ? K : Q;
                float* cent = s ? o.k_cent : o.q_cent;
                if ((e = assign_side<D>(g, C, ws, w, s, X, cent, 1, st)) != SA_OK) return e;
                if ((e = means(s, X, s ? o.k_count : o.q_count, cent)) != SA_OK) return e;
            }
        }
    }
    // the final partition in sorted order (the layout and the value means read it)
    for (int s = 0; s < 2 && fused; ++s)
        if ((e = sort_side(g, C, ws, w, s, s ? o.k_count : o.q_count, st)) != SA_OK) return e;
    if (o.v_cent) {
        if ((e = segmean<D>(g, C, V, reinterpret_cast<const int32_t*>(ws + w.sorted[1]), o.k_count,
                            reinterpret_cast<const int32_t*>(ws + w.cstart[1]), o.v_cent, st,
                            cs.mode == SA_CLUSTER_TILES)) != SA_OK)
            return e;
    }
    const int nbp = padded_block_count(g, cs);
    for (int s = 0; s < 2; ++s) {
        const unsigned tiles = (unsigned)ceil_div((int64_t)nbp * g.block, kTok);
        hipLaunchKernelGGL(k_layout, dim3(tiles, (unsigned)g.BH()), dim3(kTok), 0, st,
                           reinterpret_cast<const int32_t*>(ws + w.sorted[s]),
                           s ? o.k_count : o.q_count,
                           reinterpret_cast<const int32_t*>(ws + w.cstart[s]),
                           s ? o.k_order : o.q_order, s ? o.k_blk : o.q_blk,
                           s ? o.k_cnt : o.q_cnt, g.N, C, g.block, nbp);
        if ((e = hip_check(hipGetLastError(), "k_layout launch")) != SA_OK) return e;
    }
    return SA_OK;
}

}  // namespace

int padded_block_count(const Geometry& g, const sa_cluster_spec& cs) {
    return cs.mode == SA_CLUSTER_TILES ? cs.n_clusters
                                       : (int)ceil_div(g.N, g.block) + cs.n_clusters;
}

size_t cluster_workspace_bytes(const Geometry& g, const sa_cluster_spec& cs) {
    const size_t a = cluster_ws(g, cs).total;
    if (cs.mode != SA_CLUSTER_TILES) return a;
    const size_t b = sics_workspace_bytes(g, cs);     // sparse_attn_sics shares the buffer
    return a > b ? a : b;
}

sa_status launch_cluster(const Geometry& g, const sa_cluster_spec& cs, const uint16_t* Q,
                         const uint16_t* K, const uint16_t* V, const ClusterOut& o, char* ws,
                         hipStream_t st) {
    return g.d == 128 ? cluster_t<128>(g, cs, Q, K, V, o, ws, st)
                      : cluster_t<64>(g, cs, Q, K, V, o, ws, st);
}

sa_status launch_cluster_gather(const Geometry& g, const sa_cluster_spec& cs, const int32_t* order,
                                const uint16_t* src, uint16_t* dst, hipStream_t st) {
    const int64_t np = (int64_t)padded_block_count(g, cs) * g.block;
    const unsigned nblk = (unsigned)ceil_div(np * (g.d / 8), 256);
    if (g.d == 128)
        hipLaunchKernelGGL((k_gather_rows<128>), dim3(nblk, (unsigned)g.BH()), dim3(256), 0, st, src,
                           order, dst, g.N, np);
    else
        hipLaunchKernelGGL((k_gather_rows<64>), dim3(nblk, (unsigned)g.BH()), dim3(256), 0, st, src,
                           order, dst, g.N, np);
    return hip_check(hipGetLastError(), "k_gather_rows launch");
}

sa_status launch_cluster_scatter(const Geometry& g, const sa_cluster_spec& cs, const int32_t* order,
                                 const uint16_t* src, uint16_t* dst, const float* lse_src,
                                 float* lse_dst, hipStream_t st) {
    const int64_t np = (int64_t)padded_block_count(g, cs) * g.block;
    const unsigned nblk = (unsigned)ceil_div(np * (g.d / 8), 256);
    if (g.d == 128)
        hipLaunchKernelGGL((k_scatter_rows<128>), dim3(nblk, (unsigned)g.BH()), dim3(256), 0, st, src,
                           order, dst, lse_src, lse_dst, g.N, np);
    else
        hipLaunchKernelGGL((k_scatter_rows<64>), dim3(nblk, (unsigned)g.BH()), dim3(256), 0, st, src,
                           order, dst, lse_src, lse_dst, g.N, np);
    return hip_check(hipGetLastError(), "k_scatter_rows launch");
}

size_t cluster_select_workspace_bytes(const Geometry& g, const sa_cluster_spec& cs) {
    const int C = cs.n_clusters;
    const int nbp = padded_block_count(g, cs);
    size_t o = 0;
    o = align_up(o + (size_t)g.BH() * C * C * 4, 256);      // scores
    o = align_up(o + (size_t)g.BH() * C * C, 256);          // keep flags
    o = align_up(o + (size_t)g.BH() * nbp * 4, 256);        // row counts
    o = align_up(o + (size_t)g.H * 8, 256);                 // token budgets
    return o;
}

sa_status launch_cluster_select(const Geometry& g, const sa_cluster_spec& cs, const ClusterSel& a,
                                const int64_t* budget_host, char* ws, hipStream_t st) {
    const int C = cs.n_clusters;
    const int nbp = padded_block_count(g, cs);
    size_t o = 0;
    float* S = reinterpret_cast<float*>(ws + o);
    o = align_up(o + (size_t)g.BH() * C * C * 4, 256);
    uint8_t* keep = reinterpret_cast<uint8_t*>(ws + o);
    o = align_up(o + (size_t)g.BH() * C * C, 256);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + o);
    o = align_up(o + (size_t)g.BH() * nbp * 4, 256);
    int64_t* budget = reinterpret_cast<int64_t*>(ws + o);
    if (a.scores) S = a.scores;
    sa_status e;
    if ((e = launch_pooled_scores(g.d, a.q_cent, a.k_cent, S, C, g.scale, g.BH(), st)) != SA_OK) return e;
    if (a.rule == SA_RULE_TOPK) {
        for (int h0 = 0; h0 < g.H; h0 += kBudgetChunk) {
            BudgetChunk c{};
            const int n = g.H - h0 < kBudgetChunk ? g.H - h0 : kBudgetChunk;
            for (int t = 0; t < n; ++t) c.v[t] = budget_host[h0 + t];
            hipLaunchKernelGGL(k_set_budget, dim3(1), dim3(kBudgetChunk), 0, st, budget + h0, c, n);
            if ((e = hip_check(hipGetLastError(), "k_set_budget launch")) != SA_OK) return e;
        }
    }
    CSelArgs ca{};
    ca.S = S; ca.nk = a.k_count; ca.budget = budget; ca.keep = keep;
    ca.C = C; ca.H = g.H; ca.rule = a.rule; ca.diag = a.diag; ca.mass = a.mass;
    if (cs.mode == SA_CLUSTER_TILES && cs.tile_coherence) {
        ca.coh = cs.tile_coherence;
        ca.shape_idx = cs.shape_idx;
        ca.n_shapes = cs.n_shapes;
        ca.ticket = (double)cs.ticket;
    }
    int cpad = 2;
    while (cpad < C) cpad <<= 1;
    ca.Cpad = cpad;
    hipLaunchKernelGGL(k_cselect, dim3((unsigned)(g.BH() * C)), dim3(kSelThreads), (size_t)cpad * 12, st, ca);
    if ((e = hip_check(hipGetLastError(), "k_cselect launch")) != SA_OK) return e;
    const int64_t rows = g.BH() * nbp;
    hipLaunchKernelGGL(k_crow_count, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, st, keep,
                       a.k_count, a.q_blk, counts, rows, nbp, C, g.block);
    if ((e = hip_check(hipGetLastError(), "k_crow_count launch")) != SA_OK) return e;
    if ((e = launch_row_scan(counts, a.row_ptr, rows, st)) != SA_OK) return e;
    hipLaunchKernelGGL(k_crow_fill, dim3((unsigned)ceil_div(rows, 4)), dim3(256), 0, st, keep,
                       a.k_count, a.q_blk, a.row_ptr, a.col_idx, rows, nbp, C, g.block);
    if ((e = hip_check(hipGetLastError(), "k_crow_fill launch")) != SA_OK) return e;
    if (a.k_mean) {
        if (g.d == 128)
            hipLaunchKernelGGL((k_block_comp<128>), dim3(nbp, (unsigned)g.BH()), dim3(128), 0, st,
                               a.k_cent, a.v_cent, a.k_blk, a.k_cnt, a.k_mean, a.v_sum, nbp, C);
        else
            hipLaunchKernelGGL((k_block_comp<64>), dim3(nbp, (unsigned)g.BH()), dim3(64), 0, st,
                               a.k_cent, a.v_cent, a.k_blk, a.k_cnt, a.k_mean, a.v_sum, nbp, C);
        if ((e = hip_check(hipGetLastError(), "k_block_comp launch")) != SA_OK) return e;
    }
    return SA_OK;
}

sa_status launch_cluster_centroids(const Geometry& g, const sa_cluster_spec& cs, const uint16_t* Kp,
                                   const uint16_t* Vp, const int32_t* k_count,
                                   const int32_t* k_blk, const int32_t* k_cnt, float* k_cent,
                                   float* v_cent, float* k_mean, float* v_sum, hipStream_t st) {
    const int C = cs.n_clusters;
    const int nbp = padded_block_count(g, cs);
    const int64_t np = (int64_t)nbp * g.block;
    const dim3 grid((unsigned)C, (unsigned)g.BH());
    sa_status e;
    for (int s = 0; s < 2; ++s) {
        const uint16_t* X = s ? Vp : Kp;
        float* out = s ? v_cent : k_cent;
        if (g.d == 128)
            hipLaunchKernelGGL((k_cmean_padded<128>), grid, dim3(256), 0, st, X, k_count, out, np, C, g.block);
        else
            hipLaunchKernelGGL((k_cmean_padded<64>), grid, dim3(256), 0, st, X, k_count, out, np, C, g.block);
        if ((e = hip_check(hipGetLastError(), "k_cmean_padded launch")) != SA_OK) return e;
    }
    if (g.d == 128)
        hipLaunchKernelGGL((k_block_comp<128>), dim3(nbp, (unsigned)g.BH()), dim3(128), 0, st,
                           k_cent, v_cent, k_blk, k_cnt, k_mean, v_sum, nbp, C);
    else
        hipLaunchKernelGGL((k_block_comp<64>), dim3(nbp, (unsigned)g.BH()), dim3(64), 0, st,
                           k_cent, v_cent, k_blk, k_cnt, k_mean, v_sum, nbp, C);
    return hip_check(hipGetLastError(), "k_block_comp launch");
}

}  // namespace sa
