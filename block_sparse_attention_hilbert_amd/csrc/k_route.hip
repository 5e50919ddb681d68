// Error-aware routing keys for gfx950 (SVG-EAR page, section 2B).
//
// For every query block i (represented by its mean qbar_i) and KV block j,
// with the logits l_t = scale * qbar_i . k_t of the n_j tokens of block j and
// m = max_t l_t, the key is
//
//   key[i,j] = ln || A - Ahat ||_2 + m - ln n_j
//   A    = sum_t exp(l_t - m) v_t              (what block j contributes)
//   Ahat = n_j exp(S_ij - m) vbar_j            (its centroid replacement)
//
// S_ij is the pooled score of the score-based rules and vbar_j = v_sum_j / n_j,
// so Ahat is exactly the term the centroid compensation adds for a skipped
// block.  Keeping the blocks with the largest keys drops the blocks whose
// centroid replacement is most accurate per token of work saved.
//
// The work is one small dense attention of the query means against every key:
// two contractions per block pair, both on v_mfma_f32_32x32x16_bf16.
//   * L^T = K_j qbar^T: K (bf16, exact) is the A operand; qbar (fp32) enters
//     as the sum of two bf16 operands, hi = bf16(qbar), lo = bf16(qbar - hi),
//     which carries 16 significant bits.
//   * A^T = V_j^T W^T: V^T (bf16, exact, re-laid out per block) is the A
//     operand; the weights W = exp(l - m) enter as a hi/lo bf16 pair.
// Each lane owns one query column of both products, so the max over the
// block's keys, the error sum over the channels and the key are lane-local up
// to one half-wave swap.  K rows are read in the order that puts the logits of
// one 16-key step into consecutive accumulator registers of a lane (bits 2 and
// 3 of the row index swapped), so W feeds the second product without any data
// movement between lanes.
//
// One workgroup: 4 waves x 32 query blocks, a run of RJ KV blocks of one
// (batch, head); K_j and V_j^T are staged in LDS once per KV block and shared
// by the four waves.
#include <math.h>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kQPerWave = 32;
constexpr int kQPerGroup = 4 * kQPerWave;
constexpr int RJ = 4;                       // KV blocks per workgroup

__device__ __forceinline__ uint16_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_val(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Splits 8 fp32 values into bf16 hi and lo parts (x ~= hi + lo to 2^-16 relative).
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const uint16_t h0 = bf16_rne(x[2 * p]), h1 = bf16_rne(x[2 * p + 1]);
        const uint16_t l0 = bf16_rne(x[2 * p] - bf16_val(h0));
        const uint16_t l1 = bf16_rne(x[2 * p + 1] - bf16_val(h1));
        h[p] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        l[p] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
    lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// K row order inside a 32-row tile: bits 2 and 3 of the row index swapped.
__device__ __forceinline__ int swap23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ float half_swap_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int BLK>
__global__ __launch_bounds__(kThreads, 2) void k_err(const float* __restrict__ qm,
                                                    const uint16_t* __restrict__ K,
                                                    const uint16_t* __restrict__ Vt,
                                                    const float* __restrict__ v_sum,
                                                    const float* __restrict__ S,
                                                    float* __restrict__ keys, int N, int nb,
                                                    float scale, const int32_t* __restrict__ order) {
    constexpr int KS = D / 16;            // channel steps of L^T
    constexpr int KT = BLK / 32;          // 32-key tiles
    constexpr int DT = D / 32;            // 32-channel tiles of A^T
    constexpr int KROW = D + 8;           // LDS row pitch of K (bf16)
    constexpr int VROW = BLK + 8;         // LDS row pitch of V^T (bf16)
    __shared__ uint16_t ks_lds[BLK * KROW];
    __shared__ uint16_t vs_lds[D * VROW];
    __shared__ float vbar[D];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, h = lane >> 5;
    const int64_t bh = blockIdx.z;
    const int q = blockIdx.x * kQPerGroup + wave * kQPerWave + col;
    const bool q_ok = q < nb;
    const int j0 = blockIdx.y * RJ;
    const int j1 = min(nb, j0 + RJ);
    const float c = scale * 1.44269504088896340736f;   // logits in log2 units

    // query means as hi/lo bf16 B operands, held for the whole workgroup
    bf16x8 qhi[KS], qlo[KS];
    {
        const float* qrow = qm + (bh * nb + (q_ok ? q : 0)) * (int64_t)D;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            float x[8];
            const float4 a = reinterpret_cast<const float4*>(qrow + s * 16 + 8 * h)[0];
            const float4 b = reinterpret_cast<const float4*>(qrow + s * 16 + 8 * h)[1];
            x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
            x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
            if (!q_ok) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = 0.f;
            }
            split8(x, qhi[s], qlo[s]);
        }
    }

    for (int j = j0; j < j1; ++j) {
        const int nj = min(BLK, N - j * BLK);
        __syncthreads();   // the previous block's tiles are no longer read
        {
            // key r of block j: token j*BLK + r of the block order (through
            // the token order when one is given)
            const uint16_t* src = K + bh * N * (int64_t)D;
            for (int p = tid; p < BLK * (D / 8); p += kThreads) {
                const int r = p / (D / 8), ch = p % (D / 8);
                uint4 v = make_uint4(0, 0, 0, 0);
                if (r < nj) {
                    const int t = order ? order[j * BLK + r] : j * BLK + r;
                    v = *reinterpret_cast<const uint4*>(src + (int64_t)t * D + ch * 8);
                }
                *reinterpret_cast<uint4*>(&ks_lds[r * KROW + ch * 8]) = v;
            }
            const uint16_t* vsrc = Vt + (bh * nb + j) * (int64_t)D * BLK;
            for (int p = tid; p < D * (BLK / 8); p += kThreads) {
                const int d = p / (BLK / 8), kc = p % (BLK / 8);
                *reinterpret_cast<uint4*>(&vs_lds[d * VROW + kc * 8]) =
                    *reinterpret_cast<const uint4*>(vsrc + (int64_t)d * BLK + kc * 8);
            }
            for (int d = tid; d < D; d += kThreads)
                vbar[d] = v_sum[(bh * nb + j) * (int64_t)D + d] / (float)nj;
        }
        __syncthreads();

        // L^T = K_j qbar^T (raw dot products; the scale is applied in exp2)
        f32x16 s[KT];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            s[kt] = f32x16{};
            const uint16_t* krow = &ks_lds[(kt * 32 + swap23(col)) * KROW + 8 * h];
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + st * 16));
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qhi[st], s[kt], 0, 0, 0);
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qlo[st], s[kt], 0, 0, 0);
            }
        }

        // keys past the end of the sequence take no part; max over the block
        float mx = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int g = r >> 2, e = r & 3;
                const int key = kt * 32 + 16 * (g >> 1) + 8 * h + 4 * (g & 1) + e;
                if (key >= nj) s[kt][r] = -__builtin_inff();
                mx = fmaxf(mx, s[kt][r]);
            }
        }
        mx = half_swap_max(mx);
        const float nbase = -c * mx;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                s[kt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][r], c, nbase));
        }

        // A^T = V_j^T W^T
        f32x16 acc[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                float w[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) w[t] = s[kt][8 * s2 + t];
                bf16x8 whi, wlo;
                split8(w, whi, wlo);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const bf16x8 a = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const uint4*>(
                                    &vs_lds[(dt * 32 + col) * VROW + kt * 32 + 16 * s2 + 8 * h]));
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, whi, acc[dt], 0, 0, 0);
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wlo, acc[dt], 0, 0, 0);
                }
            }
        }

        // || A - Ahat ||^2 over the channels, Ahat = n_j exp(S_ij - m) vbar_j
        const float sij = q_ok ? S[(bh * nb + q) * (int64_t)nb + j] : 0.f;
        const float zhat = (float)nj * __builtin_amdgcn_exp2f(sij * 1.44269504088896340736f + nbase);
        float e2 = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int d = dt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                const float diff = acc[dt][r] - zhat * vbar[d];
                e2 = __builtin_fmaf(diff, diff, e2);
            }
        }
        e2 = half_swap_sum(e2);
        if (h == 0 && q_ok)
            keys[(bh * nb + q) * (int64_t)nb + j] = 0.5f * logf(e2) + scale * mx - logf((float)nj);
    }
}

template <int D, int BLK>
sa_status launch_t(const Geometry& g, const float* qm, const uint16_t* K, const uint16_t* Vt,
                   const float* v_sum, const float* S, float* keys, hipStream_t stream) {
    const dim3 grid((unsigned)ceil_div(g.nb, kQPerGroup), (unsigned)ceil_div(g.nb, RJ),
                    (unsigned)g.BH());
    hipLaunchKernelGGL((k_err<D, BLK>), grid, dim3(kThreads), 0, stream, qm, K, Vt, v_sum, S, keys,
                       g.N, g.nb, g.scale, g.order);
    return hip_check(hipGetLastError(), "k_err launch");
}

}  // namespace

sa_status launch_route_keys(const Geometry& g, const float* qm, const uint16_t* K,
                            const uint16_t* Vt, const float* v_sum, const float* S, float* keys,
                            hipStream_t stream) {
    if (g.d == 128)
        return g.block == 128 ? launch_t<128, 128>(g, qm, K, Vt, v_sum, S, keys, stream)
                              : launch_t<128, 64>(g, qm, K, Vt, v_sum, S, keys, stream);
    return g.block == 128 ? launch_t<64, 128>(g, qm, K, Vt, v_sum, S, keys, stream)
                          : launch_t<64, 64>(g, qm, K, Vt, v_sum, S, keys, stream);
}

}  // namespace sa
