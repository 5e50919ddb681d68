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
// One work item: 8 waves x 32 query blocks against one KV block j of one
// (batch, head); K_j and V_j^T are staged in LDS once per item and shared by
// the eight waves (see k_err for the persistent, double-buffered schedule).
#include <math.h>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kQPerWave = 32;
constexpr int kQPerGroup = kWaves * kQPerWave;   // query blocks per work item

// Splits 8 finite fp32 values into bf16 hi and lo parts, both rounded to
// nearest even (the conversion instruction): x ~= hi + lo to 2^-16 relative.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        hi[e] = (__bf16)x[e];
        lo[e] = (__bf16)(x[e] - (float)hi[e]);
    }
}

// K row order inside a 32-row tile: bits 2 and 3 of the row index swapped.
__device__ __forceinline__ int swap23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Workgroup barrier after this wave's LDS writes have landed (global loads
// and stores in flight are not waited for: their results are used only by
// the wave that issued them, after the waits the compiler places).
__device__ __forceinline__ void wg_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
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
struct ErrCfg {
    static constexpr int KS = D / 16;            // channel steps of L^T
    static constexpr int KT = BLK / 32;          // 32-key tiles
    static constexpr int DT = D / 32;            // 32-channel tiles of A^T
    static constexpr int KROW = D + 8;           // LDS row pitch of K (bf16)
    static constexpr int VROW = BLK + 8;         // LDS row pitch of V^T (bf16)
    static constexpr int K_ELEMS = BLK * KROW;
    static constexpr int V_ELEMS = D * VROW;
    static constexpr int KCH = BLK * (D / 8);    // 16-byte chunks of a K tile
    static constexpr int VCH = D * (BLK / 8);    // and of a V^T tile
    static constexpr int PK = KCH / kThreads;    // chunks per thread and tile
    static constexpr int PV = VCH / kThreads;
    // one stage: K tile, V^T tile (bf16) and the centroid values (fp32)
    static constexpr int STAGE_BYTES = (K_ELEMS + V_ELEMS) * 2 + D * 4;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    static_assert(PK * kThreads == KCH && PV * kThreads == VCH, "whole chunks per thread");
    static_assert(STAGE_BYTES % 16 == 0, "16-byte aligned stages");
};

// Persistent grid over the work items (b*h, query group xg of 256 query
// blocks, KV block j), item = ((bh * nxg) + xg) * nb + j; workgroup w takes a
// contiguous range, so each K/V tile is staged once for all the query blocks
// of its head.  An item runs in four phases per wave: M1 (the score product,
// matrix cores), V1 (mask, max, exp2 weights, hi/lo split), M2 (the value
// product) and V2 (the error and the key).  The two groups of four waves run
// one phase apart ("ping-pong"): the second group starts one barrier late,
// so on every SIMD one wave's matrix phase overlaps the other wave's vector
// phase and a barrier closes every phase.  Group 0 loads the next item's K
// tile (and centroid values) during its M1 and stores it to the other LDS
// stage in its V1, group 1 does the same with the V^T tile one phase later;
// the other stage's last reader (group 1's M2 of the previous item) is past
// by then, and both stores land before the next item's M1.
template <int D, int BLK>
__global__ __launch_bounds__(kThreads, 1) void k_err(const float* __restrict__ qm,
                                                    const uint16_t* __restrict__ K,
                                                    const uint16_t* __restrict__ Vt,
                                                    const float* __restrict__ v_sum,
                                                    const float* __restrict__ S,
                                                    float* __restrict__ keys, int N, int nb,
                                                    float scale, const int32_t* __restrict__ order,
                                                    int64_t items, int nxg) {
    using C = ErrCfg<D, BLK>;
    constexpr int GT = kThreads / 2;                 // threads of one wave group
    constexpr int GK = C::KCH / GT;                  // K chunks per group-0 thread
    constexpr int GV = C::VCH / GT;                  // V^T chunks per group-1 thread
    static_assert(GK * GT == C::KCH && GV * GT == C::VCH, "whole chunks per thread");
    extern __shared__ __attribute__((aligned(16))) unsigned char err_lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, h = lane >> 5;
    const bool lagging = wave >= kWaves / 2;
    const int gt = tid & (GT - 1);                   // thread index inside the group
    const float c = scale * 1.44269504088896340736f;   // logits in log2 units
    const int64_t beg = items * blockIdx.x / gridDim.x;
    const int64_t end = items * (blockIdx.x + 1) / gridDim.x;

    auto k_tile = [&](int st) { return reinterpret_cast<uint16_t*>(err_lds + st * C::STAGE_BYTES); };
    auto v_tile = [&](int st) { return k_tile(st) + C::K_ELEMS; };
    auto vbar_of = [&](int st) {
        return reinterpret_cast<float*>(err_lds + st * C::STAGE_BYTES + (C::K_ELEMS + C::V_ELEMS) * 2);
    };
    // K chunk p of item `item`: key r of block j is token j*BLK + r of the
    // block order (through the token order when one is given); rows past the
    // sequence are zero
    auto k_chunk = [&](int64_t item, int p) __attribute__((always_inline)) -> u32x4 {
        const int j = (int)(item % nb);
        const int64_t bh = item / ((int64_t)nxg * nb);
        const int nj = min(BLK, N - j * BLK);
        const int r = p / (D / 8), ch = p % (D / 8);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < nj) {
            const int t = order ? clamp_token(order[j * BLK + r], N) : j * BLK + r;
            v = *reinterpret_cast<const u32x4*>(K + (bh * N + t) * (int64_t)D + ch * 8);
        }
        return v;
    };
    auto v_chunk = [&](int64_t item, int p) __attribute__((always_inline)) -> u32x4 {
        const int j = (int)(item % nb);
        const int64_t bh = item / ((int64_t)nxg * nb);
        const int d = p / (BLK / 8), kc = p % (BLK / 8);
        return *reinterpret_cast<const u32x4*>(Vt + ((bh * nb + j) * (int64_t)D + d) * BLK + kc * 8);
    };
    auto vbar_val = [&](int64_t item, int d) __attribute__((always_inline)) -> float {
        const int j = (int)(item % nb);
        const int64_t bh = item / ((int64_t)nxg * nb);
        const int nj = min(BLK, N - j * BLK);
        return v_sum[(bh * nb + j) * (int64_t)D + d] / (float)nj;
    };
    auto k_put = [&](int st, int p, u32x4 v) __attribute__((always_inline)) {
        const int r = p / (D / 8), ch = p % (D / 8);
        *reinterpret_cast<u32x4*>(&k_tile(st)[r * C::KROW + ch * 8]) = v;
    };
    auto v_put = [&](int st, int p, u32x4 v) __attribute__((always_inline)) {
        const int d = p / (BLK / 8), kc = p % (BLK / 8);
        *reinterpret_cast<u32x4*>(&v_tile(st)[d * C::VROW + kc * 8]) = v;
    };

    // the first item's tiles, by every thread
    if (beg < end) {
        for (int p = tid; p < C::KCH; p += kThreads) k_put(0, p, k_chunk(beg, p));
        for (int p = tid; p < C::VCH; p += kThreads) v_put(0, p, v_chunk(beg, p));
        if (tid < D) vbar_of(0)[tid] = vbar_val(beg, tid);
    }
    __syncthreads();

    // staging registers of this thread's share of the next item
    u32x4 sreg[GK > GV ? GK : GV];
    float vb = 0.f;

    bf16x8 qhi[C::KS], qlo[C::KS];
    int64_t cur_g = -1;
    f32x16 s[C::KT];
    bf16x8 whi[C::KT][2], wlo[C::KT][2];
    f32x16 acc[C::DT];
    float mx = 0.f, nbase = 0.f, sij = 0.f;

    if (lagging) wg_barrier();
    for (int64_t it = beg; it < end; ++it) {
        const int st = (int)((it - beg) & 1);
        const int j = (int)(it % nb);
        const int64_t g = it / nb;                       // bh * nxg + xg
        const int64_t bh = g / nxg;
        const int q = (int)(g % nxg) * kQPerGroup + wave * kQPerWave + col;
        const bool q_ok = q < nb;
        const bool more = it + 1 < end;
        const int nj = min(BLK, N - j * BLK);
        const uint16_t* ks_lds = k_tile(st);
        const uint16_t* vs_lds = v_tile(st);

        // ---- M1: L^T = K_j qbar^T (raw dot products; the scale is applied in exp2)
        wg_barrier();
        if (more) {
            // this group's share of the next item, into registers (the chunk
            // indices are formed here: hoisted, they would hold registers
            // across the whole loop)
            int g0 = gt;
            asm volatile("" : "+v"(g0));
            if (!lagging) {
#pragma unroll
                for (int n = 0; n < GK; ++n) sreg[n] = k_chunk(it + 1, g0 + n * GT);
                if (g0 < D) vb = vbar_val(it + 1, g0);
            } else {
#pragma unroll
                for (int n = 0; n < GV; ++n) sreg[n] = v_chunk(it + 1, g0 + n * GT);
            }
        }
        if (g != cur_g) {
            cur_g = g;
            const float* qrow = qm + (bh * nb + (q_ok ? q : 0)) * (int64_t)D;
#pragma unroll
            for (int s2 = 0; s2 < C::KS; ++s2) {
                float x[8];
                const float4 a = reinterpret_cast<const float4*>(qrow + s2 * 16 + 8 * h)[0];
                const float4 b = reinterpret_cast<const float4*>(qrow + s2 * 16 + 8 * h)[1];
                x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
                x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
                if (!q_ok) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = 0.f;
                }
                split8(x, qhi[s2], qlo[s2]);
            }
        }
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt) {
            s[kt] = f32x16{};
            const uint16_t* krow = &ks_lds[(kt * 32 + swap23(col)) * C::KROW + 8 * h];
#pragma unroll
            for (int st2 = 0; st2 < C::KS; ++st2) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(krow + st2 * 16));
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qhi[st2], s[kt], 0, 0, 0);
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qlo[st2], s[kt], 0, 0, 0);
            }
        }

        // ---- V1: the next item's share to the other stage; mask, max, weights
        wg_barrier();
        if (more) {
            int g0 = gt;
            asm volatile("" : "+v"(g0));
            if (!lagging) {
#pragma unroll
                for (int n = 0; n < GK; ++n) k_put(st ^ 1, g0 + n * GT, sreg[n]);
                if (g0 < D) vbar_of(st ^ 1)[g0] = vb;
            } else {
#pragma unroll
                for (int n = 0; n < GV; ++n) v_put(st ^ 1, g0 + n * GT, sreg[n]);
            }
        }
        sij = q_ok ? S[(bh * nb + q) * (int64_t)nb + j] : 0.f;
        // keys past the end of the sequence take no part (a short last
        // block only)
        if (nj < BLK) {
#pragma unroll
            for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gg = r >> 2, e = r & 3;
                    const int key = kt * 32 + 16 * (gg >> 1) + 8 * h + 4 * (gg & 1) + e;
                    if (key >= nj) s[kt][r] = -__builtin_inff();
                }
            }
        }
        mx = -__builtin_inff();
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
        }
        mx = half_swap_max(mx);
        nbase = -c * mx;
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                float w[8];
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    w[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][8 * s2 + t], c, nbase));
                split8(w, whi[kt][s2], wlo[kt][s2]);
            }
        }

        // ---- M2: A^T = V_j^T W^T
        wg_barrier();
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) acc[dt] = f32x16{};
#pragma unroll
        for (int kt = 0; kt < C::KT; ++kt) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
                for (int dt = 0; dt < C::DT; ++dt) {
                    const bf16x8 a = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const uint4*>(
                                    &vs_lds[(dt * 32 + col) * C::VROW + kt * 32 + 16 * s2 + 8 * h]));
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, whi[kt][s2], acc[dt], 0, 0, 0);
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, wlo[kt][s2], acc[dt], 0, 0, 0);
                }
            }
        }

        // ---- V2: || A - Ahat ||^2 over the channels, Ahat = n_j exp(S_ij - m) vbar_j
        wg_barrier();
        const float* vbar = vbar_of(st);
        const float zhat = (float)nj * __builtin_amdgcn_exp2f(sij * 1.44269504088896340736f + nbase);
        float e2 = 0.f;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) {
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
    if (!lagging) wg_barrier();
}

template <int D, int BLK>
sa_status launch_t(const Geometry& g, const float* qm, const uint16_t* K, const uint16_t* Vt,
                   const float* v_sum, const float* S, float* keys, hipStream_t stream) {
    using C = ErrCfg<D, BLK>;
    const void* fn = (const void*)k_err<D, BLK>;
    sa_status st = ensure_max_lds(fn, C::LDS_BYTES, "k_err");
    if (st != SA_OK) return st;
    int resident = 0;
    if ((st = resident_workgroups(fn, kThreads, C::LDS_BYTES, &resident)) != SA_OK) return st;
    const int nxg = (int)ceil_div(g.nb, kQPerGroup);
    const int64_t items = g.BH() * nxg * (int64_t)g.nb;
    const int64_t grid = items < resident ? items : resident;
    if (grid <= 0) return SA_OK;
    hipLaunchKernelGGL((k_err<D, BLK>), dim3((unsigned)grid), dim3(kThreads), C::LDS_BYTES, stream, qm,
                       K, Vt, v_sum, S, keys, g.N, g.nb, g.scale, g.order, items, nxg);
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
