// Block-sparse attention forward for gfx950 (SVG-EAR page, section 2B:
// streaming softmax update over the computed blocks without materialising the
// logits; SPADE page, part 3: a head-wise sparse attention kernel).  With
// compensation, every skipped KV block contributes one centroid pseudo-token
// (SVG-EAR page, section 2A): key = block mean of K, value = block mean of V,
// weight = the block's token count (a logit bias of log n_j).
//
// Mapping onto CDNA4
//   * one workgroup = one (batch, head, query block); wave w owns 32 queries.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: the B operand (Q^T) stays in
//     registers for the whole row, the A operand (K) is read from LDS.  In the
//     32x32 accumulator layout a lane holds one query column, so the softmax
//     statistics of a query are lane-local; the two lane halves that share a
//     query exchange their maximum once per tile (xor 32).
//   * O^T = V^T P^T on the same instruction: P goes from the S^T accumulators
//     straight into the B operand.  K rows are loaded in an order that swaps
//     bits 2 and 3 of the row index inside every 16 rows, which makes the 8
//     probabilities a lane holds per k-step 8 consecutive keys; V is stored
//     transposed in LDS so those 8 keys are one 16-byte LDS read.
//   * online softmax in the log2 domain (scale*log2(e) folded into one FMA).
//   * blockIdx -> row remap keeps consecutive query blocks of a head on one
//     XCD (workgroups are dealt round-robin to the 8 XCDs), so the K/V blocks
//     they share are served from that XCD's L2.
#include <math.h>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Row order of K inside a 32-row tile: bits 2 and 3 of the row index swapped.
__device__ __forceinline__ int swap23(int r) {
    return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

struct FwdArgs {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    const int32_t* row_ptr;
    const int32_t* col_idx;
    const uint16_t* kbar;    // [BH][nb][D] bf16 centroid keys (compensation) or null
    const uint16_t* vbar;    // [BH][nb][D] bf16 centroid values
    uint16_t* O;
    float* lse;
    int32_t N, nb;
    int64_t rows;
    float c;                 // scale * log2(e)
};

template <int D, int BLK>
struct Lds {
    static constexpr int KST = D + 8;        // bf16 per K row (+16 B: bank shift)
    static constexpr int VST = BLK + 8;      // bf16 per V^T row
    static constexpr int K_BYTES = BLK * KST * 2;
    static constexpr int V_BYTES = D * VST * 2;
    static constexpr int BIAS_BYTES = BLK * 4;
    static constexpr int BASE = K_BYTES + V_BYTES + BIAS_BYTES;
};

// Stage BLK key rows and the matching value rows (transposed) into LDS.
// Rows r >= nvalid are zero.  src_row(r) gives the global row of tile row r.
template <int D, int BLK, int NT, typename RowFn>
__device__ __forceinline__ void stage_tile(const uint16_t* __restrict__ Kg,
                                           const uint16_t* __restrict__ Vg, int nvalid,
                                           RowFn src_row, uint16_t* Ks, uint16_t* Vt) {
    using L = Lds<D, BLK>;
    constexpr int CH = D / 8;
    const int tid = threadIdx.x;
    // K: row-major, 16-byte chunks
#pragma unroll
    for (int c = tid; c < BLK * CH; c += NT) {
        const int r = c / CH, ch = c % CH;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < nvalid) v = *reinterpret_cast<const uint4*>(Kg + src_row(r) * D + ch * 8);
        *reinterpret_cast<uint4*>(Ks + r * L::KST + ch * 8) = v;
    }
    // V: 8 keys x 8 channels per thread, transposed in registers
#pragma unroll
    for (int g = tid; g < (BLK / 8) * CH; g += NT) {
        const int dg = g % CH, kg = g / CH;
        uint32_t w[8][4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint4 v = make_uint4(0, 0, 0, 0);
            const int r = kg * 8 + e;
            if (r < nvalid) v = *reinterpret_cast<const uint4*>(Vg + src_row(r) * D + dg * 8);
            w[e][0] = v.x; w[e][1] = v.y; w[e][2] = v.z; w[e][3] = v.w;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            uint32_t o[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const uint32_t x = w[2 * p][c >> 1], y = w[2 * p + 1][c >> 1];
                o[p] = (c & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
            }
            *reinterpret_cast<uint4*>(Vt + (dg * 8 + c) * L::VST + kg * 8) =
                make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

// One KV tile of the online softmax for the 32 queries of this wave.
template <int D, int BLK>
__device__ __forceinline__ void attend_tile(const uint16_t* Ks, const uint16_t* Vt,
                                            const float* bias, bool use_bias,
                                            const bf16x8 (&qf)[D / 16], f32x16 (&oacc)[D / 32],
                                            float& m_run, float& l_run, float c) {
    using L = Lds<D, BLK>;
    constexpr int KT = BLK / 32;
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, h = lane >> 5;
    const int krow = swap23(r32);

    f32x16 s[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
        f32x16 acc = {};
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            const bf16x8 a = as_bf16x8(
                *reinterpret_cast<const uint4*>(Ks + (kt * 32 + krow) * L::KST + st * 16 + h * 8));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], acc, 0, 0, 0);
        }
        s[kt] = acc;
    }

    // logits in the log2 domain and the tile maximum of this query
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float t = s[kt][i] * c;
            if (use_bias) t += bias[kt * 32 + swap23(8 * (i >> 2) + 4 * h + (i & 3))];
            s[kt][i] = t;
            mx = fmaxf(mx, t);
        }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float base = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - base);
    float sum = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(s[kt][i] - base);
            s[kt][i] = p;
            sum += p;
        }
    l_run = l_run * alpha + sum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = (__bf16)s[kt][8 * s2 + e];
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(
                    Vt + (dt * 32 + r32) * L::VST + kt * 32 + 16 * s2 + 8 * h));
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[dt], 0, 0, 0);
            }
        }
}

template <int D, int BLK, bool COMP>
__global__ __launch_bounds__(BLK * 2) void k_bsattn_fwd(FwdArgs a) {
    using L = Lds<D, BLK>;
    constexpr int NT = BLK * 2;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
    uint16_t* Vt = reinterpret_cast<uint16_t*>(smem + L::K_BYTES);
    float* bias = reinterpret_cast<float*>(smem + L::K_BYTES + L::V_BYTES);
    int16_t* skip = reinterpret_cast<int16_t*>(smem + L::BASE);   // COMP: [nb]
    unsigned char* kept = smem + L::BASE + 2 * (size_t)a.nb;        // COMP: [nb]
    __shared__ int s_nskip;

    // XCD-aware remap: the workgroups dealt to one XCD take consecutive rows
    const int64_t G = a.rows;
    const int64_t w = blockIdx.x;
    const int64_t q8 = G / 8, rem = G % 8, x = w % 8;
    const int64_t row = x * q8 + (x < rem ? x : rem) + w / 8;

    const int i = (int)(row % a.nb);
    const int64_t bh = row / a.nb;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r32 = lane & 31, h = lane >> 5;
    const int64_t head_off = bh * (int64_t)a.N * D;
    const uint16_t* Kh = a.K + head_off;
    const uint16_t* Vh = a.V + head_off;

    // this lane's query and its Q^T fragments (B operand)
    const int q_local = wave * 32 + r32;
    const int qn = i * BLK + q_local;
    bf16x8 qf[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (qn < a.N) v = *reinterpret_cast<const uint4*>(a.Q + head_off + (int64_t)qn * D + st * 16 + h * 8);
        qf[st] = as_bf16x8(v);
    }

    f32x16 oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    const int beg = a.row_ptr[row], end = a.row_ptr[row + 1];
    const int last_n = a.N - (a.nb - 1) * BLK;
    for (int e = beg; e < end; ++e) {
        const int j = a.col_idx[e];
        if ((unsigned)j >= (unsigned)a.nb) continue;
        const int nvalid = j == a.nb - 1 ? last_n : BLK;
        __syncthreads();
        stage_tile<D, BLK, NT>(Kh, Vh, nvalid, [&](int r) { return (int64_t)j * BLK + r; }, Ks, Vt);
        const bool partial = nvalid < BLK;
        if (partial)
            for (int r = tid; r < BLK; r += NT) bias[r] = r < nvalid ? 0.f : -INFINITY;
        __syncthreads();
        attend_tile<D, BLK>(Ks, Vt, bias, partial, qf, oacc, m_run, l_run, a.c);
    }

    if constexpr (COMP) {
        // complement of the kept list, ascending (one wave, ballot compaction)
        __syncthreads();
        for (int j = tid; j < a.nb; j += NT) kept[j] = 0;
        __syncthreads();
        for (int e = beg + tid; e < end; e += NT) {
            const int j = a.col_idx[e];
            if ((unsigned)j < (unsigned)a.nb) kept[j] = 1;
        }
        __syncthreads();
        if (wave == 0) {
            int cnt = 0;
            for (int j0 = 0; j0 < a.nb; j0 += 64) {
                const int j = j0 + lane;
                const bool sk = j < a.nb && !kept[j];
                const unsigned long long m = __ballot(sk);
                const int pos = __popcll(m & ((1ull << lane) - 1ull));
                if (sk) skip[cnt + pos] = (int16_t)j;
                cnt += __popcll(m);
            }
            if (lane == 0) s_nskip = cnt;
        }
        __syncthreads();
        const int nskip = s_nskip;
        const uint16_t* kb = a.kbar + bh * (int64_t)a.nb * D;
        const uint16_t* vb = a.vbar + bh * (int64_t)a.nb * D;
        for (int t0 = 0; t0 < nskip; t0 += BLK) {
            const int nvalid = min(BLK, nskip - t0);
            __syncthreads();
            stage_tile<D, BLK, NT>(kb, vb, nvalid, [&](int r) { return (int64_t)skip[t0 + r]; },
                                   Ks, Vt);
            for (int r = tid; r < BLK; r += NT) {
                float b = -INFINITY;
                if (r < nvalid) {
                    const int j = skip[t0 + r];
                    b = __log2f((float)(j == a.nb - 1 ? last_n : BLK));
                }
                bias[r] = b;
            }
            __syncthreads();
            attend_tile<D, BLK>(Ks, Vt, bias, true, qf, oacc, m_run, l_run, a.c);
        }
    }

    // epilogue: O = O^T / l, lse = (m + log2 l) * ln 2
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qn < a.N) {
        uint16_t* orow = a.O + head_off + (int64_t)qn * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = dt * 32 + 8 * g + 4 * h;
                const uint32_t lo = f32_to_bf16_rne(oacc[dt][4 * g + 0] * inv) |
                                    ((uint32_t)f32_to_bf16_rne(oacc[dt][4 * g + 1] * inv) << 16);
                const uint32_t hi = f32_to_bf16_rne(oacc[dt][4 * g + 2] * inv) |
                                    ((uint32_t)f32_to_bf16_rne(oacc[dt][4 * g + 3] * inv) << 16);
                *reinterpret_cast<uint2*>(orow + d0) = make_uint2(lo, hi);
            }
        if (a.lse && h == 0)
            a.lse[bh * (int64_t)a.N + qn] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

// Centroid pseudo-tokens for compensation, rounded to bf16 for the matrix cores:
// kbar = k_mean, vbar = v_sum / n_j.
__global__ void k_comp_prep(const float* __restrict__ k_mean, const float* __restrict__ v_sum,
                            uint16_t* __restrict__ kbar, uint16_t* __restrict__ vbar,
                            int64_t total, int D, int nb, int block, int last_n) {
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * blockDim.x) {
        const int j = (int)((e / D) % nb);
        const float n = (float)(j == nb - 1 ? last_n : block);
        kbar[e] = f32_to_bf16_rne(k_mean[e]);
        vbar[e] = f32_to_bf16_rne(v_sum[e] / n);
    }
}

template <int D, int BLK, bool COMP>
sa_status launch_t(const FwdArgs& a, int nb, hipStream_t stream) {
    using L = Lds<D, BLK>;
    const size_t lds = L::BASE + (COMP ? (size_t)nb * 3 + 16 : 0);
    static bool configured = false;
    if (!configured) {
        const int most = L::BASE + (COMP ? 4096 * 3 + 16 : 0);
        sa_status st = hip_check(hipFuncSetAttribute((const void*)k_bsattn_fwd<D, BLK, COMP>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     most),
                                 "k_bsattn_fwd shared memory");
        if (st != SA_OK) return st;
        configured = true;
    }
    hipLaunchKernelGGL((k_bsattn_fwd<D, BLK, COMP>), dim3((unsigned)a.rows), dim3(BLK * 2), lds,
                       stream, a);
    return hip_check(hipGetLastError(), "k_bsattn_fwd launch");
}

}  // namespace

size_t fwd_workspace_bytes(const Geometry& g) {
    return align_up((size_t)g.BH() * g.nb * g.d * 2, 256) * 2;
}

sa_status launch_fwd(const Geometry& g, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                     const int32_t* row_ptr, const int32_t* col_idx, const float* k_mean,
                     const float* v_sum, uint16_t* O, float* lse, char* ws, hipStream_t stream) {
    const bool comp = k_mean != nullptr;
    if (comp && g.nb > 4096)
        return fail(SA_ERR_UNSUPPORTED, "compensation supports nb <= 4096 (got %d)", g.nb);
    FwdArgs a{};
    a.Q = Q; a.K = K; a.V = V; a.row_ptr = row_ptr; a.col_idx = col_idx;
    a.O = O; a.lse = lse; a.N = g.N; a.nb = g.nb; a.rows = g.rows();
    a.c = g.scale * kLog2e;
    if (comp) {
        const size_t half = align_up((size_t)g.BH() * g.nb * g.d * 2, 256);
        uint16_t* kbar = reinterpret_cast<uint16_t*>(ws);
        uint16_t* vbar = reinterpret_cast<uint16_t*>(ws + half);
        const int64_t total = g.BH() * g.nb * g.d;
        const int64_t blocks = ceil_div(total, 256);
        hipLaunchKernelGGL(k_comp_prep, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256), 0,
                           stream, k_mean, v_sum, kbar, vbar, total, g.d, g.nb, g.block,
                           g.N - (g.nb - 1) * g.block);
        sa_status st = hip_check(hipGetLastError(), "k_comp_prep launch");
        if (st != SA_OK) return st;
        a.kbar = kbar; a.vbar = vbar;
    }
    if (g.d == 128) {
        if (g.block == 128)
            return comp ? launch_t<128, 128, true>(a, g.nb, stream) : launch_t<128, 128, false>(a, g.nb, stream);
        return comp ? launch_t<128, 64, true>(a, g.nb, stream) : launch_t<128, 64, false>(a, g.nb, stream);
    }
    if (g.block == 128)
        return comp ? launch_t<64, 128, true>(a, g.nb, stream) : launch_t<64, 128, false>(a, g.nb, stream);
    return comp ? launch_t<64, 64, true>(a, g.nb, stream) : launch_t<64, 64, false>(a, g.nb, stream);
}

}  // namespace sa
