// Block selection kernels for gfx950 (wave64).
//
//   k_pool    block / sub-block means of Q and K, block means of K and block
//             sums of V (DFSAttn page, trick 2: a block is summarised by its
//             mean; SVG-EAR page, section 2A: the centroid of a skipped block).
//             HBM-bound: one pass over the tensors with 16-byte loads staged
//             through LDS; sums are exact in fp64, so any reduction order gives
//             the same fp32 result.
//   k_score   pooled scores S[i,j] = fl32(scale * dot(qbar_i, kbar_j)), the dot
//             a sequential fp32 FMA chain over the channels (one lane per block
//             pair, so the chain order is fixed); with sub-blocks the score is
//             the max over the sub-block pairs (DFSAttn page, trick 2).
//   k_select  one workgroup per query block: LDS bitonic sort by (score desc,
//             index asc), top-k or cumulative-mass cut (SVG-EAR page, sections
//             2B and 4; SVOO page, section 2A), union with the diagonal, the
//             temporal window and the rotating anchors (LVSA abstract); writes
//             a kept-block bitmap and count.  k_select_w takes the same
//             decision with one wave per query block (rows of up to 2048
//             blocks): radix select for top-k, a register sort for the mass
//             rule.
//   k_scan    exclusive scan of the counts -> CSR row pointers.
//   k_expand  bitmap -> ascending column indices.
#include <math.h>

#include "sa_internal.h"

namespace sa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float((uint32_t)b << 16);
}

// ----------------------------------------------------------------------------
// k_pool
// ----------------------------------------------------------------------------
// role 0: Q -> unit means qm            (unit = sub_block or block)
// role 1: K -> unit means km, and block means k_mean when k_mean != nullptr
// role 2: V -> block sums v_sum
struct PoolArgs {
    const uint16_t* src[3];
    const int32_t* order;    // token order of the blocks ([N]), or null: as given
    float* unit_out[3];      // [BH][n_units][D] or nullptr
    float* block_out[3];     // [BH][nb][D] or nullptr
    int32_t roles[3];
    int32_t N, nb, unit, n_units;
};

// One workgroup per (block, b*h, role).  Thread (s, ch) sums rows
// [s*SEGR, (s+1)*SEGR) of channels [8 ch, 8 ch + 8) straight from HBM (SEGR
// 16-byte loads in flight per thread, no LDS staging); the 16 segment sums
// then combine into unit and block sums.  Sums of bf16 values are exact in
// fp64, so the grouping does not change the result.
template <int D, int BLK>
__global__ __launch_bounds__(kThreads) void k_pool(PoolArgs a) {
    constexpr int CH = D / 8;             // 16-byte chunks per row
    constexpr int NS = kThreads / CH;     // row segments (16 for d = 128, 32 for d = 64)
    constexpr int SEGR = BLK / NS;        // rows per segment
    static_assert(SEGR >= 1 && NS * SEGR == BLK, "segments tile the block");
    __shared__ double seg[NS][D];

    const int blk = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int role = a.roles[blockIdx.z];
    const int tid = threadIdx.x;
    const int row0 = blk * BLK;
    const int n = min(BLK, a.N - row0);
    const int sgi = tid / CH, ch = tid % CH;
    const uint4* src = reinterpret_cast<const uint4*>(a.src[role] + bh * a.N * D) + ch;

    // the block's rows: tokens row0 .. row0+n-1 of the block order (read
    // through the token order when one is given; all indices first, so the
    // row loads stay in flight together)
    int tok[SEGR];
#pragma unroll
    for (int r = 0; r < SEGR; ++r) {
        const int row = sgi * SEGR + r;
        tok[r] = row < n ? (a.order ? clamp_token(a.order[row0 + row], a.N) : row0 + row) : -1;
    }
    uint4 v[SEGR];
#pragma unroll
    for (int r = 0; r < SEGR; ++r)
        v[r] = tok[r] >= 0 ? src[(int64_t)tok[r] * CH] : make_uint4(0, 0, 0, 0);
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < SEGR; ++r) {
        const uint32_t w[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += (double)__uint_as_float(w[e] << 16);
            acc[2 * e + 1] += (double)__uint_as_float(w[e] & 0xffff0000u);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) seg[sgi][ch * 8 + e] = acc[e];
    __syncthreads();

    const int nseg = (n + SEGR - 1) / SEGR;
    float* uo = a.unit_out[role];
    if (uo) {
        const int spb = BLK / a.unit;
        const int segs_per_unit = a.unit / SEGR;
        const int nunit = (n + a.unit - 1) / a.unit;
        for (int p = tid; p < nunit * D; p += kThreads) {
            const int u = p / D, c = p % D;
            double t = 0.0;
            for (int s2 = u * segs_per_unit; s2 < min(nseg, (u + 1) * segs_per_unit); ++s2)
                t += seg[s2][c];
            const int cnt = min(a.unit, n - u * a.unit);
            uo[((int64_t)bh * a.n_units + (int64_t)blk * spb + u) * D + c] =
                (float)(t / (double)cnt);
        }
    }
    float* bo = a.block_out[role];
    if (bo) {
        for (int c = tid; c < D; c += kThreads) {
            double t = 0.0;
            for (int s2 = 0; s2 < nseg; ++s2) t += seg[s2][c];
            const float val = role == 2 ? (float)t : (float)(t / (double)n);
            bo[((int64_t)bh * a.nb + blk) * D + c] = val;
        }
    }
}

// ----------------------------------------------------------------------------
// k_score
// ----------------------------------------------------------------------------
constexpr int kTile = 16;   // 16 x 16 threads per workgroup
constexpr int kScoreChunk = 32;   // channels of the unit means staged in LDS at a time

// Thread (ti, tj) of a workgroup takes the MT x MT block pairs (ti + 16 a,
// tj + 16 b) of its 16 MT x 16 MT tile; the unit means of the tile's query
// and key blocks are staged in LDS 32 channels at a time (rows padded by 4
// floats, so the 16 key rows a wave reads at once fall in distinct banks;
// ~17 KB per workgroup, so that several share a CU).  Each pair's dot
// product stays one sequential fp32 FMA chain over the channels, continued
// from chunk to chunk; the channel loop is unrolled so that the operand reads
// of the next step are issued under the FMAs of the current one.
template <int D, int SPB, int MT>
__global__ __launch_bounds__(kThreads) void k_score(const float* __restrict__ qm,
                                                    const float* __restrict__ km,
                                                    float* __restrict__ S, int nb,
                                                    int n_units, float scale) {
    constexpr int DC = kScoreChunk;       // channels staged at a time
    constexpr int ROW = SPB * DC + 4;     // floats per block row in LDS (+4: bank shift)
    constexpr int TB = kTile * MT;        // blocks per tile side
    extern __shared__ float lds[];
    float* qs = lds;                      // [TB][ROW]
    float* ks = lds + TB * ROW;           // [TB][ROW]

    const int64_t bh = blockIdx.z;
    const int i0 = blockIdx.y * TB, j0 = blockIdx.x * TB;
    const int tid = threadIdx.x;
    const float* qb = qm + bh * (int64_t)n_units * D;
    const float* kb = km + bh * (int64_t)n_units * D;

    const int ti = tid / kTile, tj = tid % kTile;
    float acc[MT][MT][SPB][SPB];
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < MT; ++b)
#pragma unroll
            for (int x = 0; x < SPB; ++x)
#pragma unroll
                for (int y = 0; y < SPB; ++y) acc[a][b][x][y] = 0.f;
    // channels DC at a time: stage the chunk of the unit means of TB query
    // and TB key blocks (float4), then continue every chain over it
    constexpr int V4 = SPB * DC / 4;
    for (int ch = 0; ch < D; ch += DC) {
        if (ch > 0) __syncthreads();                        // the last chunk is consumed
        for (int p = tid; p < TB * V4; p += kThreads) {
            const int b = p / V4, o = p % V4;
            const int u = o / (DC / 4), w = o % (DC / 4);   // unit within the block, float4 in the chunk
            float4 qv = make_float4(0.f, 0.f, 0.f, 0.f), kv = qv;
            if (i0 + b < nb && (i0 + b) * SPB + u < n_units)
                qv = *reinterpret_cast<const float4*>(qb + ((int64_t)(i0 + b) * SPB + u) * D + ch + 4 * w);
            if (j0 + b < nb && (j0 + b) * SPB + u < n_units)
                kv = *reinterpret_cast<const float4*>(kb + ((int64_t)(j0 + b) * SPB + u) * D + ch + 4 * w);
            *reinterpret_cast<float4*>(qs + b * ROW + o * 4) = qv;
            *reinterpret_cast<float4*>(ks + b * ROW + o * 4) = kv;
        }
        __syncthreads();
        // with many pairs per thread a full unroll would hoist every operand read
        constexpr int UNR = MT == 1 ? DC / 4 : 4;
#pragma unroll(UNR)
        for (int c = 0; c < DC; c += 4) {
            float4 qv[MT][SPB], kv[MT][SPB];
#pragma unroll
            for (int a = 0; a < MT; ++a)
#pragma unroll
                for (int x = 0; x < SPB; ++x) {
                    qv[a][x] = *reinterpret_cast<const float4*>(qs + (ti + kTile * a) * ROW + x * DC + c);
                    kv[a][x] = *reinterpret_cast<const float4*>(ks + (tj + kTile * a) * ROW + x * DC + c);
                }
#pragma unroll
            for (int a = 0; a < MT; ++a)
#pragma unroll
                for (int b = 0; b < MT; ++b)
#pragma unroll
                    for (int x = 0; x < SPB; ++x)
#pragma unroll
                        for (int y = 0; y < SPB; ++y) {
                            float s = acc[a][b][x][y];
                            s = __builtin_fmaf(qv[a][x].x, kv[b][y].x, s);
                            s = __builtin_fmaf(qv[a][x].y, kv[b][y].y, s);
                            s = __builtin_fmaf(qv[a][x].z, kv[b][y].z, s);
                            s = __builtin_fmaf(qv[a][x].w, kv[b][y].w, s);
                            acc[a][b][x][y] = s;
                        }
        }
    }
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
        for (int b = 0; b < MT; ++b) {
            const int i = i0 + ti + kTile * a, j = j0 + tj + kTile * b;
            if (i >= nb || j >= nb) continue;
            const int nu_i = min(SPB, n_units - i * SPB);       // units that exist
            const int nu_j = min(SPB, n_units - j * SPB);
            float best = -INFINITY;
#pragma unroll
            for (int x = 0; x < SPB; ++x)
#pragma unroll
                for (int y = 0; y < SPB; ++y)
                    if (x < nu_i && y < nu_j) best = fmaxf(best, scale * acc[a][b][x][y]);
            S[(bh * nb + i) * (int64_t)nb + j] = best;
        }
}

// ----------------------------------------------------------------------------
// k_select
// ----------------------------------------------------------------------------
constexpr int kInlineHeads = 64;

struct SelectArgs {
    const float* S;           // [rows][nb] scores (scored rules)
    const int32_t* k_head;    // [H] blocks kept per head (TOPK), when H > kInlineHeads
    int32_t k_inline[kInlineHeads];   // blocks kept per head, when H <= kInlineHeads
    uint32_t* bits;           // [rows][words]
    int32_t* counts;          // [rows]
    int32_t H, N, nb, nb_pad, words, block, HgW;
    int32_t rule;
    float mass;
    int32_t diag, window_frames, n_anchors;
    int64_t anchor_offset;
    int64_t rows;
};

// Monotone map of fp32 to uint32 (ascending), with -0 and +0 equal.
__device__ __forceinline__ uint32_t ordered_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0) u = 0;                     // -0 -> +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kThreads) void k_select(SelectArgs a) {
    extern __shared__ unsigned char smem[];
    const int nb = a.nb, P = a.nb_pad;
    unsigned long long* key = reinterpret_cast<unsigned long long*>(smem);  // [P]
    double* cum = reinterpret_cast<double*>(smem);                         // aliases key
    int32_t* ord = reinterpret_cast<int32_t*>(smem + (size_t)P * 8);       // [P]
    unsigned char* keep = smem + (a.rule != SA_RULE_NONE ? (size_t)P * 12 : 0);  // [words*32]
    __shared__ int32_t s_cut;
    __shared__ int32_t s_count;

    const int64_t row = blockIdx.x;
    const int i = (int)(row % nb);
    const int h = (int)((row / nb) % a.H);
    const int tid = threadIdx.x;

    for (int j = tid; j < a.words * 32; j += kThreads) keep[j] = 0;
    if (tid == 0) { s_cut = nb; s_count = 0; }

    if (a.rule != SA_RULE_NONE) {
        const float* S = a.S + row * (int64_t)nb;
        // sort keys: (score descending, index ascending) as one ascending uint64
        for (int j = tid; j < P; j += kThreads) {
            key[j] = j < nb ? ((unsigned long long)(~ordered_bits(S[j])) << 32) | (uint32_t)j
                            : ~0ull;
        }
        __syncthreads();
        for (int size = 2; size <= P; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int t = tid; t < P / 2; t += kThreads) {
                    const int lo = 2 * t - (t & (stride - 1));
                    const int hi = lo + stride;
                    const bool up = (lo & size) == 0;
                    const unsigned long long x = key[lo], y = key[hi];
                    if ((x > y) == up) { key[lo] = y; key[hi] = x; }
                }
                __syncthreads();
            }
        }
        for (int r = tid; r < nb; r += kThreads) ord[r] = (int32_t)(key[r] & 0xffffffffu);
        __syncthreads();

        int m;
        if (a.rule == SA_RULE_TOPK) {
            m = a.H <= kInlineHeads ? a.k_inline[h] : a.k_head[h];
        } else {
            // p_r = exp(S_r - S_max) in fp64, summed sequentially in rank order
            const double smax = (double)S[ord[0]];
            for (int r = tid; r < nb; r += kThreads) cum[r] = exp((double)S[ord[r]] - smax);
            __syncthreads();
            if (tid == 0) {
                // the same sequential sum, 32 values at a time through registers
                // so that the LDS loads are not serialised behind the adds
                constexpr int CK = 32;
                double run = 0.0;
                int r = 0;
                for (; r + CK <= nb; r += CK) {
                    double v[CK];
#pragma unroll
                    for (int k = 0; k < CK; ++k) v[k] = cum[r + k];
#pragma unroll
                    for (int k = 0; k < CK; ++k) { run += v[k]; v[k] = run; }
#pragma unroll
                    for (int k = 0; k < CK; ++k) cum[r + k] = v[k];
                }
                for (; r < nb; ++r) { run += cum[r]; cum[r] = run; }
            }
            __syncthreads();
            const double thr = (double)a.mass * cum[nb - 1];
            for (int r = tid; r < nb; r += kThreads)
                if (cum[r] >= thr) atomicMin(&s_cut, r + 1);
            __syncthreads();
            m = s_cut;
        }
        for (int r = tid; r < m; r += kThreads) keep[ord[r]] = 1;
    }
    __syncthreads();

    if (a.diag && tid == 0) keep[i] = 1;
    if (a.window_frames >= 0) {
        const int r = a.window_frames;
        const int lo_i = (i * a.block) / a.HgW;
        const int hi_i = (min(a.N, (i + 1) * a.block) - 1) / a.HgW;
        for (int j = tid; j < nb; j += kThreads) {
            const int lo_j = (j * a.block) / a.HgW;
            const int hi_j = (min(a.N, (j + 1) * a.block) - 1) / a.HgW;
            if (lo_j <= hi_i + r && hi_j >= lo_i - r) keep[j] = 1;
        }
    }
    if (a.n_anchors > 0) {
        const int64_t step = nb / a.n_anchors;
        for (int m = tid; m < a.n_anchors; m += kThreads)
            keep[(int)((a.anchor_offset + m * step) % nb)] = 1;
    }
    __syncthreads();

    uint32_t* out = a.bits + row * (int64_t)a.words;
    int local = 0;
    for (int w = tid; w < a.words; w += kThreads) {
        uint32_t word = 0;
        for (int b = 0; b < 32; ++b) word |= (uint32_t)keep[w * 32 + b] << b;
        out[w] = word;
        local += __popc(word);
    }
    if (local) atomicAdd(&s_count, local);
    __syncthreads();
    if (tid == 0) a.counts[row] = s_count;
}

// ----------------------------------------------------------------------------
// k_select_w: the same decision, one wave per query block (nb <= 2048)
// ----------------------------------------------------------------------------
// The row's sort keys (score descending, index ascending, as one ascending
// uint64) sit in registers, E per lane: element e is lane e / E, register
// e % E.  Top-k needs only the set of the k smallest keys: a radix select over
// the key's bytes (LDS histogram per wave), stopping once the k-th key's
// bucket holds exactly the keys still wanted.  The mass rule needs the rank
// order: a bitonic sort over the registers (lane shuffles for strides of E or
// more), then p_r = exp(S_r - S_max) in fp64 per element and the cumulative
// sum taken strictly in rank order by one scalar chain (total first, then the
// cut), exactly as the workgroup kernel does.  No workgroup barriers.
constexpr int kSelWaves = kThreads / 64;   // rows per workgroup
constexpr int kSelMaxWords = 64;           // bitmap words per row

__device__ __forceinline__ float ordered_to_float(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// x of lane ^ M: DPP quad permutes for M = 1, 2 (no LDS round trip), the
// LDS crossbar's swizzle (bit-mask mode) for M = 4 .. 16, the half-wave swap
// for M = 32
template <int M>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x) {
    if constexpr (M == 1)
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);   // [1,0,3,2]
    else if constexpr (M == 2)
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);   // [2,3,0,1]
    else if constexpr (M < 32)
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, (M << 10) | 0x1F);
    else {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return r[0] == x ? r[1] : r[0];
    }
}

template <int M>
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t v) {
    const uint32_t lo = xor_lane<M>((uint32_t)v);
    const uint32_t hi = xor_lane<M>((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Hand-off between lanes of one wave through LDS: every LDS access the wave
// issued before it has completed (its writes and atomics are visible to every
// lane) before any access after it.
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();
}

// one compare-exchange stage across lanes (partner lane ^ M)
template <int E, int M>
__device__ __forceinline__ void cross_stage(uint64_t (&k)[E], int lane, int size, int stride) {
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int e = lane * E + r;
        const uint64_t o = xor_lane_u64<M>(k[r]);
        const bool take_min = ((e & stride) == 0) == ((e & size) == 0);
        const uint64_t mn = o < k[r] ? o : k[r], mx = o < k[r] ? k[r] : o;
        k[r] = take_min ? mn : mx;
    }
}

// ascending bitonic sort of the wave's 64 E keys
template <int E>
__device__ __forceinline__ void wave_sort(uint64_t (&k)[E], int lane) {
    constexpr int P = 64 * E;
#pragma unroll
    for (int size = 2; size <= P; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= E) {
                switch (stride / E) {
                case 1: cross_stage<E, 1>(k, lane, size, stride); break;
                case 2: cross_stage<E, 2>(k, lane, size, stride); break;
                case 4: cross_stage<E, 4>(k, lane, size, stride); break;
                case 8: cross_stage<E, 8>(k, lane, size, stride); break;
                case 16: cross_stage<E, 16>(k, lane, size, stride); break;
                default: cross_stage<E, 32>(k, lane, size, stride); break;
                }
            } else {
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    if (r & stride) continue;
                    const bool up = ((lane * E + r) & size) == 0;
                    const uint64_t x = k[r], y = k[r + stride];
                    const bool sw = (x > y) == up;
                    k[r] = sw ? y : x;
                    k[r + stride] = sw ? x : y;
                }
            }
        }
    }
}

template <int E>
__global__ __launch_bounds__(kThreads) void k_select_w(SelectArgs a) {
    __shared__ uint32_t s_bits[kSelWaves][kSelMaxWords];
    __shared__ uint32_t s_hist[kSelWaves][256];
    extern __shared__ double s_cum[];                  // mass rule: [kSelWaves][64 E]
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * kSelWaves + wv;
    if (row >= a.rows) return;
    const int nb = a.nb;
    const int i = (int)(row % nb);
    const int h = (int)((row / nb) % a.H);
    uint32_t* bits = s_bits[wv];
    for (int w = lane; w < kSelMaxWords; w += 64) bits[w] = 0;
    wave_lds_sync();
    auto mark = [&](int j) {
        if ((uint32_t)j < (uint32_t)nb) atomicOr(&bits[j >> 5], 1u << (j & 31));
    };

    if (a.rule != SA_RULE_NONE) {
        const float* S = a.S + row * (int64_t)nb;
        uint64_t k[E];
#pragma unroll
        for (int r = 0; r < E; ++r) {
            const int j = lane * E + r;
            k[r] = j < nb ? ((uint64_t)(~ordered_bits(S[j])) << 32) | (uint32_t)j : ~0ull;
        }
        if (a.rule == SA_RULE_TOPK) {
            int m = a.H <= kInlineHeads ? a.k_inline[h] : a.k_head[h];
            m = m < 0 ? 0 : (m > nb ? nb : m);
            if (m > 0) {
                uint32_t* hist = s_hist[wv];
                uint64_t prefix = 0, mask = 0;
                uint32_t krem = (uint32_t)m;
                for (int pass = 0; pass < 8; ++pass) {
                    const int sh = 56 - 8 * pass;
                    wave_lds_sync();          // the last pass's reads are done
                    for (int b = lane; b < 256; b += 64) hist[b] = 0;
                    wave_lds_sync();
#pragma unroll
                    for (int r = 0; r < E; ++r)
                        if ((k[r] & mask) == prefix) atomicAdd(&hist[(uint32_t)(k[r] >> sh) & 255u], 1u);
                    wave_lds_sync();
                    uint32_t c[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) c[q] = hist[lane * 4 + q];
                    const uint32_t lsum = c[0] + c[1] + c[2] + c[3];
                    uint32_t incl = lsum;
#pragma unroll
                    for (int off = 1; off < 64; off <<= 1) {
                        const uint32_t y = (uint32_t)__shfl_up((int)incl, off, 64);
                        if (lane >= off) incl += y;
                    }
                    // the lane holding the bucket of the krem-th candidate
                    const int L = __ffsll((unsigned long long)__ballot(incl >= krem)) - 1;
                    uint32_t below = (uint32_t)__builtin_amdgcn_readlane((int)(incl - lsum), L);
                    int b = 0;
                    uint32_t cb = 0;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t cq = (uint32_t)__builtin_amdgcn_readlane((int)c[q], L);
                        if (cb == 0 && below + cq >= krem) {
                            b = L * 4 + q;
                            cb = cq;
                        } else if (cb == 0) {
                            below += cq;
                        }
                    }
                    krem -= below;
                    prefix |= (uint64_t)b << sh;
                    mask |= (uint64_t)255 << sh;
                    if (cb == krem) break;   // the whole bucket is kept
                }
#pragma unroll
                for (int r = 0; r < E; ++r)
                    if ((k[r] & mask) <= prefix) mark((int)(uint32_t)k[r]);
            }
        } else {
            wave_sort<E>(k, lane);
            // p_r = exp(S_r - S_max) in fp64, rank r = lane E + reg
            const double smax =
                (double)ordered_to_float(~(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(k[0] >> 32)));
            double* cum = s_cum + wv * 64 * E;
#pragma unroll
            for (int r = 0; r < E; ++r)
                cum[lane * E + r] =
                    lane * E + r < nb ? exp((double)ordered_to_float(~(uint32_t)(k[r] >> 32)) - smax) : 0.0;
            // the running sum strictly in rank order, by one lane, 8 values
            // per LDS round trip; the ranks past nb add +0.0, which leaves a
            // non-negative sum unchanged
            wave_lds_sync();
            if (lane == 0) {
                double run = 0.0;
                for (int c = 0; c < nb; c += 8) {
                    double v[8];
#pragma unroll
                    for (int q = 0; q < 8; ++q) v[q] = cum[c + q];
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        run += v[q];
                        v[q] = run;
                    }
#pragma unroll
                    for (int q = 0; q < 8; ++q) cum[c + q] = v[q];
                }
            }
            wave_lds_sync();
            // the cut: the first rank whose running sum reaches mass x total
            const double thr = (double)a.mass * cum[nb - 1];
            int first = E;
#pragma unroll
            for (int r = E - 1; r >= 0; --r)
                if (lane * E + r < nb && cum[lane * E + r] >= thr) first = r;
            const uint64_t hit = __ballot(first < E);
            int m = nb;
            if (hit) {
                const int L = __ffsll((unsigned long long)hit) - 1;
                m = L * E + __builtin_amdgcn_readlane(first, L) + 1;
            }
#pragma unroll
            for (int r = 0; r < E; ++r)
                if (lane * E + r < m) mark((int)(uint32_t)k[r]);
        }
    }

    if (a.diag && lane == 0) mark(i);
    if (a.window_frames >= 0) {
        // the blocks whose frames meet [lo_i - r, hi_i + r]: a block's first
        // and last frame grow with its index, so they form one range [jb, ja]
        const int r = a.window_frames;
        const int lo_i = (i * a.block) / a.HgW;
        const int hi_i = (min(a.N, (i + 1) * a.block) - 1) / a.HgW;
        const int A = hi_i + r, B = lo_i - r;
        int ja = -1, jb = 0;
        if (A >= 0) ja = min(nb - 1, (int)(((int64_t)(A + 1) * a.HgW - 1) / a.block));
        if (B > 0) {
            const int64_t t = (int64_t)B * a.HgW + 1;
            jb = t > a.N ? nb : (int)((t + a.block - 1) / a.block) - 1;
        }
        for (int w = lane; w < a.words; w += 64) {
            const int b0 = max(jb, 32 * w), b1 = min(ja, 32 * w + 31);
            if (b0 <= b1) {
                const int n = b1 - b0 + 1;
                const uint32_t m = (n == 32 ? ~0u : ((1u << n) - 1u)) << (b0 - 32 * w);
                atomicOr(&bits[w], m);
            }
        }
    }
    if (a.n_anchors > 0) {
        const int64_t step = nb / a.n_anchors;
        for (int m = lane; m < a.n_anchors; m += 64) mark((int)((a.anchor_offset + m * step) % nb));
    }
    wave_lds_sync();
    uint32_t* out = a.bits + row * (int64_t)a.words;
    int local = 0;
    for (int w = lane; w < a.words; w += 64) {
        const uint32_t word = bits[w];
        out[w] = word;
        local += __popc(word);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off, 64);
    if (lane == 0) a.counts[row] = local;
}

// ----------------------------------------------------------------------------
// k_scan: exclusive scan of counts[R] -> row_ptr[R+1], one workgroup
// ----------------------------------------------------------------------------
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 16;

__global__ __launch_bounds__(kScanThreads) void k_scan(const int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ row_ptr,
                                                       int64_t R) {
    __shared__ int32_t wsum[kScanThreads / 64];
    __shared__ int32_t s_carry;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int64_t base = 0; base < R; base += (int64_t)kScanThreads * kScanItems) {
        int32_t v[kScanItems];
        int32_t sum = 0;
        const int64_t my = base + (int64_t)tid * kScanItems;
#pragma unroll
        for (int k = 0; k < kScanItems; ++k) {
            v[k] = (my + k < R) ? counts[my + k] : 0;
            sum += v[k];
        }
        // inclusive scan of per-thread sums within the wave
        int32_t x = sum;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) wsum[wid] = x;
        __syncthreads();
        if (wid == 0) {
            int32_t w = lane < kScanThreads / 64 ? wsum[lane] : 0;
#pragma unroll
            for (int off = 1; off < kScanThreads / 64; off <<= 1) {
                const int32_t y = __shfl_up(w, off, 64);
                if (lane >= off) w += y;
            }
            if (lane < kScanThreads / 64) wsum[lane] = w;
        }
        __syncthreads();
        int32_t run = s_carry + (wid ? wsum[wid - 1] : 0) + (x - sum);
#pragma unroll
        for (int k = 0; k < kScanItems; ++k) {
            if (my + k < R) row_ptr[my + k] = run;
            run += v[k];
        }
        __syncthreads();
        if (tid == kScanThreads - 1) s_carry = run;
        __syncthreads();
    }
    if (tid == 0) row_ptr[R] = s_carry;
}

// ----------------------------------------------------------------------------
// k_expand: one wave per row, bitmap -> ascending column list
// ----------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_expand(const uint32_t* __restrict__ bits,
                                                     const int32_t* __restrict__ row_ptr,
                                                     int32_t* __restrict__ col_idx,
                                                     int64_t R, int words) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (row >= R) return;
    const uint32_t* b = bits + row * (int64_t)words;
    int32_t base = row_ptr[row];
    for (int w0 = 0; w0 < words; w0 += 64) {
        const int w = w0 + lane;
        uint32_t word = w < words ? b[w] : 0u;
        const int cnt = __popc(word);
        int x = cnt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        int pos = base + x - cnt;
        while (word) {
            const int bit = __ffs(word) - 1;
            col_idx[pos++] = w * 32 + bit;
            word &= word - 1;
        }
        base += __shfl(x, 63, 64);
    }
}

// Writes up to kInlineHeads per-head budgets, passed by value, to device memory
// (stream-ordered; no host buffer has to outlive the call).
struct HeadChunk {
    int32_t k[kInlineHeads];
};

__global__ void k_set_heads(int32_t* __restrict__ dst, HeadChunk c, int n) {
    if ((int)threadIdx.x < n) dst[threadIdx.x] = c.k[threadIdx.x];
}

template <int D, int BLK>
void launch_pool_t(const PoolArgs& a, int nroles, int64_t BH, int nb, hipStream_t s) {
    hipLaunchKernelGGL((k_pool<D, BLK>), dim3(nb, (unsigned)BH, nroles), dim3(kThreads), 0, s, a);
}

template <int D, int SPB>
sa_status launch_score_t(const float* qm, const float* km, float* S, int nb, int n_units,
                         float scale, int64_t BH, hipStream_t s) {
    // two by two block pairs per thread when a block has one or two units
    constexpr int MT = SPB <= 2 ? 2 : 1;
    constexpr int TB = kTile * MT;
    const dim3 grid((nb + TB - 1) / TB, (nb + TB - 1) / TB, (unsigned)BH);
    const size_t lds = 2 * TB * (SPB * kScoreChunk + 4) * sizeof(float);
    if (lds > 65536) {
        sa_status st = ensure_max_lds((const void*)k_score<D, SPB, MT>, (int)lds,
                                      "k_score shared memory");
        if (st != SA_OK) return st;
    }
    hipLaunchKernelGGL((k_score<D, SPB, MT>), grid, dim3(kThreads), lds, s, qm, km, S, nb, n_units,
                       scale);
    return hip_check(hipGetLastError(), "k_score launch");
}

template <int D>
sa_status launch_score_d(int spb, const float* qm, const float* km, float* S, int nb,
                         int n_units, float scale, int64_t BH, hipStream_t s) {
    switch (spb) {
    case 1: return launch_score_t<D, 1>(qm, km, S, nb, n_units, scale, BH, s);
    case 2: return launch_score_t<D, 2>(qm, km, S, nb, n_units, scale, BH, s);
    case 4: return launch_score_t<D, 4>(qm, km, S, nb, n_units, scale, BH, s);
    default: return launch_score_t<D, 8>(qm, km, S, nb, n_units, scale, BH, s);
    }
}

}  // namespace

SelectPlan make_select_plan(const Geometry& g, const sa_select_spec& s) {
    SelectPlan p{};
    p.rule = s.rule;
    p.unit = s.sub_block ? s.sub_block : g.block;
    p.n_units = (int32_t)ceil_div(g.N, p.unit);
    p.spb = g.block / p.unit;
    p.nb_pad = 1;
    while (p.nb_pad < g.nb) p.nb_pad <<= 1;
    if (p.nb_pad < 2) p.nb_pad = 2;
    p.words = (int32_t)ceil_div(g.nb, 32);
    p.mass = s.mass;
    p.diag = s.diag;
    p.window_frames = s.window_frames;
    p.n_anchors = s.n_anchors;
    p.anchor_offset = s.anchor_offset;
    p.want_comp = s.want_comp;
    size_t off = 0;
    const bool scored = s.rule != SA_RULE_NONE;
    const size_t means = scored ? (size_t)g.BH() * p.n_units * g.d * sizeof(float) : 0;
    p.off_qm = off; off = align_up(off + means, 256);
    p.off_km = off; off = align_up(off + means, 256);
    p.off_scores = off;
    off = align_up(off + (scored ? (size_t)g.rows() * g.nb * sizeof(float) : 0), 256);
    p.off_bits = off; off = align_up(off + (size_t)g.rows() * p.words * sizeof(uint32_t), 256);
    p.off_counts = off; off = align_up(off + (size_t)g.rows() * sizeof(int32_t), 256);
    p.off_k = off; off = align_up(off + (size_t)g.H * sizeof(int32_t), 256);
    const bool err = s.rule == SA_RULE_ERR;
    p.v_blocks = err ? static_cast<uint16_t*>(s.v_blocks) : nullptr;
    p.off_vt = off;
    off = align_up(off + (err && !p.v_blocks ? (size_t)g.BH() * g.nb * g.d * g.block * 2 : 0), 256);
    p.off_keys = off;
    off = align_up(off + (err ? (size_t)g.rows() * g.nb * sizeof(float) : 0), 256);
    p.total = off;
    return p;
}

sa_status launch_pooled_scores(int d, const float* qm, const float* km, float* S, int n,
                               float scale, int64_t BH, hipStream_t stream) {
    return d == 128 ? launch_score_d<128>(1, qm, km, S, n, n, scale, BH, stream)
                    : launch_score_d<64>(1, qm, km, S, n, n, scale, BH, stream);
}

sa_status launch_row_scan(const int32_t* counts, int32_t* row_ptr, int64_t R, hipStream_t stream) {
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, stream, counts, row_ptr, R);
    return hip_check(hipGetLastError(), "k_scan launch");
}

sa_status launch_centroids(const Geometry& g, const uint16_t* K, const uint16_t* V, float* k_mean,
                           float* v_sum, hipStream_t stream) {
    PoolArgs pa{};
    pa.order = g.order;
    pa.src[1] = K; pa.src[2] = V;
    pa.block_out[1] = k_mean; pa.block_out[2] = v_sum;
    pa.roles[0] = 1; pa.roles[1] = 2;
    pa.N = g.N; pa.nb = g.nb; pa.unit = g.block; pa.n_units = g.nb;
    if (g.d == 128) {
        if (g.block == 128) launch_pool_t<128, 128>(pa, 2, g.BH(), g.nb, stream);
        else launch_pool_t<128, 64>(pa, 2, g.BH(), g.nb, stream);
    } else {
        if (g.block == 128) launch_pool_t<64, 128>(pa, 2, g.BH(), g.nb, stream);
        else launch_pool_t<64, 64>(pa, 2, g.BH(), g.nb, stream);
    }
    return hip_check(hipGetLastError(), "k_pool launch");
}

sa_status launch_select(const Geometry& g, const SelectPlan& p, const int32_t* k_host,
                        const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                        int32_t* row_ptr, int32_t* col_idx, float* scores, float* k_mean,
                        float* v_sum, char* ws, hipStream_t stream) {
    const bool scored = p.rule != SA_RULE_NONE;
    const bool err = p.rule == SA_RULE_ERR;
    float* qm = reinterpret_cast<float*>(ws + p.off_qm);
    float* km = reinterpret_cast<float*>(ws + p.off_km);
    // pooled scores; with the error rule they only feed the routing keys,
    // which take their place as the ranking key (and as the scores output)
    float* S = (scores && !err) ? scores : reinterpret_cast<float*>(ws + p.off_scores);
    float* keys = err ? (scores ? scores : reinterpret_cast<float*>(ws + p.off_keys)) : nullptr;
    uint32_t* bits = reinterpret_cast<uint32_t*>(ws + p.off_bits);
    int32_t* counts = reinterpret_cast<int32_t*>(ws + p.off_counts);
    int32_t* k_dev = reinterpret_cast<int32_t*>(ws + p.off_k);
    sa_status st;

    // 1. pooling
    PoolArgs pa{};
    pa.order = g.order;
    pa.src[0] = Q; pa.src[1] = K; pa.src[2] = V;
    pa.N = g.N; pa.nb = g.nb; pa.unit = p.unit; pa.n_units = p.n_units;
    int nroles = 0;
    if (scored) {
        pa.unit_out[0] = qm;
        pa.roles[nroles++] = 0;
    }
    if (scored || p.want_comp) {
        pa.unit_out[1] = scored ? km : nullptr;
        pa.block_out[1] = p.want_comp ? k_mean : nullptr;
        pa.roles[nroles++] = 1;
    }
    if (p.want_comp) {
        pa.block_out[2] = v_sum;
        pa.roles[nroles++] = 2;
    }
    if (nroles) {
        if (g.d == 128) {
            if (g.block == 128) launch_pool_t<128, 128>(pa, nroles, g.BH(), g.nb, stream);
            else launch_pool_t<128, 64>(pa, nroles, g.BH(), g.nb, stream);
        } else {
            if (g.block == 128) launch_pool_t<64, 128>(pa, nroles, g.BH(), g.nb, stream);
            else launch_pool_t<64, 64>(pa, nroles, g.BH(), g.nb, stream);
        }
        if ((st = hip_check(hipGetLastError(), "k_pool launch")) != SA_OK) return st;
    }

    // 2. scores
    if (scored) {
        st = g.d == 128
                 ? launch_score_d<128>(p.spb, qm, km, S, g.nb, p.n_units, g.scale, g.BH(), stream)
                 : launch_score_d<64>(p.spb, qm, km, S, g.nb, p.n_units, g.scale, g.BH(), stream);
        if (st != SA_OK) return st;
    }

    // 2b. error-aware routing keys
    if (err) {
        uint16_t* vt = p.v_blocks ? p.v_blocks : reinterpret_cast<uint16_t*>(ws + p.off_vt);
        if ((st = launch_vt_layout(g, V, vt, stream)) != SA_OK) return st;
        if ((st = launch_route_keys(g, qm, K, vt, v_sum, S, keys, stream)) != SA_OK) return st;
    }

    // 3. selection
    SelectArgs sa{};
    if (p.rule == SA_RULE_TOPK || err) {
        if (g.H <= kInlineHeads) {
            for (int h = 0; h < g.H; ++h) sa.k_inline[h] = k_host[h];
        } else {
            for (int h0 = 0; h0 < g.H; h0 += kInlineHeads) {
                HeadChunk c{};
                const int n = g.H - h0 < kInlineHeads ? g.H - h0 : kInlineHeads;
                for (int t = 0; t < n; ++t) c.k[t] = k_host[h0 + t];
                hipLaunchKernelGGL(k_set_heads, dim3(1), dim3(kInlineHeads), 0, stream,
                                   k_dev + h0, c, n);
                if ((st = hip_check(hipGetLastError(), "k_set_heads launch")) != SA_OK) return st;
            }
        }
    }
    sa.S = err ? keys : S; sa.k_head = k_dev; sa.bits = bits; sa.counts = counts;
    sa.H = g.H; sa.N = g.N; sa.nb = g.nb; sa.nb_pad = p.nb_pad; sa.words = p.words;
    sa.block = g.block; sa.HgW = g.Hg * g.W; sa.rule = err ? SA_RULE_TOPK : p.rule; sa.mass = p.mass;
    sa.diag = p.diag; sa.window_frames = p.window_frames; sa.n_anchors = p.n_anchors;
    sa.anchor_offset = p.anchor_offset;
    sa.rows = g.rows();
    if (p.nb_pad <= 64 * 32) {
        // one wave per row, E = nb_pad / 64 keys per lane
        const dim3 grid((unsigned)ceil_div(g.rows(), kSelWaves));
        // without scores no keys are held: the one-key build
        const int E = !scored || p.nb_pad <= 64 ? 1 : p.nb_pad / 64;
        // mass rule: the running sums of each wave's row in LDS
        const size_t lds = p.rule == SA_RULE_MASS ? (size_t)kSelWaves * 64 * E * sizeof(double) : 0;
        if (E == 32 && lds > 0) {
            st = ensure_max_lds((const void*)k_select_w<32>, (int)lds, "k_select shared memory");
            if (st != SA_OK) return st;
        }
        switch (E) {
        case 1: hipLaunchKernelGGL(k_select_w<1>, grid, dim3(kThreads), lds, stream, sa); break;
        case 2: hipLaunchKernelGGL(k_select_w<2>, grid, dim3(kThreads), lds, stream, sa); break;
        case 4: hipLaunchKernelGGL(k_select_w<4>, grid, dim3(kThreads), lds, stream, sa); break;
        case 8: hipLaunchKernelGGL(k_select_w<8>, grid, dim3(kThreads), lds, stream, sa); break;
        case 16: hipLaunchKernelGGL(k_select_w<16>, grid, dim3(kThreads), lds, stream, sa); break;
        default: hipLaunchKernelGGL(k_select_w<32>, grid, dim3(kThreads), lds, stream, sa); break;
        }
    } else {
        const size_t lds = scored ? (size_t)p.nb_pad * 12 + (size_t)p.words * 32
                                  : (size_t)p.words * 32 + 16;
        hipLaunchKernelGGL(k_select, dim3((unsigned)g.rows()), dim3(kThreads), lds, stream, sa);
    }
    if ((st = hip_check(hipGetLastError(), "k_select launch")) != SA_OK) return st;

    // 4. CSR
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, stream, counts, row_ptr, g.rows());
    if ((st = hip_check(hipGetLastError(), "k_scan launch")) != SA_OK) return st;
    hipLaunchKernelGGL(k_expand, dim3((unsigned)ceil_div(g.rows(), kThreads / 64)), dim3(kThreads),
                       0, stream, bits, row_ptr, col_idx, g.rows(), p.words);
    return hip_check(hipGetLastError(), "k_expand launch");
}

}  // namespace sa
