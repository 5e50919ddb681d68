// Block-sparse attention forward for gfx950 (SVG-EAR page, section 2B:
// streaming softmax update over the computed blocks without materialising the
// logits; SPADE page, part 3: a head-wise sparse attention kernel).  With
// compensation, every skipped KV block contributes one centroid pseudo-token
// (SVG-EAR page, section 2A): key = block mean of K, value = block mean of V,
// weight = the block's token count (a logit bias of log n_j).
//
// Mapping onto CDNA4
//   * one workgroup = one (batch, head, query block).  Wave (qg, kh) owns 64
//     queries (query group qg) and one half of the keys of every KV tile (kh);
//     the two key halves are merged once at the end, like two KV splits.
//     64 queries per wave means every K / V operand read from LDS feeds two
//     matrix-core instructions, halving LDS traffic per flop.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: Q^T (B operand) stays in
//     registers for the whole row, K (A operand) is read from LDS.  In the
//     32x32 accumulator layout a lane holds one query column, so the softmax
//     statistics are lane-local; the two lane halves sharing a query exchange
//     their maximum once per tile (xor 32).
//   * O^T = V^T P^T on the same instruction: P goes from the S^T accumulators
//     into the B operand.  K rows are read in an order that swaps bits 2 and 3
//     of the row index, which makes the 8 probabilities a lane holds per
//     k-step 8 consecutive keys; V is pre-transposed per block in HBM (a cheap
//     bandwidth-bound pass) so those 8 keys are one 16-byte LDS read.
//   * K and V^T tiles move HBM -> LDS with global_load_lds_dwordx4 (no
//     register staging), double-buffered: tile t+1 is in flight while tile t
//     is computed.  Tiles use an XOR swizzle of their 16-byte chunks so that
//     the row-strided operand reads are bank-conflict free.
//   * online softmax in the log2 domain with lazy rescaling: the running
//     maximum only moves (and O, l are only rescaled) when a tile raises it by
//     more than 2^8.
//   * blockIdx -> row remap keeps consecutive query blocks of a head on one
//     XCD (workgroups are dealt round-robin to the 8 XCDs), so the K/V blocks
//     they share are served from that XCD's L2.
#include <math.h>

#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;      // log2 headroom before the running max moves

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

// x[lane] op x[lane ^ 32] through the VALU half-wave swap (no LDS round trip):
// the two results of v_permlane32_swap hold x of this lane and of its partner.
__device__ __forceinline__ float xmax32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct FwdArgs {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* Vt;      // [BH][nb][D][BLK] transposed V blocks (zero-padded keys)
    const int32_t* row_ptr;
    const int32_t* col_idx;
    const uint16_t* kbar;    // [BH][nb][D] centroid keys (compensation) or null
    const uint16_t* vbart;   // [BH][ntc][D][BLK] transposed centroid values
    uint16_t* O;
    float* lse;
    int32_t* sched;          // [3][8] per-XCD row range start, end and pull counter
    int32_t N, nb, ntc;
    int64_t rows;
    float c;                 // scale * log2(e)
};

// Query tiles (of 32 queries) per wave.  Two halve the LDS operand traffic per
// flop but need ~360 registers (one wave per SIMD); one keeps a wave under 256
// registers so that two waves share every SIMD and the hardware overlaps one
// wave's matrix-core work with the other's softmax.
#ifndef SA_NQT
#define SA_NQT 1
#endif
constexpr int NQT = SA_NQT;

template <int D, int BLK>
struct Cfg {
    static constexpr int QW = 32 * NQT;             // queries per wave
    static constexpr int NWQ = BLK / QW;            // query groups
    static constexpr int NW = NWQ * 2;              // x 2 key halves
    static constexpr int NT = NW * 64;
    static constexpr int KH = BLK / 2;              // keys per half
    static constexpr int KTW = KH / 32;             // 32-key MFMA tiles per wave
    static constexpr int KRB = D * 2;               // bytes per K row
    static constexpr int VRB = BLK * 2;             // bytes per V^T row
    static constexpr int KCH = KRB / 16;            // 16-byte chunks per K row
    static constexpr int VCH = VRB / 16;
    static constexpr int K_BYTES = BLK * KRB;
    static constexpr int V_BYTES = D * VRB;
    static constexpr int STAGE = K_BYTES + V_BYTES + BLK * 4;   // + bias
    static constexpr int MERGE = NWQ * (NQT * (D / 32) * 64 * 16 * 4 + 2 * NQT * 32 * 4);
    static constexpr int BASE = 2 * STAGE > MERGE ? 2 * STAGE : MERGE;
    static constexpr int MAX_NB = 4096;                 // list / flag capacity
};

// Byte offset, inside a tile of ROWS rows of RB bytes, of the 16-byte chunk that
// lane `lane` of wave `wave` fetches with DMA instruction n.  The tile's 16-byte
// chunks are XOR-swizzled by the row index; every wave instruction fills 1 KB
// of LDS, lane L landing at byte L*16 of the wave's slice.
template <int RB, int NW>
__device__ __forceinline__ uint32_t dma_src_offset(int n, int wave, int lane, int max_row) {
    constexpr int CH = RB / 16;
    const int lin = (n * NW + wave) * 1024 + lane * 16;
    const int row = lin / RB;
    const int chunk = ((lin % RB) / 16) ^ (row & (CH - 1));
    return (uint32_t)((row < max_row ? row : max_row) * RB + chunk * 16);
}

// HBM -> LDS copy of one tile: global_load_lds_dwordx4 per wave instruction,
// source = base (uniform, SGPRs) + this lane's offset, destination = the wave's
// 1 KB slice.  Issued through inline assembly so that the compiler does not
// treat every later LDS read as dependent on these copies (it cannot tell the
// two stages apart and would wait for all of them, which removes the overlap
// of the copy of tile t+1 with the compute of tile t); completion is ordered
// explicitly by the s_waitcnt vmcnt(0) + barrier at the top of every tile.  The
// instruction has no register results; M0 carries the LDS address and is
// restored afterwards.
template <int ROWS, int RB, int NW>
__device__ __forceinline__ void dma_tile(unsigned char* tile, const unsigned char* base,
                                         const uint32_t (&off)[ROWS * RB / (1024 * NW)], int wave) {
    constexpr int INSTR = ROWS * RB / (1024 * NW);
    static_assert(INSTR * 1024 * NW == ROWS * RB, "tile must be a whole number of wave slices");
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)tile;
#pragma unroll
    for (int n = 0; n < INSTR; ++n) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + (n * NW + wave) * 1024);
        uint32_t saved;
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %2, %3\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(dst), "v"(off[n]), "s"(base)
            : "memory");
    }
}

// One row = one (batch, head, query block): all its kept tiles, then (with
// compensation) the centroid tiles, then the merge of the two key halves.
template <int D, int BLK, bool COMP>
__device__ __forceinline__ void process_row(const FwdArgs& a, int64_t row, unsigned char* smem) {
    using C = Cfg<D, BLK>;
    unsigned char* kept = smem + C::BASE;                              // COMP: [nb] flags
    int16_t* list = reinterpret_cast<int16_t*>(smem + C::BASE + C::MAX_NB);  // kept blocks

    const int i = (int)(row % a.nb);
    const int64_t bh = row / a.nb;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qg = wave >> 1, kh = wave & 1;
    const int r32 = lane & 31, h = lane >> 5;
    const int64_t head_off = bh * (int64_t)a.N * D;
    const unsigned char* Kh = reinterpret_cast<const unsigned char*>(a.K + head_off);
    const unsigned char* Vth =
        reinterpret_cast<const unsigned char*>(a.Vt + bh * (int64_t)a.nb * D * BLK);
    const int last_n = a.N - (a.nb - 1) * BLK;

    // Q^T fragments (B operand) of this wave's 64 queries
    bf16x8 qf[NQT][D / 16];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) {
        const int qn = i * BLK + qg * C::QW + nt * 32 + r32;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (qn < a.N)
                v = *reinterpret_cast<const uint4*>(a.Q + head_off + (int64_t)qn * D + st * 16 + h * 8);
            qf[nt][st] = as_bf16x8(v);
        }
    }

    const int beg = a.row_ptr[row], end = a.row_ptr[row + 1];
    const int nk = end - beg;
    const int T = nk + (COMP ? a.ntc : 0);
    // the row's kept blocks (clamped into range) and, for compensation, flags
    if constexpr (COMP)
        for (int j = tid; j < a.nb; j += C::NT) kept[j] = 0;
    for (int e = tid; e < nk; e += C::NT) {
        int j = a.col_idx[beg + e];
        j = j < 0 ? 0 : (j >= a.nb ? a.nb - 1 : j);
        list[e] = (int16_t)j;
    }
    __syncthreads();
    if constexpr (COMP) {
        for (int e = tid; e < nk; e += C::NT) kept[list[e]] = 1;
        __syncthreads();
    }

    // per-lane DMA source offsets (full tiles; the clamped set for a short block)
    constexpr int KI = C::K_BYTES / (1024 * C::NW), VI = C::V_BYTES / (1024 * C::NW);
    uint32_t koff[KI], voff[VI];
#pragma unroll
    for (int n = 0; n < KI; ++n) koff[n] = dma_src_offset<C::KRB, C::NW>(n, wave, lane, BLK - 1);
#pragma unroll
    for (int n = 0; n < VI; ++n) voff[n] = dma_src_offset<C::VRB, C::NW>(n, wave, lane, D - 1);

    // Issues the HBM -> LDS copies of tile t into stage buffer b and writes its
    // key bias (0 / -inf for a short last block; log2 n_j / -inf for centroids).
    const float inv_c = 1.f / a.c;
    auto issue = [&](int t, int b) {
        unsigned char* st = smem + b * C::STAGE;
        float* bias = reinterpret_cast<float*>(st + C::K_BYTES + C::V_BYTES);
        if (!COMP || t < nk) {
            const int j = __builtin_amdgcn_readfirstlane(list[t]);
            const unsigned char* kb = Kh + (int64_t)j * BLK * C::KRB;
            const unsigned char* vb = Vth + (int64_t)j * D * C::VRB;
            const int nval = j == a.nb - 1 ? last_n : BLK;
            if (nval == BLK) {
                dma_tile<BLK, C::KRB, C::NW>(st, kb, koff, wave);
            } else {
                uint32_t ko[KI];
#pragma unroll
                for (int n = 0; n < KI; ++n) ko[n] = dma_src_offset<C::KRB, C::NW>(n, wave, lane, nval - 1);
                dma_tile<BLK, C::KRB, C::NW>(st, kb, ko, wave);
                for (int r = tid; r < BLK; r += C::NT) bias[r] = r < nval ? 0.f : -INFINITY;
            }
            dma_tile<D, C::VRB, C::NW>(st + C::K_BYTES, vb, voff, wave);
        } else {
            const int tc = t - nk;
            const int j0 = tc * BLK;
            const int nval = a.nb - j0 < BLK ? a.nb - j0 : BLK;
            const unsigned char* kb =
                reinterpret_cast<const unsigned char*>(a.kbar + (bh * a.nb + j0) * (int64_t)D);
            uint32_t ko[KI];
#pragma unroll
            for (int n = 0; n < KI; ++n) ko[n] = dma_src_offset<C::KRB, C::NW>(n, wave, lane, nval - 1);
            dma_tile<BLK, C::KRB, C::NW>(st, kb, ko, wave);
            const unsigned char* vb = reinterpret_cast<const unsigned char*>(
                a.vbart + (bh * a.ntc + tc) * (int64_t)D * BLK);
            dma_tile<D, C::VRB, C::NW>(st + C::K_BYTES, vb, voff, wave);
            for (int r = tid; r < BLK; r += C::NT) {
                const int j = j0 + r;
                float bv = -INFINITY;
                if (j < a.nb && !kept[j]) bv = __log2f((float)(j == a.nb - 1 ? last_n : BLK)) * inv_c;
                bias[r] = bv;
            }
        }
    };

    f32x16 oacc[D / 32][NQT];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) oacc[dt][nt] = f32x16{};
    float m_run[NQT], l_run[NQT];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) { m_run[nt] = -INFINITY; l_run[nt] = 0.f; }

    // One KV tile for this wave: S^T = K Q^T over its key half, online softmax
    // (log2 domain, lazy rescale), O^T += V^T P^T.  Operands are streamed from
    // LDS.  A tile with masked or weighted keys (short last block: -inf past its
    // end; centroid tiles: log2 n_j, -inf for kept blocks) adds its key bias,
    // stored divided by the log2-domain scale c, to the raw scores; the max is
    // taken on raw scores (c > 0), and c s - m is one FMA.
    const bf16x2 kOnes2 = {(__bf16)1.f, (__bf16)1.f};
    auto attend = [&](const unsigned char* Ks, const unsigned char* Vs, const float* bias,
                      bool biased) {
        f32x16 s[C::KTW][NQT];
#pragma unroll
        for (int kt = 0; kt < C::KTW; ++kt)
#pragma unroll
            for (int nt = 0; nt < NQT; ++nt) s[kt][nt] = f32x16{};
#pragma unroll
        for (int st = 0; st < D / 16; ++st)
#pragma unroll
            for (int kt = 0; kt < C::KTW; ++kt) {
                const int krow = kh * C::KH + kt * 32 + swap23(r32);
                const int pos = (st * 2 + h) ^ (krow & (C::KCH - 1));
                const bf16x8 kop = as_bf16x8(*reinterpret_cast<const uint4*>(Ks + krow * C::KRB + pos * 16));
#pragma unroll
                for (int nt = 0; nt < NQT; ++nt)
                    s[kt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qf[nt][st], s[kt][nt], 0, 0, 0);
            }
        if (biased) {
#pragma unroll
            for (int kt = 0; kt < C::KTW; ++kt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int key = kh * C::KH + kt * 32 + 16 * (g >> 1) + 8 * h + 4 * (g & 1);
                    const float4 bv = *reinterpret_cast<const float4*>(bias + key);
                    const float b4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                    for (int nt = 0; nt < NQT; ++nt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) s[kt][nt][4 * g + e] += b4[e];
                }
        }

        bf16x8 pb[C::KTW][2][NQT];
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < C::KTW; ++kt)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kt][nt][e]);
            mx = xmax32(mx) * a.c;
            if (mx > m_run[nt] + kLazy) {
                const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - mx);
                l_run[nt] *= alpha;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt) oacc[dt][nt] *= alpha;
                m_run[nt] = mx;
            }
            const float nbase = m_run[nt] == -INFINITY ? 0.f : -m_run[nt];
            // the row sum adds the bf16 weights that enter P V
            float sum = l_run[nt];
#pragma unroll
            for (int kt = 0; kt < C::KTW; ++kt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        pb[kt][s2][nt][e] =
                            (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][nt][8 * s2 + e], a.c, nbase));
                    const bf16x8 w = pb[kt][s2][nt];
                    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 0, 1), kOnes2, sum, false);
                    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 2, 3), kOnes2, sum, false);
                    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 4, 5), kOnes2, sum, false);
                    sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(w, w, 6, 7), kOnes2, sum, false);
                }
            l_run[nt] = sum;
        }

#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const int d = dt * 32 + r32;
#pragma unroll
            for (int kt = 0; kt < C::KTW; ++kt)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int chunk = (kh * C::KH + kt * 32 + 16 * s2 + 8 * h) / 8;
                    const int pos = chunk ^ (d & (C::VCH - 1));
                    const bf16x8 vop = as_bf16x8(*reinterpret_cast<const uint4*>(Vs + d * C::VRB + pos * 16));
#pragma unroll
                    for (int nt = 0; nt < NQT; ++nt)
                        oacc[dt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[kt][s2][nt], oacc[dt][nt], 0, 0, 0);
                }
        }
    };

    if (T > 0) issue(0, 0);
    for (int t = 0; t < T; ++t) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (t + 1 < T) issue(t + 1, (t + 1) & 1);
        const unsigned char* Ks = smem + (t & 1) * C::STAGE;
        const unsigned char* Vs = Ks + C::K_BYTES;
        const float* bias = reinterpret_cast<const float*>(Vs + C::V_BYTES);
        bool biased = COMP && t >= nk;
        if (!biased) biased = last_n < BLK && __builtin_amdgcn_readfirstlane(list[t]) == a.nb - 1;
        attend(Ks, Vs, bias, biased);
    }

    // merge the two key halves of every query group, then write O and lse
    float l_tot[NQT];
#pragma unroll
    for (int nt = 0; nt < NQT; ++nt) l_tot[nt] = xsum32(l_run[nt]);
    __syncthreads();                                   // stage buffers are free
    float4* mo = reinterpret_cast<float4*>(smem + qg * (C::MERGE / C::NWQ));
    float* ml = reinterpret_cast<float*>(smem + qg * (C::MERGE / C::NWQ) + NQT * (D / 32) * 64 * 16 * 4);
    if (kh == 1) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int nt = 0; nt < NQT; ++nt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    mo[((dt * NQT + nt) * 4 + g) * 64 + lane] =
                        make_float4(oacc[dt][nt][4 * g], oacc[dt][nt][4 * g + 1],
                                    oacc[dt][nt][4 * g + 2], oacc[dt][nt][4 * g + 3]);
        if (h == 0)
#pragma unroll
            for (int nt = 0; nt < NQT; ++nt) {
                ml[nt * 32 + r32] = m_run[nt];
                ml[NQT * 32 + nt * 32 + r32] = l_tot[nt];
            }
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
        for (int nt = 0; nt < NQT; ++nt) {
            const float m1 = ml[nt * 32 + r32], l1 = ml[NQT * 32 + nt * 32 + r32];
            const float m0 = m_run[nt];
            const float m = fmaxf(m0, m1);
            const float mb = m == -INFINITY ? 0.f : m;
            const float a0 = __builtin_amdgcn_exp2f(m0 - mb), a1 = __builtin_amdgcn_exp2f(m1 - mb);
            const float l = l_tot[nt] * a0 + l1 * a1;
            const float inv = l > 0.f ? 1.f / l : 0.f;
            const int qn = i * BLK + qg * C::QW + nt * 32 + r32;
            if (qn < a.N) {
                uint16_t* orow = a.O + head_off + (int64_t)qn * D;
#pragma unroll
                for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 o1 = mo[((dt * NQT + nt) * 4 + g) * 64 + lane];
                        const float v0 = (oacc[dt][nt][4 * g + 0] * a0 + o1.x * a1) * inv;
                        const float v1 = (oacc[dt][nt][4 * g + 1] * a0 + o1.y * a1) * inv;
                        const float v2 = (oacc[dt][nt][4 * g + 2] * a0 + o1.z * a1) * inv;
                        const float v3 = (oacc[dt][nt][4 * g + 3] * a0 + o1.w * a1) * inv;
                        const uint32_t lo = f32_to_bf16_rne(v0) | ((uint32_t)f32_to_bf16_rne(v1) << 16);
                        const uint32_t hi = f32_to_bf16_rne(v2) | ((uint32_t)f32_to_bf16_rne(v3) << 16);
                        *reinterpret_cast<uint2*>(orow + dt * 32 + 8 * g + 4 * h) = make_uint2(lo, hi);
                    }
                if (a.lse && h == 0)
                    a.lse[bh * (int64_t)a.N + qn] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
            }
        }
    }
}

// Persistent grid.  The rows are split into 8 contiguous ranges of equal work
// (k_sched); workgroup w pulls rows of range w % 8 -- the XCD it is dealt to --
// in order, so concurrently running rows of one XCD are neighbouring query
// blocks that share K/V blocks in that XCD's L2.  A workgroup whose range is
// exhausted takes rows from the other ranges.
template <int D, int BLK, bool COMP>
__global__ __launch_bounds__(BLK * 4 / NQT) __attribute__((amdgpu_waves_per_eu(NQT == 1 ? 2 : 1)))
void k_bsattn_fwd(FwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    __shared__ int s_row;
    const int x0 = blockIdx.x % 8;
    for (int k = 0; k < 8; ++k) {
        const int x = (x0 + k) % 8;
        const int start = a.sched[x], stop = a.sched[8 + x];
        for (;;) {
            if (threadIdx.x == 0) {
                const int idx = start < stop ? atomicAdd(&a.sched[16 + x], 1) : 0;
                s_row = start + idx < stop ? start + idx : -1;
            }
            __syncthreads();
            const int row = s_row;
            __syncthreads();
            if (row < 0) break;
            process_row<D, BLK, COMP>(a, row, smem);
        }
    }
}

// Splits the R rows into 8 contiguous ranges of (nearly) equal work, where a
// row costs its number of tiles plus a fixed overhead; resets the pull counters.
constexpr int kSchedThreads = 1024;
constexpr int kSchedItems = 8;

__global__ __launch_bounds__(kSchedThreads) void k_sched(const int32_t* __restrict__ row_ptr,
                                                         int32_t* __restrict__ sched, int64_t R,
                                                         int extra) {
    __shared__ long long wsum[kSchedThreads / 64];
    __shared__ long long s_total, s_carry;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    auto cost = [&](int64_t r) -> long long {
        return (long long)(row_ptr[r + 1] - row_ptr[r]) + extra;
    };
    // total work
    long long part = 0;
    for (int64_t r = tid; r < R; r += kSchedThreads) part += cost(r);
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) wsum[wid] = part;
    if (tid < 8) { sched[tid] = (int32_t)R; sched[8 + tid] = (int32_t)R; sched[16 + tid] = 0; }
    __syncthreads();
    if (tid == 0) {
        long long t = 0;
        for (int k = 0; k < kSchedThreads / 64; ++k) t += wsum[k];
        s_total = t;
        s_carry = 0;
        sched[0] = 0;
    }
    __syncthreads();
    const long long total = s_total;
    // exclusive prefix of the costs; range x starts at the row whose work
    // interval [prefix, prefix + cost) contains x/8 of the total
    for (int64_t base = 0; base < R; base += (int64_t)kSchedThreads * kSchedItems) {
        long long c[kSchedItems], sum = 0;
        const int64_t my = base + (int64_t)tid * kSchedItems;
#pragma unroll
        for (int k = 0; k < kSchedItems; ++k) {
            c[k] = my + k < R ? cost(my + k) : 0;
            sum += c[k];
        }
        long long xs = sum;
        for (int off = 1; off < 64; off <<= 1) {
            const long long y = __shfl_up(xs, off, 64);
            if (lane >= off) xs += y;
        }
        __syncthreads();
        if (lane == 63) wsum[wid] = xs;
        __syncthreads();
        long long run = s_carry + xs - sum;
        for (int k = 0; k < wid; ++k) run += wsum[k];
#pragma unroll
        for (int k = 0; k < kSchedItems; ++k) {
            if (my + k < R) {
                for (int x = 1; x < 8; ++x) {
                    const long long tgt = (long long)x * total;      // 8 * (x/8 of the total)
                    if (run * 8 <= tgt && tgt < (run + c[k]) * 8) sched[x] = (int32_t)(my + k);
                }
            }
            run += c[k];
        }
        __syncthreads();
        if (tid == kSchedThreads - 1) s_carry = run;
        __syncthreads();
    }
    __syncthreads();
    if (tid < 8) sched[8 + tid] = tid < 7 ? sched[tid + 1] : (int32_t)R;
}

// V blocks transposed to [D][BLK] (keys past the end of the sequence are 0).
template <int D, int BLK>
__global__ __launch_bounds__(256) void k_vt_prep(const uint16_t* __restrict__ V,
                                                 uint16_t* __restrict__ Vt, int N, int nb) {
    __shared__ uint16_t tile[BLK][D + 8];
    const int j = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int n = min(BLK, N - j * BLK);
    const uint16_t* src = V + (bh * N + (int64_t)j * BLK) * D;
    for (int c = threadIdx.x; c < BLK * (D / 8); c += 256) {
        const int r = c / (D / 8), ch = c % (D / 8);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < n) v = *reinterpret_cast<const uint4*>(src + (int64_t)r * D + ch * 8);
        *reinterpret_cast<uint4*>(&tile[r][ch * 8]) = v;
    }
    __syncthreads();
    uint16_t* dst = Vt + (bh * nb + j) * (int64_t)D * BLK;
    for (int p = threadIdx.x; p < D * (BLK / 8); p += 256) {
        const int d = p / (BLK / 8), kc = p % (BLK / 8);
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)tile[kc * 8 + 2 * e][d] | ((uint32_t)tile[kc * 8 + 2 * e + 1][d] << 16);
        *reinterpret_cast<uint4*>(dst + (int64_t)d * BLK + kc * 8) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Centroid pseudo-tokens for compensation, rounded to bf16 for the matrix
// cores: kbar = k_mean [nb][D]; vbar = v_sum / n_j, stored transposed in
// tiles of BLK blocks [ntc][D][BLK] (blocks past nb are 0).
template <int D, int BLK>
__global__ __launch_bounds__(256) void k_comp_prep(const float* __restrict__ k_mean,
                                                   const float* __restrict__ v_sum,
                                                   uint16_t* __restrict__ kbar,
                                                   uint16_t* __restrict__ vbart, int nb, int ntc,
                                                   int last_n) {
    const int tc = blockIdx.x;
    const int64_t bh = blockIdx.y;
    for (int p = threadIdx.x; p < BLK * D; p += 256) {
        const int r = p / D, d = p % D;
        const int j = tc * BLK + r;
        if (j < nb) {
            const int64_t e = (bh * nb + j) * (int64_t)D + d;
            kbar[e] = f32_to_bf16_rne(k_mean[e]);
        }
    }
    for (int p = threadIdx.x; p < BLK * D; p += 256) {
        const int d = p / BLK, r = p % BLK;
        const int j = tc * BLK + r;
        uint16_t v = 0;
        if (j < nb) {
            const float n = (float)(j == nb - 1 ? last_n : BLK);
            v = f32_to_bf16_rne(v_sum[(bh * nb + j) * (int64_t)D + d] / n);
        }
        vbart[((bh * ntc + tc) * (int64_t)D + d) * BLK + r] = v;
    }
}

struct WsLayout {
    size_t sched, vt, kbar, vbart, total;
};

WsLayout ws_layout(const Geometry& g, bool comp) {
    WsLayout L{};
    const int64_t ntc = ceil_div(g.nb, g.block);
    size_t off = 0;
    L.sched = off; off = align_up(off + 24 * sizeof(int32_t), 256);
    L.vt = off; off = align_up(off + (size_t)g.BH() * g.nb * g.d * g.block * 2, 256);
    if (comp) {
        L.kbar = off; off = align_up(off + (size_t)g.BH() * g.nb * g.d * 2, 256);
        L.vbart = off; off = align_up(off + (size_t)g.BH() * ntc * g.d * g.block * 2, 256);
    }
    L.total = off;
    return L;
}

template <int D, int BLK, bool COMP>
sa_status launch_t(const FwdArgs& a, const Geometry& g, const uint16_t* V, uint16_t* vt,
                   const float* k_mean, const float* v_sum, uint16_t* kbar, uint16_t* vbart,
                   hipStream_t stream) {
    using C = Cfg<D, BLK>;
    hipLaunchKernelGGL((k_vt_prep<D, BLK>), dim3(g.nb, (unsigned)g.BH()), dim3(256), 0, stream, V,
                       vt, g.N, g.nb);
    sa_status st = hip_check(hipGetLastError(), "k_vt_prep launch");
    if (st != SA_OK) return st;
    if (COMP) {
        hipLaunchKernelGGL((k_comp_prep<D, BLK>), dim3(a.ntc, (unsigned)g.BH()), dim3(256), 0, stream,
                           k_mean, v_sum, kbar, vbart, g.nb, a.ntc, g.N - (g.nb - 1) * BLK);
        if ((st = hip_check(hipGetLastError(), "k_comp_prep launch")) != SA_OK) return st;
    }
    const size_t lds = C::BASE + C::MAX_NB + 2 * (size_t)g.nb;
    static bool configured = false;
    if (!configured) {
        const int most = C::BASE + C::MAX_NB + 2 * C::MAX_NB;
        st = hip_check(hipFuncSetAttribute((const void*)k_bsattn_fwd<D, BLK, COMP>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, most),
                       "k_bsattn_fwd shared memory");
        if (st != SA_OK) return st;
        configured = true;
    }
    if (a.rows == 0) return SA_OK;
    hipLaunchKernelGGL(k_sched, dim3(1), dim3(kSchedThreads), 0, stream, a.row_ptr, a.sched,
                       a.rows, (COMP ? a.ntc : 0) + 2);
    if ((st = hip_check(hipGetLastError(), "k_sched launch")) != SA_OK) return st;
    // persistent grid: as many workgroups as the chip holds at once
    static int resident = 0;
    if (resident == 0) {
        int dev = 0, cus = 0, per_cu = 0;
        if ((st = hip_check(hipGetDevice(&dev), "hipGetDevice")) != SA_OK) return st;
        st = hip_check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev),
                       "multiprocessor count");
        if (st != SA_OK) return st;
        st = hip_check(hipOccupancyMaxActiveBlocksPerMultiprocessor(
                           &per_cu, (const void*)k_bsattn_fwd<D, BLK, COMP>, C::NT,
                           C::BASE + C::MAX_NB + 2 * C::MAX_NB),
                       "occupancy query");
        if (st != SA_OK) return st;
        resident = cus * (per_cu > 0 ? per_cu : 1);
    }
    const int64_t grid = a.rows < resident ? a.rows : resident;
    hipLaunchKernelGGL((k_bsattn_fwd<D, BLK, COMP>), dim3((unsigned)grid), dim3(C::NT), lds, stream, a);
    return hip_check(hipGetLastError(), "k_bsattn_fwd launch");
}

}  // namespace

size_t fwd_workspace_bytes(const Geometry& g, bool comp) { return ws_layout(g, comp).total; }

sa_status launch_fwd(const Geometry& g, const uint16_t* Q, const uint16_t* K, const uint16_t* V,
                     const int32_t* row_ptr, const int32_t* col_idx, const float* k_mean,
                     const float* v_sum, uint16_t* O, float* lse, char* ws, hipStream_t stream) {
    const bool comp = k_mean != nullptr;
    if (g.nb > 4096) return fail(SA_ERR_UNSUPPORTED, "attention supports nb <= 4096 (got %d)", g.nb);
    const WsLayout L = ws_layout(g, comp);
    FwdArgs a{};
    a.Q = Q; a.K = K; a.row_ptr = row_ptr; a.col_idx = col_idx;
    a.O = O; a.lse = lse; a.N = g.N; a.nb = g.nb; a.rows = g.rows();
    a.ntc = (int32_t)ceil_div(g.nb, g.block);
    a.c = g.scale * kLog2e;
    uint16_t* vt = reinterpret_cast<uint16_t*>(ws + L.vt);
    uint16_t* kbar = comp ? reinterpret_cast<uint16_t*>(ws + L.kbar) : nullptr;
    uint16_t* vbart = comp ? reinterpret_cast<uint16_t*>(ws + L.vbart) : nullptr;
    a.Vt = vt; a.kbar = kbar; a.vbart = vbart;
    a.sched = reinterpret_cast<int32_t*>(ws + L.sched);
#define SA_LAUNCH(D_, B_)                                                                      \
    return comp ? launch_t<D_, B_, true>(a, g, V, vt, k_mean, v_sum, kbar, vbart, stream)      \
                : launch_t<D_, B_, false>(a, g, V, vt, k_mean, v_sum, kbar, vbart, stream)
    if (g.d == 128) {
        if (g.block == 128) SA_LAUNCH(128, 128);
        SA_LAUNCH(128, 64);
    }
    if (g.block == 128) SA_LAUNCH(64, 128);
    SA_LAUNCH(64, 64);
#undef SA_LAUNCH
}

}  // namespace sa
