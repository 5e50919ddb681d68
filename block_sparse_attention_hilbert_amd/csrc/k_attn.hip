// Block-sparse attention forward for gfx950 (SVG-EAR page, section 2B:
// streaming softmax update over the computed blocks without materialising the
// logits; SPADE page, part 3: a head-wise sparse attention kernel).  With
// compensation, every skipped KV block contributes one centroid pseudo-token
// (SVG-EAR page, section 2A): key = block mean of K, value = block mean of V,
// weight = the block's token count (a logit bias of log n_j).
//
// Mapping onto CDNA4
//   * one workgroup = one (batch, head, query block).  Wave (qg, kh) owns 32
//     queries (query group qg) and one half of the keys of every KV tile (kh);
//     the two key halves are merged once at the end, like two KV splits.  A
//     wave stays under 256 registers, so two waves share every SIMD.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: Q^T (B operand) stays in
//     registers for the whole row, K (A operand) is read from LDS.  In the
//     32x32 accumulator layout a lane holds one query column, so the softmax
//     statistics are lane-local; the two lane halves sharing a query exchange
//     their maximum once per tile (v_permlane32_swap).
//   * O^T = V^T P^T on the same instruction: P goes from the S^T accumulators
//     into the B operand.  K rows are read in an order that swaps bits 2 and 3
//     of the row index, which makes the 8 probabilities a lane holds per
//     k-step 8 consecutive keys; V is pre-transposed per block in HBM (a cheap
//     bandwidth-bound pass) so those 8 keys are one 16-byte LDS read.
//   * software pipeline of two phases per tile: a matrix phase (P_t V_t and
//     S_{t+1} = K_{t+1} Q^T, interleaved) and a vector phase (softmax of
//     S_{t+1}).  With 8 waves, waves w and w + 4 share a SIMD; the second four
//     run one phase behind the first four (one extra barrier at the start), so
//     on every SIMD one wave's matrix phase overlaps the other's vector phase
//     and the barriers keep the two in alternation.
//   * K and V^T tiles move HBM -> LDS with global_load_lds_dwordx4 (no
//     register staging) into two K slots and two V slots: the copies of K_{t+2}
//     and V_{t+1} are in flight while P_t V_t and S_{t+1} are computed.  Tiles
//     use an XOR swizzle of their 16-byte chunks so that the row-strided
//     operand reads are bank-conflict free.
//   * online softmax in the log2 domain with lazy rescaling: the running
//     maximum only moves (and O, l are only rescaled) when a tile raises it by
//     more than 2^8.
//   * persistent grid with per-XCD row ranges (see k_bsattn_fwd).
#include <math.h>

#include <type_traits>

#include "sa_internal.h"

namespace sa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLazy = 8.0f;      // log2 headroom before the running max moves
#ifndef SA_PF
#define SA_PF 5                    // LDS operand reads in flight in the matrix phase
#endif
#ifndef SA_SGB
#define SA_SGB 1
#endif
#ifndef SA_VPRIO
#define SA_VPRIO 1                 // wave priority of the vector phase (4-wave workgroups)
#endif

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

// Workgroup barrier without a memory fence: LDS operands are consumed (waited
// for) inside the phase that reads them, and the tile copies are completed
// with explicit vmcnt waits, so the fence's waits would only stall the copies
// in flight.  The memory clobber keeps the compiler from moving LDS accesses
// across it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }
// The scheduling fence keeps the compiler from hoisting the wait above the
// vector work before it (which touches no memory): the copies in flight then
// land while the softmax runs instead of stalling it.
__device__ __forceinline__ void copies_done() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// int32 entries of the scheduling header before the row list
constexpr int kSchedHead = 32;

struct FwdArgs {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* Vt;      // [BH][nb][D][BLK] transposed V blocks (zero-padded keys)
    const int32_t* row_ptr;
    const int32_t* col_idx;
    const uint16_t* kbar;    // [BH][nb][D] centroid keys (compensation) or null
    const uint16_t* vbart;   // [BH][ntc][D][BLK] transposed centroid values
    const int16_t* cnt;      // [BH][nb] tokens of each KV block
    uint16_t* O;
    float* lse;
    const int32_t* order;    // token order of the blocks ([N]) or null: Q, O, lse rows go
                             // through it (K comes already in block order)
    int32_t* sched;          // [0..7] / [8..15] start / end of each range's part of the
                             // row list, [16..23] pull counters;
                             // [24] = 1 when the block counts come from the caller;
                             // [25] workgroups of the launch that are done;
                             // [kSchedHead ..) the rows, longest first
    int32_t N, nb, ntc;
    int64_t rows;
    float c;                 // scale * log2(e)
    // row-map kernels only (MAP): order is a per-head map [BH][N] from the rows
    // of the block layout to the tokens of Q, O and lse (a negative entry: no
    // token, the row is skipped), qmap_stride = N, qN tokens per head of Q, O, lse
    int64_t qmap_stride;
    int32_t qN;
};

template <int D, int BLK>
struct Cfg {
    static constexpr int NWQ = BLK / 32;            // query groups of 32 queries
    static constexpr int NW = NWQ * 2;              // x 2 key halves
    static constexpr int NT = NW * 64;
    // 8 waves: two phase groups of 4 (one wave of each per SIMD); the first
    // group issues all tile copies.  4 waves (64-token blocks): one group, and
    // two workgroups share a CU.
    static constexpr bool PING = NW == 8;
    static constexpr int NWI = PING ? NW / 2 : NW;  // waves issuing copies
    static constexpr int KH = BLK / 2;              // keys per half
    static constexpr int KTW = KH / 32;             // 32-key MFMA tiles per wave
    static constexpr int KRB = D * 2;               // bytes per K row
    static constexpr int VRB = BLK * 2;             // bytes per V^T row
    static constexpr int KCH = KRB / 16;            // 16-byte chunks per K row
    static constexpr int VCH = VRB / 16;
    static constexpr int K_BYTES = BLK * KRB;
    static constexpr int V_BYTES = D * VRB;
    static constexpr int KI = K_BYTES / (1024 * NWI);   // copy instructions per issuing wave
    static constexpr int VI = V_BYTES / (1024 * NWI);
    static constexpr int NSTEP = KTW * D / 16;      // MFMAs of each product per tile
    static constexpr int SLOTS = 2 * K_BYTES + 2 * V_BYTES;
    static constexpr int MERGE = NWQ * ((D / 32) * 64 * 16 * 4 + 2 * 64 * 4);
    static constexpr int BASE = SLOTS > MERGE ? SLOTS : MERGE;
    static constexpr int MAX_NB = 4096;                 // list / flag capacity
    static_assert(KI * 1024 * NWI == K_BYTES && VI * 1024 * NWI == V_BYTES, "whole wave slices");
    static_assert(NSTEP == (D / 32) * KTW * 2, "both products take the same number of steps");
};

// Byte offset, inside a tile of rows of RB bytes, of the 16-byte chunk that lane
// `lane` of issuing wave `wi` fetches with copy instruction n.  The tile's
// 16-byte chunks are XOR-swizzled by the row index; every wave instruction
// fills 1 KB of LDS, lane L landing at byte L*16 of the wave's slice.  Rows
// above max_row are clamped to it.
template <int RB, int NWI>
__device__ __forceinline__ uint32_t dma_src_offset(int n, int wi, int lane, int max_row) {
    constexpr int CH = RB / 16;
    const int lin = (n * NWI + wi) * 1024 + lane * 16;
    const int row = lin / RB;
    const int chunk = ((lin % RB) / 16) ^ (row & (CH - 1));
    return (uint32_t)((row < max_row ? row : max_row) * RB + chunk * 16);
}

// HBM -> LDS copy of one tile: global_load_lds_dwordx4 per wave instruction,
// source = base (uniform, SGPRs) + this lane's offset, destination = the wave's
// 1 KB slice.  Issued through inline assembly so that the compiler does not
// treat every later LDS read as dependent on these copies (it cannot tell the
// slots apart and would wait for all of them); completion is ordered
// explicitly by copies_done() + a barrier.  The instruction has no register
// results; M0 carries the LDS address and is restored afterwards.
template <int RB, int INSTR, int NWI>
__device__ __forceinline__ void dma_tile(unsigned char* tile, const unsigned char* base, int max_row,
                                         int wi, int lane) {
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_void_t*)tile;
    // the base is wave-uniform by construction; say so, so that it sits in SGPRs
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const unsigned char* sbase = reinterpret_cast<const unsigned char*>((uintptr_t)ub);
#pragma unroll
    for (int n = 0; n < INSTR; ++n) {
        const uint32_t dst = __builtin_amdgcn_readfirstlane(lds0 + (n * NWI + wi) * 1024);
        uint32_t saved;
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %2, %3\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(dst), "v"(dma_src_offset<RB, NWI>(n, wi, lane, max_row)), "s"(sbase)
            : "memory");
    }
}

// The same copy for a tile whose rows are all in range: lane offsets of copy
// instruction n are off0 + n NWI 1 KB (the swizzle of a row depends on the row
// modulo the chunks per row, which a step of NWI KB does not change), and M0
// advances by NWI KB per instruction.  Two instructions per assembly block;
// every M0 value is formed outside the assembly (SALU arithmetic inside it
// would change SCC behind the compiler's back).
template <int INSTR, int NWI>
__device__ __forceinline__ void dma_tile_fast(unsigned char* tile, const unsigned char* base,
                                              uint32_t off0, int wi) {
    static_assert(INSTR % 2 == 0, "an even number of copy instructions per wave and tile");
    constexpr uint32_t STRIDE = NWI * 1024;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void_t*)tile + (uint32_t)wi * 1024u);
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t ub = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const unsigned char* sbase = reinterpret_cast<const unsigned char*>((uintptr_t)ub);
#pragma unroll
    for (int n = 0; n < INSTR; n += 2) {
        const uint32_t d0 = __builtin_amdgcn_readfirstlane(dst + n * STRIDE);
        const uint32_t d1 = __builtin_amdgcn_readfirstlane(dst + (n + 1) * STRIDE);
        uint32_t saved;
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %1\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %3, %5\n\t"
            "s_mov_b32 m0, %2\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %4, %5\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "s"(d0), "s"(d1), "v"(off0 + n * STRIDE), "v"(off0 + (n + 1) * STRIDE), "s"(sbase)
            : "memory");
    }
}

// One row = one (batch, head, query block): all its kept tiles, then (with
// compensation) the centroid tiles, then the merge of the two key halves.
template <int D, int BLK, bool COMP, bool MAP>
__device__ __forceinline__ void process_row(const FwdArgs& a, int64_t row, unsigned char* smem,
                                            bool var_cnt) {
    using C = Cfg<D, BLK>;
    using yes = std::true_type;
    using no = std::false_type;
    unsigned char* kslot = smem;                                       // 2 K tiles
    unsigned char* vslot = smem + 2 * C::K_BYTES;                      // 2 V^T tiles
    // COMP: [nb] centroid weight of each block: its token count when skipped,
    // 0 when kept or empty
    unsigned char* cw = smem + C::BASE;
    int16_t* list = reinterpret_cast<int16_t*>(smem + C::BASE + C::MAX_NB);  // kept blocks
    int16_t* lcnt = list + a.nb;                                       // their token counts
    // COMP: key bias of a centroid of n tokens, log2(n) / c (-inf for n = 0)
    const float* lut = reinterpret_cast<const float*>(lcnt + a.nb);

    const int i = (int)(row % a.nb);
    const int64_t bh = row / a.nb;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qg = wave >> 1, kh = wave & 1;
    const bool issuer = wave < C::NWI;
    const bool lagging = C::PING && wave >= C::NWI;
    const int r32 = lane & 31, h = lane >> 5;
    const int64_t head_off = bh * (int64_t)a.N * D;           // K (block layout)
    const int64_t q_head_off = MAP ? bh * (int64_t)a.qN * D : head_off;   // Q, O (token layout)
    const unsigned char* Kh = reinterpret_cast<const unsigned char*>(a.K + head_off);
    const unsigned char* Vth =
        reinterpret_cast<const unsigned char*>(a.Vt + bh * (int64_t)a.nb * D * BLK);
    const int last_n = a.N - (a.nb - 1) * BLK;

    // Q^T fragments (B operand) of this wave's 32 queries; query qn of the
    // block order is token qtok of the caller's order
    bf16x8 qf[D / 16];
    const int qn = i * BLK + qg * 32 + r32;
    // (through a per-head map, a row with no token is skipped: zero queries,
    // nothing stored)
    int qtok = 0;
    bool qvalid = qn < a.N;
    if constexpr (MAP) {
        const int t = qvalid ? a.order[bh * a.qmap_stride + qn] : -1;
        qvalid = t >= 0;
        qtok = qvalid ? clamp_token(t, a.qN) : 0;
    } else {
        qtok = qvalid ? (a.order ? clamp_token(a.order[qn], a.N) : qn) : 0;
    }
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (qvalid) v = *reinterpret_cast<const uint4*>(a.Q + q_head_off + (int64_t)qtok * D + st * 16 + h * 8);
        qf[st] = as_bf16x8(v);
    }

    // a row longer than nb (a malformed CSR) is cut to its first nb entries and
    // a negative length taken as empty: the LDS lists below hold nb entries
    const int beg = __builtin_amdgcn_readfirstlane(a.row_ptr[row]);
    const int nk = min(max(__builtin_amdgcn_readfirstlane(a.row_ptr[row + 1]) - beg, 0), a.nb);
    const int T = nk + (COMP ? a.ntc : 0);
    const int16_t* cnt_h = a.cnt + bh * a.nb;
    // token count of block j: the caller's (var_cnt) or the fixed layout's
    auto count_of = [&](int j) -> int {
        return var_cnt ? (int)cnt_h[j] : (j == a.nb - 1 ? last_n : BLK);
    };
    // the row's kept blocks (clamped into range) with their token counts and,
    // for compensation, the centroid weights
    if constexpr (COMP)
        for (int j = tid; j < a.nb; j += C::NT) cw[j] = (unsigned char)count_of(j);
    for (int e = tid; e < nk; e += C::NT) {
        int j = a.col_idx[beg + e];
        j = j < 0 ? 0 : (j >= a.nb ? a.nb - 1 : j);
        list[e] = (int16_t)j;
        if (var_cnt) lcnt[e] = cnt_h[j];
    }
    __syncthreads();
    if constexpr (COMP) {
        for (int e = tid; e < nk; e += C::NT) cw[list[e]] = 0;
        __syncthreads();
    }

    // copies of tile u (kept block list[u], or centroid tile u - nk) into slot b
    // Copies of tile u (kept block j = list[u], read by the caller ahead of
    // time, or centroid tile u - nk) into slot b.  Tiles whose rows are all in
    // range take the fast path with this lane's precomputed offsets; a short
    // last block or centroid tile has its rows clamped (finite, masked by the
    // bias).
    const uint32_t koff0 = dma_src_offset<C::KRB, C::NWI>(0, wave, lane, BLK - 1);
    const uint32_t voff0 = dma_src_offset<C::VRB, C::NWI>(0, wave, lane, D - 1);
    auto issue_k = [&](int u, int b, int j) {
        unsigned char* dst = kslot + b * C::K_BYTES;
        if (!COMP || u < nk) {
            const unsigned char* src = Kh + (int64_t)j * BLK * C::KRB;
            if (j == a.nb - 1 && last_n < BLK)
                dma_tile<C::KRB, C::KI, C::NWI>(dst, src, last_n - 1, wave, lane);
            else
                dma_tile_fast<C::KI, C::NWI>(dst, src, koff0, wave);
        } else {
            const int j0 = (u - nk) * BLK;
            const int nval = a.nb - j0 < BLK ? a.nb - j0 : BLK;
            const unsigned char* src =
                reinterpret_cast<const unsigned char*>(a.kbar + (bh * a.nb + j0) * (int64_t)D);
            if (nval < BLK)
                dma_tile<C::KRB, C::KI, C::NWI>(dst, src, nval - 1, wave, lane);
            else
                dma_tile_fast<C::KI, C::NWI>(dst, src, koff0, wave);
        }
    };
    auto issue_v = [&](int u, int b, int j) {
        unsigned char* dst = vslot + b * C::V_BYTES;
        const unsigned char* src;
        if (!COMP || u < nk)
            src = Vth + (int64_t)j * D * C::VRB;
        else
            src = reinterpret_cast<const unsigned char*>(a.vbart + (bh * a.ntc + (u - nk)) * (int64_t)D * BLK);
        dma_tile_fast<C::VI, C::NWI>(dst, src, voff0, wave);
    };
    // list entry u, clamped into the list (entries past it are centroid tiles
    // or past the row: their value is not used)
    auto list_at = [&](int u) -> int { return (int)list[u < nk ? u : (nk > 0 ? nk - 1 : 0)]; };
    // the list index of the short last block of the sequence, if the row keeps it
    const int short_u = !var_cnt && last_n < BLK && nk > 0 &&
                                __builtin_amdgcn_readfirstlane(list_at(nk - 1)) == a.nb - 1
                            ? nk - 1
                            : -1;


    f32x16 oacc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 s[C::KTW];            // S^T of the next tile (matrix phase -> vector phase)
    bf16x8 pb[C::KTW][2];        // P^T of the current tile (vector phase -> matrix phase)

    // Matrix phase of step t: O^T += V_t^T P_t^T (PV) and S^T = K_{t+1} Q^T (S),
    // interleaved so that the accumulator chains alternate.  Operand reads run
    // PF instructions ahead of the matrix-core instructions that consume them.
    auto matrix_phase = [&](auto do_pv, auto do_s, int t) {
        constexpr bool DS = decltype(do_s)::value, DP = decltype(do_pv)::value;
        constexpr int NOP = (DS ? C::NSTEP : 0) + (DP ? C::NSTEP : 0);
        constexpr int PF = SA_PF;
        const unsigned char* Ks = kslot + ((t + 1) & 1) * C::K_BYTES;
        const unsigned char* Vs = vslot + (t & 1) * C::V_BYTES;
        // op k: S step k/2 (even) and PV step k/2 (odd) when both run
        auto is_s = [&](int k) { return DS && (!DP || (k & 1) == 0); };
        auto step = [&](int k) { return DS && DP ? k >> 1 : k; };
        // Operand addresses by XOR.  The slots start 256-byte aligned, so a K
        // row starts KRB-aligned; its 16-byte chunk c sits at position
        // c ^ (row & (KCH - 1)), and the row's low bits are those of
        // swap23(r32) (kh KH + 32 kt is a multiple of KCH).  Chunk 2 st + h of
        // row kh KH + 32 kt + swap23(r32) is therefore at kbase ^ (32 st) +
        // 32 kt KRB, where kbase holds the lane's row and 16 (h ^ (row &
        // (KCH - 1))); the XOR only touches bits below KRB.  V^T row
        // d = 32 dt + r32, key chunk 2 m + h: vbase ^ (32 m) + 32 dt VRB.  One
        // XOR per read and two base registers per phase.
        const uint32_t ks32 = (uint32_t)(uintptr_t)(const lds_void_t*)Ks;
        const uint32_t vs32 = (uint32_t)(uintptr_t)(const lds_void_t*)Vs;
        uint32_t kbase = ks32 + (uint32_t)((kh * C::KH + swap23(r32)) * C::KRB) +
                               16u * (uint32_t)(h ^ (swap23(r32) & (C::KCH - 1)));
        uint32_t vbase = vs32 + (uint32_t)(r32 * C::VRB) + 16u * (uint32_t)(h ^ (r32 & (C::VCH - 1)));
        // opaque to the optimiser: the per-read XORs are formed here, each
        // phase, instead of being hoisted out of the tile loop into registers
        asm volatile("" : "+v"(kbase), "+v"(vbase));
        auto lds16 = [](uint32_t addr) -> bf16x8 {
            typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>((uintptr_t)addr));
        };
        auto load = [&](int k) -> bf16x8 {
            const int u = step(k);
            if (is_s(k)) {
                const int kt = u % C::KTW, st = u / C::KTW;
                return lds16((kbase ^ (32u * st)) + (uint32_t)(kt * 32 * C::KRB));
            }
            const int dt = u % (D / 32), q = u / (D / 32);
            const int kt = q >> 1, s2 = q & 1;
            const int m = (kh * C::KH + kt * 32 + 16 * s2) / 16;      // chunk pair of the 16 keys
            return lds16((vbase ^ (32u * m)) + (uint32_t)(dt * 32 * C::VRB));
        };
        bf16x8 ring[PF];
#pragma unroll
        for (int k = 0; k < PF && k < NOP; ++k) ring[k] = load(k);
#pragma unroll
        for (int k = 0; k < NOP; ++k) {
            const bf16x8 op = ring[k % PF];
            if (k + PF < NOP) ring[k % PF] = load(k + PF);
            const int u = step(k);
            if (is_s(k)) {
                const int kt = u % C::KTW, st = u / C::KTW;
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, qf[st], st == 0 ? f32x16{} : s[kt], 0, 0, 0);
            } else {
                const int dt = u % (D / 32), q = u / (D / 32);
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op, pb[q >> 1][q & 1], oacc[dt], 0, 0, 0);
            }
        }
#if SA_SGB
        // keep the order: PF reads, then (1 read, 1 MFMA) pairs, then the tail
#pragma unroll
        for (int k = 0; k < PF && k < NOP; ++k) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int k = 0; k < NOP; ++k) {
            if (k + PF < NOP) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
#endif
    };

    // Vector phase: online softmax of S^T of tile u into P^T.  A tile with
    // masked or weighted keys (short block: -inf past its token count; centroid
    // tile: log2 n_j, -inf for kept or empty blocks and past nb) adds that key bias,
    // divided by the log2-domain scale c, to the raw scores; the max is taken on
    // raw scores (c > 0), and c s - m is one FMA.
    auto vector_phase = [&](int u) {
        const bool cent = COMP && u >= nk;
        int nval = BLK;
        if (!cent) {
            if (var_cnt)
                nval = __builtin_amdgcn_readfirstlane((int)lcnt[u]);
            else if (u == short_u)
                nval = last_n;
        }
        if (cent || nval < BLK) {
            const int j0 = (u - nk) * BLK;
#pragma unroll
            for (int kt = 0; kt < C::KTW; ++kt)
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = kh * C::KH + kt * 32 + 16 * (g >> 1) + 8 * h + 4 * (g & 1) + e;
                        float b;
                        if (cent) {
                            const int j = j0 + key;
                            b = lut[j < a.nb ? cw[j] : 0];
                        } else {
                            b = key < nval ? 0.f : -INFINITY;
                        }
                        s[kt][4 * g + e] += b;
                    }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < C::KTW; ++kt)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kt][e]);
        mx = xmax32(mx) * a.c;
        if (mx > m_run + kLazy) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) oacc[dt] *= alpha;
            m_run = mx;
        }
        const float nbase = m_run == -INFINITY ? 0.f : -m_run;
        // fp32 row sum in four independent chains (plain adds: the dot-product
        // instructions share the matrix core's issue and stall behind the
        // other wave's matrix instructions)
        float sum4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < C::KTW; ++kt)
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][8 * s2 + e], a.c, nbase));
                    pb[kt][s2][e] = (__bf16)x;
                    sum4[e & 3] += x;
                }
            }
        l_run += (sum4[0] + sum4[1]) + (sum4[2] + sum4[3]);
    };

    // Pipeline over the T tiles.  Step t (t = -1 .. T-1) = matrix phase (P_t V_t,
    // S_{t+1}; the issuing waves start the copies of K_{t+2} and V_{t+1}), then
    // vector phase (softmax of S_{t+1}).  A barrier precedes each phase; the
    // lagging group passes one extra barrier first, the leading one after the
    // last step, so both pass the same number.
    // block indices of the next step's copies, read from LDS one step ahead
    int pre_k = 0, pre_v = 0;
    if (T > 0) {
        if (issuer) issue_k(0, 0, __builtin_amdgcn_readfirstlane(list_at(0)));
        copies_done();
        wg_barrier();
        if (lagging) wg_barrier();
        // step -1: S_0
        wg_barrier();
        if (issuer) {
            if (T > 1) issue_k(1, 1, __builtin_amdgcn_readfirstlane(list_at(1)));
            issue_v(0, 0, __builtin_amdgcn_readfirstlane(list_at(0)));
            pre_k = list_at(2);
            pre_v = list_at(1);
        }
        matrix_phase(no{}, yes{}, -1);
        if (C::PING) wg_barrier();
        vector_phase(0);
        copies_done();
        for (int t = 0; t + 1 < T; ++t) {
            wg_barrier();
            if (issuer) {
                const int jk = __builtin_amdgcn_readfirstlane(pre_k), jv = __builtin_amdgcn_readfirstlane(pre_v);
                if (t + 2 < T) issue_k(t + 2, t & 1, jk);
                issue_v(t + 1, (t + 1) & 1, jv);
                pre_k = list_at(t + 3);
                pre_v = list_at(t + 2);
            }
            matrix_phase(yes{}, yes{}, t);
            if (C::PING) wg_barrier();
            // 4-wave workgroups (64-token blocks) run free beside a second
            // workgroup on the CU: the vector phase takes issue priority over
            // the other workgroup's matrix work on the SIMD, whose queued
            // matrix instructions keep the matrix core busy meanwhile
            if constexpr (!C::PING) __builtin_amdgcn_s_setprio(SA_VPRIO);
            vector_phase(t + 1);
            if constexpr (!C::PING) __builtin_amdgcn_s_setprio(0);
            copies_done();
        }
        // step T-1: P_{T-1} V_{T-1}
        wg_barrier();
        matrix_phase(yes{}, no{}, T - 1);
        if (C::PING) wg_barrier();
        if (C::PING && !lagging) wg_barrier();
    }

    // Merge the two key halves of every query group.  Wave kh finalises the
    // output channel tiles dt in [kh HD, kh HD + HD) and takes the partner's
    // partial sums of those tiles from LDS (the sum of the two scaled halves
    // is the same either way round).  The two lanes of a query (h = 0, 1)
    // then swap halves across the half-wave, so that each lane writes whole
    // 8-channel groups: lane h = 0 the groups 0 and 2 of a tile, h = 1 the
    // groups 1 and 3, one 16-byte store each.
    constexpr int HD = D / 64;
    const float l_tot = xsum32(l_run);
    __syncthreads();                                   // tile slots are free
    unsigned char* mbase = smem + qg * (C::MERGE / C::NWQ);
    float4* mo = reinterpret_cast<float4*>(mbase);     // [wave kh][HD tiles][4 groups][64 lanes]
    float* ml = reinterpret_cast<float*>(mbase + (D / 32) * 64 * 16 * 4);   // [wave kh][m, l][32]
    // (kh is uniform but not a constant: each half is its own code path, so
    // that the accumulator tiles keep constant register indices)
    auto send = [&](auto KHC) {
        constexpr int K = decltype(KHC)::value;
#pragma unroll
        for (int t = 0; t < HD; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                mo[((K * HD + t) * 4 + g) * 64 + lane] =
                    make_float4(oacc[(1 - K) * HD + t][4 * g], oacc[(1 - K) * HD + t][4 * g + 1],
                                oacc[(1 - K) * HD + t][4 * g + 2], oacc[(1 - K) * HD + t][4 * g + 3]);
    };
    if (kh == 0)
        send(std::integral_constant<int, 0>{});
    else
        send(std::integral_constant<int, 1>{});
    if (h == 0) {
        ml[kh * 64 + r32] = m_run;
        ml[kh * 64 + 32 + r32] = l_tot;
    }
    __syncthreads();
    const int ok = 1 - kh;
    const float m1 = ml[ok * 64 + r32], l1 = ml[ok * 64 + 32 + r32];
    const float m = fmaxf(m_run, m1);
    const float mb = m == -INFINITY ? 0.f : m;
    const float a0 = __builtin_amdgcn_exp2f(m_run - mb), a1 = __builtin_amdgcn_exp2f(m1 - mb);
    const float l = kh == 0 ? l_tot * a0 + l1 * a1 : l1 * a1 + l_tot * a0;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    auto finish = [&](auto KHC) {
        constexpr int K = decltype(KHC)::value;
        uint16_t* orow = a.O + q_head_off + (int64_t)qtok * D;
#pragma unroll
        for (int t = 0; t < HD; ++t) {
            constexpr int OK = 1 - K;
            const int dt = K * HD + t;
            uint32_t pk[4][2];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 o1 = mo[((OK * HD + t) * 4 + g) * 64 + lane];
                const float v0 = (oacc[dt][4 * g + 0] * a0 + o1.x * a1) * inv;
                const float v1 = (oacc[dt][4 * g + 1] * a0 + o1.y * a1) * inv;
                const float v2 = (oacc[dt][4 * g + 2] * a0 + o1.z * a1) * inv;
                const float v3 = (oacc[dt][4 * g + 3] * a0 + o1.w * a1) * inv;
                pk[g][0] = f32_to_bf16_rne(v0) | ((uint32_t)f32_to_bf16_rne(v1) << 16);
                pk[g][1] = f32_to_bf16_rne(v2) | ((uint32_t)f32_to_bf16_rne(v3) << 16);
            }
#pragma unroll
            for (int g0 = 0; g0 < 4; g0 += 2) {
                // lanes 0-31 keep group g0 and receive the partner's part of
                // it; lanes 32-63 keep group g0 + 1 likewise
                uint32_t w[4];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const auto r = __builtin_amdgcn_permlane32_swap(pk[g0][e], pk[g0 + 1][e], false, false);
                    if (h == 0) {
                        w[e] = pk[g0][e];           // channels 8 g0 + 0..3 (own)
                        w[2 + e] = r[1];            // channels 8 g0 + 4..7 (partner's)
                    } else {
                        w[e] = r[0];                // channels 8 (g0+1) + 0..3 (partner's)
                        w[2 + e] = pk[g0 + 1][e];   // channels 8 (g0+1) + 4..7 (own)
                    }
                }
                *reinterpret_cast<uint4*>(orow + dt * 32 + 8 * (g0 + h)) = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
    };
    if (qvalid) {
        if (kh == 0)
            finish(std::integral_constant<int, 0>{});
        else
            finish(std::integral_constant<int, 1>{});
        if (a.lse && kh == 0 && h == 0)
            a.lse[bh * (int64_t)(MAP ? a.qN : a.N) + qtok] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
    }
}

// Persistent grid.  k_sched splits the rows into 8 contiguous ranges of equal
// work and lists each range's rows long ones first (by length class, in row
// order within a class); workgroup w pulls rows of range w % 8 -- the XCD it
// is dealt to -- in that order, so concurrently running rows of one XCD are
// mostly neighbouring query blocks that share K/V blocks in that XCD's L2,
// and the last rows handed out are short ones.  A workgroup whose range is
// exhausted takes rows from the other ranges.  Which workgroup runs a row
// does not change its result.
template <int D, int BLK, bool COMP, bool MAP>
__global__ __launch_bounds__(BLK * 4) __attribute__((amdgpu_waves_per_eu(2)))
void k_bsattn_fwd(FwdArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    // the tile slots start 256-byte aligned: operand addresses are formed by XOR
    unsigned char* smem = smem_raw + ((256u - ((uint32_t)(uintptr_t)(lds_void_t*)smem_raw & 255u)) & 255u);
    __shared__ int s_row;
    // block token counts from the caller (else the fixed layout's)
    const bool var_cnt = __builtin_amdgcn_readfirstlane(a.sched[24]) != 0;
    if constexpr (COMP) {
        // key bias of a centroid by its token count (log2 domain, divided by c)
        using C = Cfg<D, BLK>;
        float* lut = reinterpret_cast<float*>(smem + C::BASE + C::MAX_NB + 4 * a.nb);
        const float inv_c = 1.f / a.c;
        for (int n = threadIdx.x; n <= BLK; n += C::NT) lut[n] = n ? __log2f((float)n) * inv_c : -INFINITY;
        __syncthreads();
    }
    const int x0 = blockIdx.x % 8;
    for (int k = 0; k < 8; ++k) {
        const int x = (x0 + k) % 8;
        const int start = a.sched[x], stop = a.sched[8 + x];   // list positions of range x
        for (;;) {
            if (threadIdx.x == 0) {
                const int idx = start < stop ? atomicAdd(&a.sched[16 + x], 1) : 0;
                s_row = start + idx < stop ? a.sched[kSchedHead + start + idx] : -1;
            }
            __syncthreads();
            const int row = s_row;
            __syncthreads();
            if (row < 0) break;
            process_row<D, BLK, COMP, MAP>(a, row, smem, var_cnt);
        }
    }
    // The last workgroup to finish re-arms the pull counters for the next
    // launch: every other workgroup has made its last pull before counting
    // itself done.
    if (threadIdx.x == 0) {
        __threadfence();
        if (atomicAdd(&a.sched[25], 1) == (int)gridDim.x - 1) {
            for (int x = 0; x < 8; ++x) a.sched[16 + x] = 0;
            a.sched[25] = 0;
        }
    }
}

constexpr int kSchedThreads = 1024;
constexpr int kSchedItems = 8;
constexpr int kSchedCls = 9;                    // length classes
constexpr int kSchedSlots = 256;                // 128-token rows running at once (one per CU)

// The row list of the persistent grid.  The rows are split into 8 contiguous
// ranges of (nearly) equal work, a row costing its tiles (kept blocks clamped
// to [0, nb], the attention kernel's own clamp) plus a fixed overhead.  Inside
// a range the rows are listed by length class, longest first -- class
// min(8, floor(4 len / mean len)) -- and in row order within a class, so rows
// of equal length keep their order (neighbouring query blocks run together
// and share K/V blocks in the XCD's L2) while long rows do not start last.
// Class k = min(8, floor(len / w)) with w = max(mean len / 2, 1/32 of the work
// per concurrently running workgroup (`slots` of them)): where every row is
// short against that share (many rows per workgroup) there is one class and
// the rows keep their order.  One workgroup.
__global__ __launch_bounds__(kSchedThreads) void k_sched(const int32_t* __restrict__ row_ptr,
                                                         int32_t* __restrict__ sched, int64_t R,
                                                         int nb, int extra, int slots,
                                                         int cnt_flag) {
    __shared__ long long wsum[kSchedThreads / 64];
    __shared__ long long s_total, s_carry;
    __shared__ int s_bound[9];
    __shared__ int s_cnt[8][kSchedCls];          // rows per (range, class)
    __shared__ int s_off[8][kSchedCls];          // list position of a class's first row, less
                                                 // that class's rows in earlier ranges
    __shared__ int s_wcnt[kSchedThreads / 64][kSchedCls];
    __shared__ int s_seen[kSchedCls];            // rows per class in earlier chunks
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    auto len = [&](int64_t r) -> int {
        const int n = row_ptr[r + 1] - row_ptr[r];
        return n < 0 ? 0 : (n > nb ? nb : n);
    };
    auto cost = [&](int64_t r) -> long long { return (long long)len(r) + extra; };
    // total work
    long long part = 0;
    for (int64_t r = tid; r < R; r += kSchedThreads) part += cost(r);
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
    if (lane == 0) wsum[wid] = part;
    if (tid < 8) { sched[16 + tid] = 0; }
    if (tid < 9) s_bound[tid] = (int)R;
    if (tid < 8 * kSchedCls) s_cnt[tid / kSchedCls][tid % kSchedCls] = 0;
    if (tid < kSchedCls) s_seen[tid] = 0;
    if (tid == 0) { sched[24] = cnt_flag; sched[25] = 0; }
    __syncthreads();
    if (tid == 0) {
        long long t = 0;
        for (int k = 0; k < kSchedThreads / 64; ++k) t += wsum[k];
        s_total = t;
        s_carry = 0;
        s_bound[0] = 0;
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
                    if (run * 8 <= tgt && tgt < (run + c[k]) * 8) s_bound[x] = (int)(my + k);
                }
            }
            run += c[k];
        }
        __syncthreads();
        if (tid == kSchedThreads - 1) s_carry = run;
        __syncthreads();
    }
    // a boundary no row interval contains (costs of 0 cannot occur: extra >= 1)
    // stays at R; boundaries are non-decreasing
    if (tid < 8) {
        sched[tid] = s_bound[tid];
        sched[8 + tid] = s_bound[tid + 1];
    }
    // len / w = len min(2 R, 32 slots) / (sum of the lengths)
    const long long sumlen = total - (long long)R * extra;
    const long long per = 2 * R < 32LL * slots ? 2 * R : 32LL * slots;
    auto cls = [&](int64_t r) -> int {
        if (sumlen <= 0) return 0;
        const long long k = (long long)len(r) * per / sumlen;
        return k < kSchedCls - 1 ? (int)k : kSchedCls - 1;
    };
    auto range_of = [&](int64_t r) -> int {
        int x = 0;
        for (int y = 1; y < 8; ++y) x += r >= s_bound[y] ? 1 : 0;
        return x;
    };
    for (int64_t r = tid; r < R; r += kSchedThreads) atomicAdd(&s_cnt[range_of(r)][cls(r)], 1);
    __syncthreads();
    if (tid < 8 * kSchedCls) {
        const int x = tid / kSchedCls, k = tid % kSchedCls;
        int o = s_bound[x];
        for (int q = k + 1; q < kSchedCls; ++q) o += s_cnt[x][q];
        for (int y = 0; y < x; ++y) o -= s_cnt[y][k];
        s_off[x][k] = o;
    }
    __syncthreads();
    // stable scatter, 1024 rows a round: a row's place among the rows of its
    // class before it = ballot rank in its wave + earlier waves + earlier rounds
    int32_t* list = sched + kSchedHead;
    const unsigned long long below = (1ull << lane) - 1ull;
    for (int64_t c0 = 0; c0 < R; c0 += kSchedThreads) {
        const int64_t r = c0 + tid;
        const int k = r < R ? cls(r) : -1;
        int rank = 0;
#pragma unroll
        for (int q = 0; q < kSchedCls; ++q) {
            const unsigned long long m = __ballot(k == q);
            if (k == q) rank = __popcll(m & below);
            if (lane == 0) s_wcnt[wid][q] = __popcll(m);
        }
        __syncthreads();
        if (k >= 0) {
            int before = s_seen[k] + rank;
            for (int w = 0; w < wid; ++w) before += s_wcnt[w][k];
            list[s_off[range_of(r)][k] + before] = (int32_t)r;
        }
        __syncthreads();
        if (tid < kSchedCls) {
            int t = 0;
            for (int w = 0; w < kSchedThreads / 64; ++w) t += s_wcnt[w][tid];
            s_seen[tid] += t;
        }
        __syncthreads();
    }
}

// V blocks transposed to [D][BLK] (keys past the end of the sequence are 0).
// Each thread moves one 8 x 8 sub-tile (8 keys x 8 channels) through its
// registers: 8 16-byte row loads, a transpose of the bf16 pairs, 8 16-byte
// stores of 8 consecutive keys of one channel.  Consecutive lanes take
// consecutive key groups, so 16 (8) lanes write one whole 256-byte (128-byte)
// row of the transposed block.
// With a per-head map (map_stride = N: order is [BH][N], slot -> token of V,
// negative: no token, a zero row; V holds vN tokens per head) the same for a
// layout whose rows map to the tokens of V.
template <int D, int BLK>
__global__ __launch_bounds__(256) void k_vt_prep(const uint16_t* __restrict__ V,
                                                 uint16_t* __restrict__ Vt, int N, int nb,
                                                 const int32_t* __restrict__ order,
                                                 int64_t map_stride = 0, int vN = 0) {
    constexpr int KC = BLK / 8, DC = D / 8;
    const int j = blockIdx.x;
    const int64_t bh = blockIdx.y;
    const int n = min(BLK, N - j * BLK);
    const int NV = map_stride ? vN : N;       // tokens per head of V
    const uint16_t* src = V + bh * NV * (int64_t)D;
    uint16_t* dst = Vt + (bh * nb + j) * (int64_t)D * BLK;
    for (int p = threadIdx.x; p < KC * DC; p += 256) {
        const int kc = p % KC, dc = p / KC;
        // key kc*8 + r of the block is token j*BLK + kc*8 + r of the block
        // order (read through the token order when one is given)
        int tok[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int key = kc * 8 + r;
            int t = -1;
            if (key < n) {
                if (map_stride) {
                    t = order[bh * map_stride + j * BLK + key];
                    t = t < 0 ? -1 : clamp_token(t, NV);
                } else {
                    t = order ? clamp_token(order[j * BLK + key], N) : j * BLK + key;
                }
            }
            tok[r] = t;
        }
        uint32_t w[8][4];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (tok[r] >= 0) v = *reinterpret_cast<const uint4*>(src + (int64_t)tok[r] * D + dc * 8);
            w[r][0] = v.x; w[r][1] = v.y; w[r][2] = v.z; w[r][3] = v.w;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // channel dc*8 + i of keys kc*8 .. kc*8 + 7
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t a = w[2 * q][i / 2], b = w[2 * q + 1][i / 2];
                o[q] = (i & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
            }
            *reinterpret_cast<uint4*>(dst + (int64_t)(dc * 8 + i) * BLK + kc * 8) =
                make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

// Token count of every KV block: the caller's counts (clamped to the block's
// extent) or, without them, BLK and N - (nb - 1) BLK for the last block.
__global__ void k_fill_counts(const int32_t* __restrict__ kv_count, int16_t* __restrict__ cnt,
                              int N, int nb, int blk, int64_t total) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= total) return;
    const int j = (int)(e % nb);
    const int lim = N - j * blk < blk ? N - j * blk : blk;
    int n = lim;
    if (kv_count) {
        n = kv_count[e];
        n = n < 0 ? 0 : (n > lim ? lim : n);
    }
    cnt[e] = (int16_t)n;
}

// Centroid pseudo-tokens for compensation, rounded to bf16 for the matrix
// cores: kbar = k_mean [nb][D]; vbar = v_sum / n_j (0 for an empty block), stored transposed in
// tiles of BLK blocks [ntc][D][BLK] (blocks past nb are 0).  One workgroup per
// run of kCompRun blocks, so that the launch fills the chip.
constexpr int kCompRun = 16;

template <int D, int BLK>
__global__ __launch_bounds__(256) void k_comp_prep(const float* __restrict__ k_mean,
                                                   const float* __restrict__ v_sum,
                                                   const int16_t* __restrict__ cnt,
                                                   uint16_t* __restrict__ kbar,
                                                   uint16_t* __restrict__ vbart, int nb, int ntc) {
    static_assert(BLK % kCompRun == 0, "runs do not straddle centroid tiles");
    const int j0 = blockIdx.x * kCompRun;          // first block of the run
    const int64_t bh = blockIdx.y;
    for (int p = threadIdx.x; p < kCompRun * D; p += 256) {
        const int j = j0 + p / D, d = p % D;
        if (j < nb) {
            const int64_t e = (bh * nb + j) * (int64_t)D + d;
            kbar[e] = f32_to_bf16_rne(k_mean[e]);
        }
    }
    const int tc = j0 / BLK, r0 = j0 % BLK;
    for (int p = threadIdx.x; p < kCompRun * D; p += 256) {
        const int d = p / kCompRun, r = p % kCompRun;
        const int j = j0 + r;
        uint16_t v = 0;
        if (j < nb) {
            const int n = cnt[bh * nb + j];
            if (n > 0) v = f32_to_bf16_rne(v_sum[(bh * nb + j) * (int64_t)D + d] / (float)n);
        }
        vbart[((bh * ntc + tc) * (int64_t)D + d) * BLK + r0 + r] = v;
    }
}

struct WsLayout {
    size_t sched, cnt, vt, kbar, vbart, kord, total;
};

WsLayout ws_layout(const Geometry& g, bool comp) {
    WsLayout L{};
    const int64_t ntc = ceil_div(g.nb, g.block);
    size_t off = 0;
    // V in block layout first: a selection with the error rule can write it
    // there (the caller passes the workspace start)
    L.vt = off; off = align_up(off + (size_t)g.BH() * g.nb * g.d * g.block * 2, 256);
    L.sched = off; off = align_up(off + (kSchedHead + (size_t)g.rows()) * sizeof(int32_t), 256);
    L.cnt = off; off = align_up(off + (size_t)g.BH() * g.nb * sizeof(int16_t), 256);
    if (g.order) {   // K in block order, [BH][N][D]
        L.kord = off; off = align_up(off + (size_t)g.BH() * g.N * g.d * 2, 256);
    }
    if (comp) {
        L.kbar = off; off = align_up(off + (size_t)g.BH() * g.nb * g.d * 2, 256);
        L.vbart = off; off = align_up(off + (size_t)g.BH() * ntc * g.d * g.block * 2, 256);
    }
    L.total = off;
    return L;
}

// Preparation: the block token counts, V re-laid out block by block, the
// centroid tiles with compensation, and the per-XCD row ranges.
template <int D, int BLK, bool COMP>
sa_status prepare_t(const FwdArgs& a, const Geometry& g, const uint16_t* V, uint16_t* vt,
                    const float* k_mean, const float* v_sum, const int32_t* kv_count,
                    uint16_t* kbar, uint16_t* vbart, hipStream_t stream,
                    const int32_t* vmap = nullptr, int vN = 0) {
    // the block counts are read only with the caller's counts or compensation
    sa_status st = SA_OK;
    if (COMP || kv_count) {
        int16_t* cnt = const_cast<int16_t*>(a.cnt);
        const int64_t ncnt = g.BH() * g.nb;
        hipLaunchKernelGGL(k_fill_counts, dim3((unsigned)ceil_div(ncnt, 256)), dim3(256), 0, stream,
                           kv_count, cnt, g.N, g.nb, BLK, ncnt);
        if ((st = hip_check(hipGetLastError(), "k_fill_counts launch")) != SA_OK) return st;
    }
    if (V) {   // else the workspace already holds V in block layout
        if (vmap)
            hipLaunchKernelGGL((k_vt_prep<D, BLK>), dim3(g.nb, (unsigned)g.BH()), dim3(256), 0, stream, V,
                               vt, g.N, g.nb, vmap, (int64_t)g.N, vN);
        else
            hipLaunchKernelGGL((k_vt_prep<D, BLK>), dim3(g.nb, (unsigned)g.BH()), dim3(256), 0, stream, V,
                               vt, g.N, g.nb, g.order, (int64_t)0, 0);
        if ((st = hip_check(hipGetLastError(), "k_vt_prep launch")) != SA_OK) return st;
    }
    if (COMP) {
        hipLaunchKernelGGL((k_comp_prep<D, BLK>), dim3(a.ntc * (BLK / kCompRun), (unsigned)g.BH()),
                           dim3(256), 0, stream, k_mean, v_sum, a.cnt, kbar, vbart, g.nb, a.ntc);
        if ((st = hip_check(hipGetLastError(), "k_comp_prep launch")) != SA_OK) return st;
    }
    if (a.rows == 0) return SA_OK;
    hipLaunchKernelGGL(k_sched, dim3(1), dim3(kSchedThreads), 0, stream, a.row_ptr, a.sched,
                       a.rows, g.nb, (COMP ? a.ntc : 0) + 2, kSchedSlots * (128 / BLK),
                       kv_count != nullptr ? 1 : 0);
    return hip_check(hipGetLastError(), "k_sched launch");
}

// The attention kernel on a persistent grid.
template <int D, int BLK, bool COMP, bool MAP>
sa_status run_t(const FwdArgs& a, const Geometry& g, hipStream_t stream) {
    using C = Cfg<D, BLK>;
    sa_status st = SA_OK;
    const size_t lds = 256 + C::BASE + C::MAX_NB + 4 * (size_t)g.nb + (COMP ? 4 * (BLK + 1) : 0);
    const int most = 256 + C::BASE + C::MAX_NB + 4 * C::MAX_NB + 4 * (BLK + 1);
    st = ensure_max_lds((const void*)k_bsattn_fwd<D, BLK, COMP, MAP>, most, "k_bsattn_fwd shared memory");
    if (st != SA_OK) return st;
    if (a.rows == 0) return SA_OK;
    // as many workgroups as the chip holds at once (LDS per workgroup depends on nb)
    int resident = 0;
    st = resident_workgroups((const void*)k_bsattn_fwd<D, BLK, COMP, MAP>, C::NT, lds, &resident);
    if (st != SA_OK) return st;
    const int64_t grid = a.rows < resident ? a.rows : resident;
    hipLaunchKernelGGL((k_bsattn_fwd<D, BLK, COMP, MAP>), dim3((unsigned)grid), dim3(C::NT), lds, stream, a);
    return hip_check(hipGetLastError(), "k_bsattn_fwd launch");
}

FwdArgs make_args(const Geometry& g, bool comp, const uint16_t* Q, const uint16_t* K,
                  const int32_t* row_ptr, const int32_t* col_idx, uint16_t* O, float* lse, char* ws) {
    const WsLayout L = ws_layout(g, comp);
    FwdArgs a{};
    a.Q = Q; a.K = g.order ? reinterpret_cast<const uint16_t*>(ws + L.kord) : K;
    a.order = g.order;
    a.row_ptr = row_ptr; a.col_idx = col_idx;
    a.O = O; a.lse = lse; a.N = g.N; a.nb = g.nb; a.rows = g.rows();
    a.qmap_stride = 0;
    a.qN = g.N;
    a.ntc = (int32_t)ceil_div(g.nb, g.block);
    a.c = g.scale * kLog2e;
    a.Vt = reinterpret_cast<uint16_t*>(ws + L.vt);
    a.kbar = comp ? reinterpret_cast<uint16_t*>(ws + L.kbar) : nullptr;
    a.vbart = comp ? reinterpret_cast<uint16_t*>(ws + L.vbart) : nullptr;
    a.sched = reinterpret_cast<int32_t*>(ws + L.sched);
    a.cnt = reinterpret_cast<int16_t*>(ws + L.cnt);
    return a;
}

}  // namespace

size_t fwd_workspace_bytes(const Geometry& g, bool comp) { return ws_layout(g, comp).total; }

#define SA_DISPATCH(CALL)                                   \
    if (g.d == 128) {                                       \
        if (g.block == 128) {                               \
            if (comp) return CALL(128, 128, true);          \
            return CALL(128, 128, false);                   \
        }                                                   \
        if (comp) return CALL(128, 64, true);               \
        return CALL(128, 64, false);                        \
    }                                                       \
    if (g.block == 128) {                                   \
        if (comp) return CALL(64, 128, true);               \
        return CALL(64, 128, false);                        \
    }                                                       \
    if (comp) return CALL(64, 64, true);                    \
    return CALL(64, 64, false);

sa_status launch_vt_layout(const Geometry& g, const uint16_t* V, uint16_t* Vt, hipStream_t stream) {
    const dim3 grid(g.nb, (unsigned)g.BH());
    const int32_t* o = g.order;
    if (g.d == 128) {
        if (g.block == 128) hipLaunchKernelGGL((k_vt_prep<128, 128>), grid, dim3(256), 0, stream, V, Vt, g.N, g.nb, o);
        else hipLaunchKernelGGL((k_vt_prep<128, 64>), grid, dim3(256), 0, stream, V, Vt, g.N, g.nb, o);
    } else {
        if (g.block == 128) hipLaunchKernelGGL((k_vt_prep<64, 128>), grid, dim3(256), 0, stream, V, Vt, g.N, g.nb, o);
        else hipLaunchKernelGGL((k_vt_prep<64, 64>), grid, dim3(256), 0, stream, V, Vt, g.N, g.nb, o);
    }
    return hip_check(hipGetLastError(), "k_vt_prep launch");
}

sa_status launch_fwd_prepare(const Geometry& g, const uint16_t* V, const int32_t* row_ptr,
                             const float* k_mean, const float* v_sum, const int32_t* kv_count,
                             char* ws, hipStream_t stream, const int32_t* vmap, int vN) {
    const bool comp = k_mean != nullptr;
    if (vmap && g.order) return fail(SA_ERR_UNSUPPORTED, "a row map and a token order do not combine");
    if (g.nb > 4096) return fail(SA_ERR_UNSUPPORTED, "attention supports nb <= 4096 (got %d)", g.nb);
    const FwdArgs a = make_args(g, comp, nullptr, nullptr, row_ptr, nullptr, nullptr, nullptr, ws);
    uint16_t* vt = const_cast<uint16_t*>(a.Vt);
    uint16_t* kbar = const_cast<uint16_t*>(a.kbar);
    uint16_t* vbart = const_cast<uint16_t*>(a.vbart);
#define SA_PREP(D_, B_, C_) prepare_t<D_, B_, C_>(a, g, V, vt, k_mean, v_sum, kv_count, kbar, vbart, stream, vmap, vN)
    SA_DISPATCH(SA_PREP)
#undef SA_PREP
}

sa_status launch_fwd_run_mapped(const Geometry& g, bool comp, const uint16_t* Q, const uint16_t* K,
                                const int32_t* row_ptr, const int32_t* col_idx,
                                const int32_t* qmap, int32_t qN, uint16_t* O, float* lse, char* ws,
                                hipStream_t stream) {
    if (g.nb > 4096) return fail(SA_ERR_UNSUPPORTED, "attention supports nb <= 4096 (got %d)", g.nb);
    if (g.order) return fail(SA_ERR_UNSUPPORTED, "a row map and a token order do not combine");
    FwdArgs a = make_args(g, comp, Q, K, row_ptr, col_idx, O, lse, ws);
    a.order = qmap;
    a.qmap_stride = g.N;
    a.qN = qN;
#define SA_RUN(D_, B_, C_) run_t<D_, B_, C_, true>(a, g, stream)
    SA_DISPATCH(SA_RUN)
#undef SA_RUN
}

sa_status launch_fwd_run(const Geometry& g, bool comp, const uint16_t* Q, const uint16_t* K,
                         const int32_t* row_ptr, const int32_t* col_idx, uint16_t* O, float* lse,
                         char* ws, hipStream_t stream) {
    if (g.nb > 4096) return fail(SA_ERR_UNSUPPORTED, "attention supports nb <= 4096 (got %d)", g.nb);
    const FwdArgs a = make_args(g, comp, Q, K, row_ptr, col_idx, O, lse, ws);
    if (g.order) {
        // the tile copies read whole blocks: K gathered into block order first
        const sa_status st = launch_permute(g, K, const_cast<uint16_t*>(a.K), g.order, false, stream);
        if (st != SA_OK) return st;
    }
#define SA_RUN(D_, B_, C_) run_t<D_, B_, C_, false>(a, g, stream)
    SA_DISPATCH(SA_RUN)
#undef SA_RUN
}
#undef SA_DISPATCH

}  // namespace sa
