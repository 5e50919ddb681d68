// Internal declarations shared by the host API and the kernel launchers of
// libsparse_attn.so.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sparse_attn.h"

namespace sa {

// Records a failure message for sparse_attn_last_error() and returns `st`.
sa_status fail(sa_status st, const char* fmt, ...);

// Checks a HIP call / the last launch and converts a failure to SA_ERR_HIP.
sa_status hip_check(hipError_t e, const char* what);

// Clears the calling thread's error message (every entry point starts so).
void clear_error();

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A token index read from a caller's token order, clamped into [0, n): an
// order that is not a permutation gives wrong rows, never an access outside
// the tensors.
__host__ __device__ inline int clamp_token(int t, int n) { return t < 0 ? 0 : (t >= n ? n - 1 : t); }

// Launch set-up kept per device, safe to call from several host threads:
// raises a kernel's dynamic-LDS limit to at least `bytes` on the current
// device (one HIP call per kernel and device, repeated only for a larger
// size), and the number of workgroups of `threads` threads and `lds` bytes
// the current device holds at once (one occupancy query per kernel, device
// and size).  These are the library's only host-side state.
sa_status ensure_max_lds(const void* fn, int bytes, const char* what);
sa_status resident_workgroups(const void* fn, int threads, size_t lds, int* out);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Geometry derived from a validated sa_problem.
struct Geometry {
    int32_t B, H, N, d, block, nb;
    int32_t T, Hg, W;
    float scale;
    const int32_t* order;    // device [N] token order of the blocks, or null (as given)
    int64_t BH() const { return (int64_t)B * H; }
    int64_t rows() const { return BH() * nb; }
};

// ----------------------------------------------------------------------------
// selection (k_select.hip)
// ----------------------------------------------------------------------------
struct SelectPlan {
    int32_t rule;            // SA_RULE_*
    int32_t unit;            // tokens per pooled unit: sub_block or block
    int32_t n_units;         // ceil(N / unit)
    int32_t spb;             // units per block
    int32_t nb_pad;          // sort length: next power of two >= nb
    int32_t words;           // bitmap words per row: ceil(nb / 32)
    float mass;
    int32_t diag, window_frames, n_anchors;
    int64_t anchor_offset;
    int32_t want_comp;
    // workspace carve-up (byte offsets); the error rule adds V re-laid out
    // per block and its routing keys
    size_t off_qm, off_km, off_scores, off_bits, off_counts, off_k, off_vt, off_keys, total;
    uint16_t* v_blocks;      // the caller's destination of the V layout (error rule), or null
};

SelectPlan make_select_plan(const Geometry& g, const sa_select_spec& s);

// Host-side validation shared by the entry points (sa_api.cpp): the problem
// statement (fills the geometry), the selection spec, and the pointers of a
// selection call (everything but its workspace).
sa_status check_problem(const sa_problem* p, Geometry* g);
sa_status check_spec(const Geometry& g, const sa_select_spec* s);
sa_status check_select_args(const Geometry& g, const sa_select_spec* spec, const void* Q,
                            const void* K, const void* V, const int32_t* row_ptr,
                            const int32_t* col_idx, const float* k_mean, const float* v_sum);
// A validated selection on a workspace of at least plan.total bytes: the
// per-head budgets resolved on the host, then the selection kernels.
sa_status select_on_workspace(const Geometry& g, const sa_select_spec& spec, const SelectPlan& plan,
                              const void* Q, const void* K, const void* V, int32_t* row_ptr,
                              int32_t* col_idx, float* scores, float* k_mean, float* v_sum,
                              char* ws, hipStream_t stream);

sa_status launch_select(const Geometry& g, const SelectPlan& p,
                        const int32_t* k_host, const uint16_t* Q,
                        const uint16_t* K, const uint16_t* V, int32_t* row_ptr,
                        int32_t* col_idx, float* scores, float* k_mean,
                        float* v_sum, char* ws, hipStream_t stream);

// Block means of K and block sums of V (the compensation statistics) alone.
sa_status launch_centroids(const Geometry& g, const uint16_t* K, const uint16_t* V, float* k_mean,
                           float* v_sum, hipStream_t stream);

// Pooled scores S[bh][i][j] = fl32(scale * seqfma(qm_i, km_j)) of n x n rows.
sa_status launch_pooled_scores(int d, const float* qm, const float* km, float* S, int n,
                               float scale, int64_t BH, hipStream_t stream);

// Exclusive scan counts[R] -> row_ptr[R+1].
sa_status launch_row_scan(const int32_t* counts, int32_t* row_ptr, int64_t R, hipStream_t stream);

// ----------------------------------------------------------------------------
// data-dependent block formation (k_cluster.hip)
// ----------------------------------------------------------------------------
struct ClusterOut {
    int32_t *q_order, *k_order;       // [BH][nbp*block] token per padded slot, -1 = padding
    int32_t *q_blk, *k_blk;           // [BH][nbp] cluster of each padded block, -1 = none
    int32_t *q_cnt, *k_cnt;           // [BH][nbp] tokens of each padded block
    float *q_cent, *k_cent, *v_cent;  // [BH][C][d] (v_cent optional)
    int32_t *q_count, *k_count;       // [BH][C]
};

struct ClusterSel {
    const float *q_cent, *k_cent, *v_cent;
    const int32_t *k_count, *q_blk, *k_blk, *k_cnt;
    int32_t *row_ptr, *col_idx;
    float *scores, *k_mean, *v_sum;   // scores [BH][C][C] optional; k_mean/v_sum [BH][nbp][d] optional
    int32_t rule, diag;
    float mass;
};

// Blocks of the padded clustered layout: ceil(N / block) + C, or C for tiles
// (one block per tile).
int padded_block_count(const Geometry& g, const sa_cluster_spec& cs);
size_t cluster_workspace_bytes(const Geometry& g, const sa_cluster_spec& cs);
size_t cluster_select_workspace_bytes(const Geometry& g, const sa_cluster_spec& cs);
sa_status launch_cluster(const Geometry& g, const sa_cluster_spec& cs, const uint16_t* Q,
                         const uint16_t* K, const uint16_t* V, const ClusterOut& o, char* ws,
                         hipStream_t stream);
sa_status launch_cluster_gather(const Geometry& g, const sa_cluster_spec& cs, const int32_t* order,
                                const uint16_t* src, uint16_t* dst, hipStream_t stream);
sa_status launch_cluster_scatter(const Geometry& g, const sa_cluster_spec& cs, const int32_t* order,
                                 const uint16_t* src, uint16_t* dst, const float* lse_src,
                                 float* lse_dst, hipStream_t stream);
sa_status launch_cluster_select(const Geometry& g, const sa_cluster_spec& cs, const ClusterSel& a,
                                const int64_t* budget_host, char* ws, hipStream_t stream);
// Key and value means of the clusters from K, V in the padded layout, and the
// per-block compensation statistics (a call that reuses the partition).
sa_status launch_cluster_centroids(const Geometry& g, const sa_cluster_spec& cs, const uint16_t* Kp,
                                   const uint16_t* Vp, const int32_t* k_count,
                                   const int32_t* k_blk, const int32_t* k_cnt, float* k_cent,
                                   float* v_cent, float* k_mean, float* v_sum, hipStream_t stream);

// ----------------------------------------------------------------------------
// SICS scheme generation over shaped tiles (k_tiles.hip)
// ----------------------------------------------------------------------------
// Largest tile count of the menu on the grid.
int menu_max_tiles(const Geometry& g, const sa_cluster_spec& cs);
size_t sics_workspace_bytes(const Geometry& g, const sa_cluster_spec& cs);
// Shape scores (fp64 [BH, n_shapes], optional) and the chosen shape per (b, h).
sa_status launch_sics(const Geometry& g, const sa_cluster_spec& cs, const uint16_t* Q,
                      const uint16_t* K, double* scores, int32_t* shape_idx, char* ws,
                      hipStream_t stream);
// assign[bh][n] = tile of token n under shape cs.shape_idx[bh].
sa_status launch_tile_assign(const Geometry& g, const sa_cluster_spec& cs, int32_t* assign,
                             hipStream_t stream);

// ----------------------------------------------------------------------------
// error-aware routing keys (k_route.hip)
// ----------------------------------------------------------------------------
// keys[(bh*nb + i)*nb + j] for every query block i and KV block j from the
// query block means qm [BH,nb,d], K [BH,N,d], V re-laid out per block
// Vt [BH,nb,d,block], the block sums v_sum [BH,nb,d] and the pooled scores
// S [BH*nb, nb].
sa_status launch_route_keys(const Geometry& g, const float* qm, const uint16_t* K,
                            const uint16_t* Vt, const float* v_sum, const float* S, float* keys,
                            hipStream_t stream);

// ----------------------------------------------------------------------------
// attention (k_attn.hip)
// ----------------------------------------------------------------------------
// V re-laid out block by block, [BH, nb, d, block] (keys past N are zero).
sa_status launch_vt_layout(const Geometry& g, const uint16_t* V, uint16_t* Vt, hipStream_t stream);

// Workspace of the attention call: block token counts, V transposed per block
// (+ centroid tiles).
size_t fwd_workspace_bytes(const Geometry& g, bool comp);

// kv_count: device int32 [BH, nb] token counts per KV block, or null for the
// fixed layout (block, the last one N - (nb - 1) block).
// vmap (optional, [BH][g.N], negative: no token): V holds vN tokens per head
// and the layout's rows read them through the map
sa_status launch_fwd_prepare(const Geometry& g, const uint16_t* V, const int32_t* row_ptr,
                             const float* k_mean, const float* v_sum, const int32_t* kv_count,
                             char* ws, hipStream_t stream, const int32_t* vmap = nullptr,
                             int vN = 0);
// the attention on a block layout whose rows map to the tokens of Q, O, lse
// through qmap ([BH][g.N], negative: no token) with qN tokens per head
sa_status launch_fwd_run_mapped(const Geometry& g, bool comp, const uint16_t* Q, const uint16_t* K,
                                const int32_t* row_ptr, const int32_t* col_idx,
                                const int32_t* qmap, int32_t qN, uint16_t* O, float* lse, char* ws,
                                hipStream_t stream);
sa_status launch_fwd_run(const Geometry& g, bool comp, const uint16_t* Q, const uint16_t* K,
                         const int32_t* row_ptr, const int32_t* col_idx, uint16_t* O, float* lse,
                         char* ws, hipStream_t stream);

// ----------------------------------------------------------------------------
// token reordering (k_permute.hip)
// ----------------------------------------------------------------------------
sa_status launch_permute(const Geometry& g, const uint16_t* src, uint16_t* dst,
                         const int32_t* perm, bool inverse, hipStream_t stream);

// ----------------------------------------------------------------------------
// Hilbert order (hilbert.cpp)
// ----------------------------------------------------------------------------
sa_status build_hilbert_order(int32_t T, int32_t Hg, int32_t W, int32_t* perm,
                              int32_t* inv);

}  // namespace sa
