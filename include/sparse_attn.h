/*
 * sparse_attn.h -- C ABI of the MI355X (gfx950) block-sparse video attention
 * library (libsparse_attn.so).
 *
 * The library computes training-free dynamic block-sparse self-attention for
 * video diffusion transformers in two stages:
 *
 *   1. selection  -- optional 3D Hilbert token reordering, block means of Q
 *                    and K, pooled block scores, and a per-query-block keep
 *                    list (top-k or cumulative softmax mass) unioned with a
 *                    temporal window and rotating global anchor blocks;
 *   2. attention  -- a streaming (online-softmax) forward pass over the kept
 *                    KV blocks only, optionally adding every skipped KV block
 *                    back as one centroid term.
 *
 * Sources, by page title and section:
 *   [DFS]  "DFSAttn: Dynamic Fine-grained Sparse Attention for Efficient Video
 *          Generation": trick 1 (3D Hilbert reordering), trick 2 (block and
 *          sub-block scores from block means).
 *   [EAR]  "SVG-EAR: Parameter-Free Linear Compensation for Sparse Video
 *          Generation via Error-aware Routing": section 2A (skipped blocks
 *          replaced by their centroid), 2B (selection under a fixed density
 *          budget; streaming update without materialised logits), section 4
 *          (top-p selection).
 *   [SVOO] "SVOO: Training-Free Sparse Attention for Fast Video Generation ...":
 *          section 2A (density covering a share of cumulative attention mass).
 *   [LVSA] "LVSA: Training-Free Sparse Attention for Long Video Diffusion",
 *          abstract (structured window pattern plus rotating global anchors).
 *   [SPADE]"SPADE: An Input-Adaptive Sparse Attention Engine for Fast Video
 *          Diffusion Models Inference", part 2 (keep decision per head) and
 *          part 3 (head-wise sparse attention kernel).
 *
 * Conventions shared by every entry point
 *   - Tensors Q, K, V, O are bf16, shape [B, H, N, d], contiguous, 16-byte
 *     aligned device pointers.  Token n of the latent grid (T, Hg, W) is
 *     n = (t*Hg + y)*W + x in raster order.
 *   - Blocks are contiguous runs of `block` tokens of the sequence as given
 *     (raster or Hilbert order); nb = ceil(N / block); the last block holds
 *     N - (nb-1)*block tokens.
 *   - Ownership: the caller allocates and frees every buffer (device memory
 *     for tensors, masks and workspace; host memory for host arrays).  The
 *     library allocates no memory and never synchronises the stream; the
 *     one exception is the fixed scratch array of sparse_attn_select_noalloc,
 *     a static device array reserved when the library is loaded on a GPU.
 *     Its only host state between calls is launch set-up, kept per device
 *     behind a mutex (safe from several host threads): a kernel's LDS limit
 *     raised once per device, the number of workgroups a device holds at
 *     once (queried once per kernel, device and size), and the device
 *     address of that scratch array.
 *   - Ordering: device work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream) and is asynchronous.  A workspace carries one
 *     call's intermediate state on the device (pooled means, scores, the
 *     re-laid-out V, the attention kernel's row counters): calls that share
 *     a workspace must be ordered (one stream, or synchronised streams);
 *     two such calls in flight at once race.
 *   - Errors: arguments are validated on the host before any launch; a
 *     failed check returns SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED or
 *     SA_ERR_WORKSPACE and enqueues nothing.  A failed launch returns
 *     SA_ERR_HIP.  sparse_attn_last_error() then describes the failure.
 *     Non-finite input values are not checked (undefined results).
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SA_OK = 0,
    SA_ERR_INVALID_ARG = 1,   /* malformed argument (null, size, range)         */
    SA_ERR_UNSUPPORTED = 2,   /* well-formed but outside what is implemented     */
    SA_ERR_WORKSPACE = 3,     /* workspace missing, misaligned or too small      */
    SA_ERR_HIP = 4            /* a HIP runtime call or kernel launch failed      */
} sa_status;

/* Problem statement: the dense 3D self-attention the sparse call replaces. */
typedef struct {
    int32_t B, H, N, d;   /* batch, heads, tokens, head dim (d: 64 or 128)     */
    int32_t T, Hg, W;     /* latent grid; T*Hg*W must equal N                   */
    int32_t block;        /* tokens per Q block and per KV block: 64 or 128     */
    float scale;          /* softmax scale; <= 0 selects (float)(1/sqrt(d))     */
    const int32_t* token_order;
                          /* NULL: blocks are runs of the tokens as given.
                             Else device int32 [N], a permutation: blocks are
                             runs of the sequence token_order[0], token_order[1],
                             ... (e.g. the Hilbert order of hilbert_perm_build
                             [DFS trick 1]), while Q, K, V, O and lse stay in
                             the caller's token order: the kernels read and
                             write rows through it, so no separate reordering
                             pass is needed.  Masks, scores and block
                             statistics are indexed by these blocks.  Taken by
                             sparse_attn_workspace_size, sparse_attn_select(_noalloc),
                             sparse_attn_centroids and sparse_attn_fwd(_prepare,
                             _run) (the forward workspace then also holds K in
                             block order, gathered by sparse_attn_fwd_run);
                             the other calls reject it (SA_ERR_UNSUPPORTED), as
                             does a latent-frame window (frames are runs of
                             raster blocks).  Not checked to be a permutation:
                             every entry is clamped into [0, N), so a sequence
                             that is not one gives wrong rows, never an access
                             outside the tensors (the same holds for the perm
                             of hilbert_permute / hilbert_unpermute).          */
} sa_problem;

enum {
    SA_RULE_NONE = 0,     /* structural blocks only (window, anchors, diagonal) */
    SA_RULE_TOPK = 1,     /* k highest pooled scores per query block  [EAR 2B] */
    SA_RULE_MASS = 2,     /* shortest score-ranked prefix reaching `mass` of the
                             softmax mass of the pooled scores  [EAR 4, SVOO 2A] */
    SA_RULE_ERR = 3       /* k largest compensation errors per block size  [EAR 2B
                             error-aware routing]; needs want_comp, whole blocks */
};

/* Data-dependent block formation [SVOO 2B co-clustering, EAR 2A k-means]. */
enum {
    SA_CLUSTER_COCLUSTER = 1, /* keys by affinity (dot product) to the query
                                 centroids, then queries by affinity to the key
                                 centroids, alternately  [SVOO 2B]            */
    SA_CLUSTER_KMEANS = 2,    /* k-means (squared Euclidean distance) on Q and on
                                 K separately  [EAR 2A]                       */
    SA_CLUSTER_TILES = 3      /* the tiles of one shape of a menu per (b, h),
                                 chosen by sparse_attn_sics  [SPADE parts 1-2] */
};

/* A 3D tile shape (latent frames, rows, columns) [SPADE part 1]. */
typedef struct {
    int32_t t, y, x;
} sa_tile_shape;

typedef struct {
    int32_t mode;         /* SA_CLUSTER_*                                        */
    int32_t n_clusters;   /* COCLUSTER, KMEANS: C in [1, min(N, 1024)], the same
                             for Q and K.  TILES: the largest tile count of the
                             menu (must be <= 1024)                              */
    int32_t iters;        /* COCLUSTER, KMEANS: rounds in [1, 64] (one round
                             assigns both sides); ignored by TILES               */
    int32_t n_shapes;     /* TILES: menu size in [1, 16]                         */
    const sa_tile_shape* shapes;  /* TILES: host [n_shapes]; every shape's volume
                                     t*y*x <= block, so a tile is one block      */
    const int32_t* shape_idx;     /* TILES: device int32 [B*H], the menu entry of
                                     each (b, h) (sparse_attn_sics writes it);
                                     read by sparse_attn_cluster and, with a
                                     ticket, sparse_attn_cluster_select          */
    float ticket;                 /* TILES with tile_coherence: the SICS ticket
                                     [SPADE part 2], finite in [-1, 1].  A key
                                     tile whose keys agree -- mean cosine of its
                                     ordered key pairs >= ticket, decided in
                                     fp64 -- may be kept; the others are ignored
                                     (never kept; with compensation they enter
                                     as centroids).  Unused without
                                     tile_coherence.                             */
    double* tile_coherence;       /* TILES, optional (null: no ticket, every tile
                                     may be kept): device fp64 [B*H, n_shapes,
                                     n_clusters], the mean key cosine of every
                                     tile of every menu shape (1 for a tile of
                                     fewer than two tokens; entries past a
                                     shape's tile count are not written).
                                     sparse_attn_sics writes it,
                                     sparse_attn_cluster_select reads it with
                                     shape_idx and applies the ticket           */
} sa_cluster_spec;

/* Selection rule.  Host-side struct; `topk` and `density` are host arrays. */
typedef struct {
    int32_t rule;            /* SA_RULE_*                                         */
    int32_t sub_block;       /* 0, or a power of two >= 16 dividing `block`:
                                score = max over sub-block pairs  [DFS trick 2]  */
    const int32_t* topk;     /* host [H] blocks kept per head (clamped to 1..nb),
                                or NULL to derive k from `density`               */
    const float* density;    /* host [H] in (0,1]: k = clamp(ceil(rho*nb*(1-1e-6)),
                                1, nb); used when topk == NULL                   */
    float mass;              /* SA_RULE_MASS threshold tau in (0, 1]              */
    int32_t diag;            /* 1: always keep KV block j == i                    */
    int32_t window_frames;   /* -1: off.  r >= 0: keep KV block j when the latent
                                frames it covers come within r frames of those of
                                query block i (raster order)  [LVSA]             */
    int32_t n_anchors;       /* A in [0, nb]: anchors a_m = (anchor_offset +
                                m*floor(nb/A)) mod nb kept for every row  [LVSA] */
    int64_t anchor_offset;   /* rotation of the anchors for this call (>= 0)      */
    int32_t want_comp;       /* 1: also write k_mean and v_sum for compensation   */
    void* v_blocks;          /* SA_RULE_ERR only, optional (NULL for the other
                                rules).  The error rule needs V re-laid out
                                block by block ([B,H,nb,d,block] bf16, keys past
                                N zero), the layout the forward call needs too.
                                NULL: it is built in the selection workspace.
                                Non-NULL (device, 256-byte aligned, room for
                                B*H*nb*d*block bf16): it is written here and
                                left for the caller; passing the start of a
                                forward workspace lets sparse_attn_fwd_prepare
                                skip its own re-layout (V = NULL there).
                                sparse_attn_workspace_size reads only whether
                                it is NULL.                                     */
} sa_select_spec;

/*
 * Workspace bytes needed by sparse_attn_select (spec != NULL; with the error
 * rule and spec->v_blocks == NULL this includes V re-laid out block by block)
 * or by sparse_attn_fwd (spec == NULL; the size covers calls with and without
 * compensation: V re-laid out block by block in its first 2*B*H*nb*d*block
 * bytes, then the bf16 centroid tiles and the work split).  The same buffer
 * may be reused by consecutive calls on one stream.
 */
sa_status sparse_attn_workspace_size(const sa_problem* prob,
                                     const sa_select_spec* spec, size_t* bytes);

/*
 * 3D Hilbert token order [DFS trick 1], host only.  The grid is placed in the
 * cube of side 2^b (b = ceil(log2(max(T, Hg, W))), at least 1), the cube's
 * cells are walked along the Hilbert curve (J. Skilling's construction,
 * "Programming the Hilbert curve", 2004; x on the curve's first-step axis, t
 * and y on the other two in order) and cells outside the grid are dropped.
 * perm[r] = raster index of the r-th kept cell; inv[perm[r]] = r.
 * perm and inv: caller-owned host arrays of T*Hg*W int32 each (inv may be NULL).
 * Returns SA_ERR_UNSUPPORTED when max(T,Hg,W) > 256.
 */
sa_status hilbert_perm_build(int32_t T, int32_t Hg, int32_t W,
                             int32_t* perm, int32_t* inv);

/*
 * Token reordering of one [B,H,N,d] bf16 tensor [DFS trick 1]:
 *   hilbert_permute:   dst[b,h,n,:]       = src[b,h,perm[n],:]
 *   hilbert_unpermute: dst[b,h,perm[n],:] = src[b,h,n,:]
 * perm_dev: device int32 [N], a permutation of 0..N-1 (not checked on the
 * host; entries outside [0, N) are skipped by the kernel, and a
 * non-permutation leaves rows of dst unwritten).  src and dst must not overlap.
 */
sa_status hilbert_permute(const sa_problem* prob, const void* src, void* dst,
                          const int32_t* perm_dev, void* stream);
sa_status hilbert_unpermute(const sa_problem* prob, const void* src, void* dst,
                            const int32_t* perm_dev, void* stream);

/*
 * Block selection [DFS trick 2, EAR 2B/4, SVOO 2A, LVSA, SPADE part 2].
 * For every (b, h, query block i) the row of kept KV blocks is the union of
 *   - the rule's set: blocks ranked by pooled score S[i,j] (descending; ties by
 *     lower j), the first k (TOPK) or the shortest prefix whose softmax mass
 *     sum_{first m} exp(S - S_max) reaches mass * (sum over all j) (MASS);
 *   - j == i when diag; the window blocks; the anchor blocks.
 * Pooled score: S[i,j] = fl32(scale * dot(qbar_i, kbar_j)) where qbar, kbar are
 * block means (fp32 rounding of the exact mean) and dot is a sequential fp32
 * fused-multiply-add chain over the d channels; with sub_block, qbar/kbar are
 * sub-block means and S[i,j] is the max over the sub-block pairs of (i, j).
 *
 * SA_RULE_ERR [EAR 2B] ranks the blocks of row i by the compensation error of
 * block j probed with the query block's mean qbar_i (the query centroid):
 *   m = max_t scale*qbar_i.k_t over the tokens t of block j,
 *   A = sum_t exp(scale*qbar_i.k_t - m) v_t,  Ahat = n_j exp(S[i,j] - m) vbar_j,
 *   key[i,j] = ln ||A - Ahat||_2 + m - ln n_j   (-inf when A == Ahat),
 * with vbar_j = fl32(sum_t v_t) / n_j, and keeps the k largest keys (k from
 * topk / density as for SA_RULE_TOPK; ties by lower j).  It requires
 * want_comp = 1 (the error is that of the compensation) and sub_block = 0.
 * The probe is computed on the matrix cores with bf16 hi/lo splits of qbar
 * and of the exponentials (about 16 significant bits), fp32 accumulation.
 *
 * Q, K: device bf16 [B,H,N,d] (ignored for SA_RULE_NONE).  V: device bf16, used
 *   when want_comp (else may be NULL).
 * row_ptr: device int32 [B*H*nb + 1]; col_idx: device int32, capacity
 *   B*H*nb*nb.  Row r = (b*H + h)*nb + i lists its kept KV blocks in
 *   col_idx[row_ptr[r] .. row_ptr[r+1]), strictly ascending.
 * scores: optional device fp32 [B*H*nb*nb] receiving the ranking key: S for
 *   TOPK / MASS, key for ERR (NULL: not written; never written for
 *   SA_RULE_NONE).
 * k_mean, v_sum: device fp32 [B,H,nb,d] when want_comp (block means of K;
 *   fp32 block sums of V), else NULL.
 * workspace: device, 256-byte aligned, >= sparse_attn_workspace_size(prob, spec).
 * Limits: nb <= 4096 for the scored rules (SA_ERR_UNSUPPORTED above).
 */
sa_status sparse_attn_select(const sa_problem* prob, const sa_select_spec* spec,
                             const void* Q, const void* K, const void* V,
                             int32_t* row_ptr, int32_t* col_idx, float* scores,
                             float* k_mean, float* v_sum,
                             void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_attn_select without a workspace, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Arguments, results and errors are those of
 * sparse_attn_select; the scratch the selection needs (pooled means, scores,
 * keep bitmap, per-row counts) comes from a fixed 64 MiB device array of the
 * library, one per GPU, reserved when the library is loaded on that GPU and
 * held until the process ends.  A selection that needs more scratch (see
 * sparse_attn_workspace_size) is rejected with SA_ERR_UNSUPPORTED before
 * anything is enqueued.  The call allocates and frees nothing.  Every call on
 * one GPU uses that GPU's one array: calls on one GPU must be ordered (one
 * stream, or synchronised streams); two in flight at once race.
 */
sa_status sparse_attn_select_noalloc(const sa_problem* prob, const sa_select_spec* spec,
                                     const void* Q, const void* K, const void* V,
                                     int32_t* row_ptr, int32_t* col_idx, float* scores,
                                     float* k_mean, float* v_sum, void* stream);

/*
 * Compensation statistics of the current K and V without a selection
 * [EAR 2A; mask reuse across steps: DFS trick 3, SVOO 2B].  A caller that keeps
 * the CSR of an earlier sparse_attn_select (the mask of a previous call or
 * diffusion step) and skips the selection still needs the centroids of the
 * blocks it now skips, taken from the current K and V:
 *   k_mean[b,h,j,:] = mean of K over the tokens of block j (fp32 rounding of
 *                     the exact mean, as sparse_attn_select writes it),
 *   v_sum[b,h,j,:]  = fp32 rounding of the exact sum of V over block j.
 * K, V: device bf16 [B,H,N,d], 16-byte aligned.  k_mean, v_sum: device fp32
 * [B,H,nb,d].  No workspace.  Errors: SA_ERR_INVALID_ARG for a NULL or
 * misaligned pointer, problem errors as for every call.
 */
sa_status sparse_attn_centroids(const sa_problem* prob, const void* K, const void* V,
                                float* k_mean, float* v_sum, void* stream);

/*
 * Block-sparse attention forward [EAR 2B streaming update; SPADE part 3].
 * For a query token n of block i:
 *   O[n] = sum_t exp(l_t - m) v_t / sum_t exp(l_t - m),  l_t = scale * q_n.k_t,
 * over the tokens t of the KV blocks listed in row i of (row_ptr, col_idx).
 * With compensation (k_mean and v_sum both non-NULL) [EAR 2A] every KV block j
 * NOT listed adds one centroid term: logit scale*q_n.k_mean_j, weight n_j
 * (its token count), value v_sum_j / n_j.
 * Q, K, V: device bf16 [B,H,N,d].  row_ptr/col_idx: as written by
 *   sparse_attn_select (strictly ascending rows, indices in [0, nb); not
 *   checked).  O: device bf16 [B,H,N,d].  lse: optional device fp32 [B,H,N],
 *   natural-log log-sum-exp of the logits (including compensation terms).
 * A row with no kept block and no compensation gives O = 0, lse = -inf.
 * A malformed CSR cannot make the kernel read or write outside its buffers:
 * column indices outside [0, nb) are clamped into range, a row longer than
 * nb entries is cut to its first nb, and a row with row_ptr[r+1] < row_ptr[r]
 * is taken as empty (results for such input are unspecified, but the call
 * ends normally).  row_ptr itself must hold B*H*nb + 1 entries whose values
 * index col_idx's capacity.
 * workspace: device, 256-byte aligned, >= sparse_attn_workspace_size(prob,
 *   NULL); it receives V transposed block by block (and the centroid tiles).
 * Precision: QK^T and PV on bf16 matrix cores with fp32 accumulation, softmax
 *   in fp32, output rounded to bf16.
 * Limits: nb <= 4096 (SA_ERR_UNSUPPORTED above).
 */
sa_status sparse_attn_fwd(const sa_problem* prob, const void* Q, const void* K,
                          const void* V, const int32_t* row_ptr,
                          const int32_t* col_idx, const float* k_mean,
                          const float* v_sum, void* O, float* lse,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_attn_fwd in two halves, for callers that reuse the prepared V or time
 * the attention kernel alone.  sparse_attn_fwd(...) is exactly
 * sparse_attn_fwd_prepare(...) followed by sparse_attn_fwd_run(...) on the
 * same stream, workspace and problem.
 *
 * sparse_attn_fwd_prepare: writes into the workspace V re-laid out block by
 *   block ([B,H,nb,d,block] bf16, keys past N zero; the workspace's first
 *   2*B*H*nb*d*block bytes), with compensation (k_mean, v_sum both non-NULL)
 *   the bf16 centroid keys and values, and the split of the rows into per-XCD
 *   work ranges (reads row_ptr).  V = NULL skips the re-layout: the workspace
 *   must then already start with this V in that layout, e.g. written by a
 *   sparse_attn_select with SA_RULE_ERR and spec->v_blocks = workspace, on
 *   the same stream, for the same problem and V.
 * sparse_attn_fwd_run: the attention kernel.  Reads the workspace written by
 *   the last sparse_attn_fwd_prepare on this stream, which must have had the
 *   same prob, the same row_ptr contents and with_comp = (k_mean != NULL);
 *   this is not checked.  It may be called several times per preparation
 *   (with other Q, K, O or col_idx of the same row structure).
 * Arguments, errors and limits as for sparse_attn_fwd.
 */
sa_status sparse_attn_fwd_prepare(const sa_problem* prob, const void* V,
                                  const int32_t* row_ptr, const float* k_mean,
                                  const float* v_sum, void* workspace,
                                  size_t ws_bytes, void* stream);
sa_status sparse_attn_fwd_run(const sa_problem* prob, const void* Q, const void* K,
                              const int32_t* row_ptr, const int32_t* col_idx,
                              int32_t with_comp, void* O, float* lse,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Data-dependent block formation [SVOO 2B; EAR 2A].  Instead of fixed runs of
 * `block` tokens, the blocks are clusters of tokens with similar content,
 * found per (batch, head) and separately for queries and keys:
 *   start:  C equal chunks of the token order; their means are the centroids;
 *   round:  COCLUSTER -- every key goes to the query centroid c maximising
 *           k.c, key centroids = means; every query goes to the key centroid
 *           maximising q.c, query centroids = means (key cluster c is the
 *           partner of query cluster c);
 *           KMEANS -- every query (key) goes to the query (key) centroid
 *           maximising x.c - |c|^2/2 (nearest in Euclidean distance), then
 *           centroids = means.
 * Arithmetic of the decision: x.c is a sequential fp32 fused-multiply-add
 * chain over the channels (channel order), |c|^2/2 = fl32(0.5 * that chain of
 * c with itself), one fp32 add; ties go to the lower cluster index.  Means
 * are fp32 roundings of exact sums (fp64) divided by the count; an empty
 * cluster keeps its previous centroid.
 *
 * TILES -- no iteration: the clusters of (b, h) are the tiles of menu shape
 *           shape_idx[b*H+h], the same partition for Q and K; clusters past
 *           that shape's tile count are empty and their centroids are 0.
 *
 * Padded layout: a cluster takes whole blocks of the layout -- its tokens in
 * ascending token order, then zero padding to a multiple of `block`; clusters
 * follow each other in index order.  The layout has nbp = ceil(N/block) + C
 * blocks (an upper bound for every head; TILES: nbp = C, one block per tile),
 * Np = nbp * block slots; blocks past the last cluster are empty.  Attention on the layout is a plain sa_problem
 * with N = Np (T = Hg = 1, W = Np) whose KV blocks carry token counts
 * (sparse_attn_fwd_prepare_counts).
 * ---------------------------------------------------------------------------
 *
 * sparse_attn_cluster_size: nbp and the workspace bytes of sparse_attn_cluster
 *   (ws_cluster) and of sparse_attn_cluster_select (ws_select).
 */
sa_status sparse_attn_cluster_size(const sa_problem* prob, const sa_cluster_spec* cspec,
                                   int32_t* nb_padded, size_t* ws_cluster, size_t* ws_select);

/*
 * SICS scheme generation [SPADE part 2: per head and step, the sum of
 * intra-block cosine similarities decides the scheme; part 1: a menu of 3D
 * tile shapes].  cspec: mode SA_CLUSTER_TILES with the menu.  For every
 * (b, h) and menu shape s: tiles of s cut the (T, Hg, W) grid ([tt*t,
 * (tt+1)*t) x ... clipped at the grid's end, numbered in raster order of the
 * tile coordinates); the score is the mean cosine similarity of the ordered
 * pairs of distinct tokens inside a tile, over queries and keys:
 *     (sum_tiles |sum_a q_a/|q_a||^2 - nq + |sum_a k_a/|k_a||^2 - nk)
 *       / (2 sum_tiles n (n - 1))
 * (nq, nk: tokens with a non-zero vector; a zero vector has cosine 0), in
 * fp64; shape_idx[b*H+h] = the shape with the largest score, the first of the
 * menu on ties.  Q, K: device bf16 [B,H,N,d].  scores: optional device fp64
 * [B*H, n_shapes].  shape_idx: device int32 [B*H].  workspace: device,
 * 256-byte aligned, >= the ws_cluster of sparse_attn_cluster_size.  The
 * partition itself is then sparse_attn_cluster with the same cspec and
 * shape_idx set: every tile is one block (nbp = n_clusters), tokens in raster
 * order inside it.
 */
sa_status sparse_attn_sics(const sa_problem* prob, const sa_cluster_spec* cspec, const void* Q,
                           const void* K, double* scores, int32_t* shape_idx, void* workspace,
                           size_t ws_bytes, void* stream);

/*
 * sparse_attn_cluster: clusters Q and K of every (b, h) and lays them out.
 * Q, K: device bf16 [B,H,N,d].  V: optional device bf16 [B,H,N,d]: with V,
 *   v_cent receives the means of V over the key clusters (compensation).
 * Outputs (device): q_order, k_order int32 [B*H, Np] (token at each padded
 *   slot, -1 for padding); q_blk, k_blk int32 [B*H, nbp] (cluster of each
 *   padded block, -1 for none); q_cnt, k_cnt int32 [B*H, nbp] (tokens in each
 *   padded block); q_cent, k_cent fp32 [B*H, C, d]; q_count, k_count int32
 *   [B*H, C] (cluster sizes).  v_cent may be NULL.
 * workspace: device, 256-byte aligned, >= ws_cluster bytes.
 */
sa_status sparse_attn_cluster(const sa_problem* prob, const sa_cluster_spec* cspec,
                              const void* Q, const void* K, const void* V,
                              int32_t* q_order, int32_t* k_order, int32_t* q_blk,
                              int32_t* k_blk, int32_t* q_cnt, int32_t* k_cnt,
                              float* q_cent, float* k_cent, float* v_cent,
                              int32_t* q_count, int32_t* k_count,
                              void* workspace, size_t ws_bytes, void* stream);

/*
 * Rows into / out of the padded layout.  gather: dst[b,h,p,:] =
 * src[b,h,order[b,h,p],:] (zeros where order = -1); src [B,H,N,d], dst
 * [B,H,Np,d].  scatter: dst[b,h,order[b,h,p],:] = src[b,h,p,:] for every slot
 * with order >= 0 (other rows of dst untouched); with lse_src/lse_dst
 * (fp32 [B,H,Np] / [B,H,N], both or neither) the same for the log-sum-exp.
 * bf16 rows, 16-byte aligned; src and dst must not overlap.
 */
sa_status sparse_attn_cluster_gather(const sa_problem* prob, const sa_cluster_spec* cspec,
                                     const int32_t* order, const void* src, void* dst,
                                     void* stream);
sa_status sparse_attn_cluster_scatter(const sa_problem* prob, const sa_cluster_spec* cspec,
                                      const int32_t* order, const void* src, void* dst,
                                      const float* lse_src, float* lse_dst, void* stream);

/*
 * sparse_attn_cluster_select: the keep decision over clusters, as CSR over
 * the padded blocks.  S[a,b] = fl32(scale * seqfma(q_cent[a], k_cent[b])).
 * Empty key clusters are never kept; the others are ranked by S (descending,
 * lower index on ties) and query cluster a keeps
 *   SA_RULE_TOPK: the shortest prefix whose key tokens reach
 *                 max(1, ceil(density[h] * N * (1 - 1e-6)));
 *   SA_RULE_MASS: the shortest prefix whose sum of n_b exp(S_b - S_max)
 *                 (fp64, rank order) reaches mass * (the total);
 * plus b = a when diag and key cluster a is not empty.  Every padded block of
 * query cluster a then keeps every padded block of its kept key clusters;
 * blocks of no cluster keep nothing.  spec: rule TOPK (density only) or MASS,
 *   diag, want_comp; sub_block, windows and anchors are not supported.
 * Inputs as written by sparse_attn_cluster (v_cent needed with want_comp).
 * row_ptr int32 [B*H*nbp + 1], col_idx int32 capacity B*H*nbp*nbp (ascending
 *   rows).  scores: optional fp32 [B*H, C, C].  k_mean, v_sum: fp32
 *   [B*H, nbp, d] with want_comp: the key centroid of the block's cluster and
 *   (block token count) x (value mean of the cluster), so that the
 *   compensation of the attention call adds, for every skipped key cluster,
 *   its centroid with the cluster's token count as weight.
 * workspace: device, 256-byte aligned, >= ws_select bytes.
 */
sa_status sparse_attn_cluster_select(const sa_problem* prob, const sa_cluster_spec* cspec,
                                     const sa_select_spec* spec, const float* q_cent,
                                     const float* k_cent, const float* v_cent,
                                     const int32_t* k_count, const int32_t* q_blk,
                                     const int32_t* k_blk, const int32_t* k_cnt,
                                     int32_t* row_ptr, int32_t* col_idx, float* scores,
                                     float* k_mean, float* v_sum,
                                     void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_attn_cluster_centroids: for a call that reuses a partition (and its
 * selection) made on an earlier call [SVOO 2B: the clustering is kept for
 * several diffusion steps]: the key and value means of every key cluster from
 * this call's K and V, already gathered into the padded layout (Kp, Vp: device
 * bf16 [B,H,Np,d], padding rows zero, e.g. by sparse_attn_cluster_gather with
 * k_order), written to k_cent, v_cent (fp32 [B*H, C, d]; clusters with no
 * token are left untouched), and the per-block compensation statistics k_mean,
 * v_sum (fp32 [B*H, nbp, d]) as sparse_attn_cluster_select writes them.
 * k_count, k_blk, k_cnt: as written by sparse_attn_cluster.  Means are fp32
 * roundings of exact sums, so unchanged inputs reproduce sparse_attn_cluster's
 * centroids bit for bit.
 */
sa_status sparse_attn_cluster_centroids(const sa_problem* prob, const sa_cluster_spec* cspec,
                                        const void* Kp, const void* Vp, const int32_t* k_count,
                                        const int32_t* k_blk, const int32_t* k_cnt, float* k_cent,
                                        float* v_cent, float* k_mean, float* v_sum, void* stream);

/*
 * sparse_attn_fwd_prepare with token counts per KV block: kv_count device
 * int32 [B*H, nb] in [0, block]; keys past the count of a block take no part
 * (masked in kept blocks; weight n_j = the count for compensation, a block
 * with count 0 contributes nothing).  sparse_attn_fwd_prepare is this call
 * with the counts of the fixed layout (block, the last one N - (nb-1)*block).
 * Follow it with sparse_attn_fwd_run as usual.
 */
sa_status sparse_attn_fwd_prepare_counts(const sa_problem* prob, const void* V,
                                         const int32_t* row_ptr, const float* k_mean,
                                         const float* v_sum, const int32_t* kv_count,
                                         void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_attn_fwd_prepare_counts over the padded clustered layout with V read
 * in the caller's token order: the padded slot p of head (b, h) holds the
 * value row V[b, h, k_order[b*H+h, p], :] (zeros where k_order = -1).  This
 * is sparse_attn_cluster_gather of V followed by
 * sparse_attn_fwd_prepare_counts on the padded problem (N_p = nbp * block
 * tokens in one flat frame), in one pass.  prob, cspec: the token-order
 * problem and the clustering.  k_order: device int32 [B*H, N_p] as written by
 * sparse_attn_cluster (not checked: an entry >= N is clamped to N - 1, a
 * negative one gives a zero row).  V: device bf16 [B,H,N,d], 16-byte aligned.  row_ptr,
 * k_mean, v_sum, kv_count, workspace: as for sparse_attn_fwd_prepare_counts
 * on the padded problem.
 */
sa_status sparse_attn_cluster_fwd_prepare(const sa_problem* prob, const sa_cluster_spec* cspec,
                                          const int32_t* k_order, const void* V,
                                          const int32_t* row_ptr, const float* k_mean,
                                          const float* v_sum, const int32_t* kv_count,
                                          void* workspace, size_t ws_bytes, void* stream);

/*
 * sparse_attn_fwd_run over the padded clustered layout with Q read and O, lse
 * written in the caller's token order [SVOO 2B: attention within the
 * clusters' blocks; SVG-EAR 2A: the permutation that makes clusters
 * contiguous]: the attention problem is that of the padded layout (N_p =
 * nbp * block tokens in one flat frame, as the workspace was prepared for by
 * sparse_attn_fwd_prepare_counts); the query row of padded slot p of head
 * (b, h) is Q[b, h, q_order[b*H+h, p], :], its output row and lse go to the
 * same token, and slots with q_order = -1 (padding) are skipped.  This is
 * sparse_attn_cluster_gather of Q, sparse_attn_fwd_run and
 * sparse_attn_cluster_scatter of O and lse in one pass.
 * prob, cspec: the token-order problem and the clustering (prob without a
 * token order).  q_order: device int32 [B*H, N_p] as written by
 * sparse_attn_cluster (entries in [0, N) or -1; not checked: an entry >= N
 * is clamped to N - 1, any negative one skips its slot).  Q, O: device bf16
 * [B,H,N,d]; lse: optional device fp32 [B,H,N]; rows of tokens that no slot
 * maps to are left untouched.  Kp: device bf16 [B,H,N_p,d] (K gathered by
 * k_order).  row_ptr, col_idx, with_comp, workspace: as for
 * sparse_attn_fwd_run on the padded problem.  All tensors 16-byte aligned.
 */
sa_status sparse_attn_cluster_fwd_run(const sa_problem* prob, const sa_cluster_spec* cspec,
                                      const int32_t* q_order, const void* Q, const void* Kp,
                                      const int32_t* row_ptr, const int32_t* col_idx,
                                      int32_t with_comp, void* O, float* lse,
                                      void* workspace, size_t ws_bytes, void* stream);

/* Text of the last failure on the calling thread ("" after success). */
const char* sparse_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
