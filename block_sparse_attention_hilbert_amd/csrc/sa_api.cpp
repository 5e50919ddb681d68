// Public C ABI of libsparse_attn.so: argument validation, workspace sizing and
// dispatch to the gfx950 kernels.  Every check runs on the host before any
// HIP call, so a rejected call enqueues nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <string>

#include "sa_internal.h"

#define SA_API extern "C" __attribute__((visibility("default")))

namespace sa {

static thread_local std::string g_last_error;

sa_status fail(sa_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

sa_status hip_check(hipError_t e, const char* what) {
    if (e == hipSuccess) return SA_OK;
    return fail(SA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

void clear_error() { g_last_error.clear(); }

// Per-device launch set-up memo (see sa_internal.h).
namespace {
struct LaunchKey {
    int dev;
    const void* fn;
    int threads;
    size_t lds;
    bool operator<(const LaunchKey& o) const {
        if (dev != o.dev) return dev < o.dev;
        if (fn != o.fn) return fn < o.fn;
        if (threads != o.threads) return threads < o.threads;
        return lds < o.lds;
    }
};
std::mutex g_launch_mu;
std::map<LaunchKey, int> g_max_lds;      // (dev, fn) -> dynamic LDS limit set
std::map<LaunchKey, int> g_resident;     // (dev, fn, threads, lds) -> workgroups
}  // namespace

sa_status ensure_max_lds(const void* fn, int bytes, const char* what) {
    int dev = 0;
    sa_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
    if (st != SA_OK) return st;
    std::lock_guard<std::mutex> lock(g_launch_mu);
    const LaunchKey key{dev, fn, 0, 0};
    auto it = g_max_lds.find(key);
    if (it != g_max_lds.end() && it->second >= bytes) return SA_OK;
    st = hip_check(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes), what);
    if (st == SA_OK) g_max_lds[key] = bytes;
    return st;
}

sa_status resident_workgroups(const void* fn, int threads, size_t lds, int* out) {
    int dev = 0;
    sa_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
    if (st != SA_OK) return st;
    std::lock_guard<std::mutex> lock(g_launch_mu);
    const LaunchKey key{dev, fn, threads, lds};
    auto it = g_resident.find(key);
    if (it != g_resident.end()) {
        *out = it->second;
        return SA_OK;
    }
    int cus = 0, per_cu = 0;
    st = hip_check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev),
                   "multiprocessor count");
    if (st != SA_OK) return st;
    st = hip_check(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds),
                   "occupancy query");
    if (st != SA_OK) return st;
    *out = g_resident[key] = cus * (per_cu > 0 ? per_cu : 1);
    return SA_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Validates the problem statement and fills the derived geometry.
sa_status check_problem(const sa_problem* p, Geometry* g) {
    if (!p) return fail(SA_ERR_INVALID_ARG, "prob is NULL");
    if (p->B < 1 || p->H < 1 || p->N < 1)
        return fail(SA_ERR_INVALID_ARG, "B, H, N must be >= 1 (got %d, %d, %d)", p->B, p->H, p->N);
    if (p->T < 1 || p->Hg < 1 || p->W < 1)
        return fail(SA_ERR_INVALID_ARG, "latent grid sides must be >= 1 (got %d x %d x %d)",
                    p->T, p->Hg, p->W);
    if ((int64_t)p->T * p->Hg * p->W != (int64_t)p->N)
        return fail(SA_ERR_INVALID_ARG, "T*Hg*W = %lld does not equal N = %d",
                    (long long)p->T * p->Hg * p->W, p->N);
    if (p->d != 64 && p->d != 128)
        return fail(SA_ERR_UNSUPPORTED, "head dim d = %d (supported: 64, 128)", p->d);
    if (p->block != 64 && p->block != 128)
        return fail(SA_ERR_UNSUPPORTED, "block = %d (supported: 64, 128)", p->block);
    if (!isfinite(p->scale))
        return fail(SA_ERR_INVALID_ARG, "scale is not finite");
    if ((int64_t)p->B * p->H * p->N * p->d > ((int64_t)1 << 40))
        return fail(SA_ERR_UNSUPPORTED, "tensor too large");
    g->B = p->B; g->H = p->H; g->N = p->N; g->d = p->d; g->block = p->block;
    g->T = p->T; g->Hg = p->Hg; g->W = p->W;
    g->nb = (int32_t)ceil_div(p->N, p->block);
    g->scale = p->scale > 0.f ? p->scale : (float)(1.0 / sqrt((double)p->d));
    g->order = p->token_order;
    return SA_OK;
}

// Calls that work on the tokens as given only.
static sa_status no_token_order(const Geometry& g, const char* call) {
    if (g.order)
        return fail(SA_ERR_UNSUPPORTED, "%s takes no token_order (blocks of the tokens as given)",
                    call);
    return SA_OK;
}

sa_status check_spec(const Geometry& g, const sa_select_spec* s) {
    if (!s) return fail(SA_ERR_INVALID_ARG, "spec is NULL");
    if (s->rule != SA_RULE_NONE && s->rule != SA_RULE_TOPK && s->rule != SA_RULE_MASS &&
        s->rule != SA_RULE_ERR)
        return fail(SA_ERR_INVALID_ARG, "unknown rule %d", s->rule);
    if (s->v_blocks && s->rule != SA_RULE_ERR)
        return fail(SA_ERR_INVALID_ARG, "v_blocks is for SA_RULE_ERR only (must be NULL)");
    if (s->v_blocks && ((uintptr_t)s->v_blocks & 255u) != 0)
        return fail(SA_ERR_INVALID_ARG, "v_blocks must be 256-byte aligned");
    if (s->rule == SA_RULE_ERR) {
        if (s->want_comp != 1)
            return fail(SA_ERR_INVALID_ARG, "SA_RULE_ERR needs want_comp = 1");
        if (s->sub_block != 0)
            return fail(SA_ERR_INVALID_ARG, "SA_RULE_ERR works on whole blocks (sub_block = 0)");
    }
    if (s->rule != SA_RULE_NONE && g.nb > 4096)
        return fail(SA_ERR_UNSUPPORTED, "scored rules support nb <= 4096 (got %d)", g.nb);
    if (g.rows() * (int64_t)g.nb > (int64_t)INT32_MAX)
        return fail(SA_ERR_UNSUPPORTED, "B*H*nb*nb exceeds the int32 range of row_ptr");
    if (s->sub_block != 0) {
        const int sb = s->sub_block;
        if (sb < 16 || (sb & (sb - 1)) != 0 || g.block % sb != 0)
            return fail(SA_ERR_INVALID_ARG,
                        "sub_block = %d must be 0 or a power of two >= 16 dividing block = %d",
                        sb, g.block);
    }
    if (s->rule == SA_RULE_TOPK || s->rule == SA_RULE_ERR) {
        if (s->topk) {
            for (int h = 0; h < g.H; ++h)
                if (s->topk[h] < 1)
                    return fail(SA_ERR_INVALID_ARG, "topk[%d] = %d must be >= 1", h, s->topk[h]);
        } else if (s->density) {
            for (int h = 0; h < g.H; ++h)
                if (!(s->density[h] > 0.f && s->density[h] <= 1.f))
                    return fail(SA_ERR_INVALID_ARG, "density[%d] = %g must be in (0, 1]", h,
                                (double)s->density[h]);
        } else {
            return fail(SA_ERR_INVALID_ARG, "SA_RULE_TOPK and SA_RULE_ERR need topk or density");
        }
    }
    if (s->rule == SA_RULE_MASS && !(s->mass > 0.f && s->mass <= 1.f))
        return fail(SA_ERR_INVALID_ARG, "mass = %g must be in (0, 1]", (double)s->mass);
    if (s->window_frames < -1)
        return fail(SA_ERR_INVALID_ARG, "window_frames = %d must be >= -1", s->window_frames);
    if (s->window_frames >= 0 && g.order)
        return fail(SA_ERR_UNSUPPORTED,
                    "a latent-frame window needs blocks of raster tokens (no token_order)");
    if (s->n_anchors < 0 || s->n_anchors > g.nb)
        return fail(SA_ERR_INVALID_ARG, "n_anchors = %d must be in [0, nb = %d]", s->n_anchors, g.nb);
    if (s->anchor_offset < 0)
        return fail(SA_ERR_INVALID_ARG, "anchor_offset must be >= 0");
    if (s->diag != 0 && s->diag != 1)
        return fail(SA_ERR_INVALID_ARG, "diag must be 0 or 1");
    if (s->want_comp != 0 && s->want_comp != 1)
        return fail(SA_ERR_INVALID_ARG, "want_comp must be 0 or 1");
    return SA_OK;
}

}  // namespace sa

using namespace sa;

SA_API sa_status sparse_attn_workspace_size(const sa_problem* prob,
                                            const sa_select_spec* spec, size_t* bytes) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if (!bytes) return fail(SA_ERR_INVALID_ARG, "bytes is NULL");
    if (spec) {
        if ((st = check_spec(g, spec)) != SA_OK) return st;
        *bytes = make_select_plan(g, *spec).total;
    } else {
        *bytes = fwd_workspace_bytes(g, true);
    }
    return SA_OK;
}

SA_API sa_status hilbert_perm_build(int32_t T, int32_t Hg, int32_t W, int32_t* perm,
                                    int32_t* inv) {
    clear_error();
    if (T < 1 || Hg < 1 || W < 1)
        return fail(SA_ERR_INVALID_ARG, "grid sides must be >= 1 (got %d x %d x %d)", T, Hg, W);
    if (T > 256 || Hg > 256 || W > 256)
        return fail(SA_ERR_UNSUPPORTED, "grid sides must be <= 256");
    if ((int64_t)T * Hg * W > (int64_t)INT32_MAX)
        return fail(SA_ERR_UNSUPPORTED, "grid too large");
    if (!perm) return fail(SA_ERR_INVALID_ARG, "perm is NULL");
    return build_hilbert_order(T, Hg, W, perm, inv);
}

static sa_status permute_common(const sa_problem* prob, const void* src, void* dst,
                                const int32_t* perm, void* stream, bool inverse) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = no_token_order(g, "hilbert_permute and hilbert_unpermute")) != SA_OK) return st;
    if (!src || !dst || !perm) return fail(SA_ERR_INVALID_ARG, "src, dst and perm must be non-NULL");
    if (!aligned16(src) || !aligned16(dst))
        return fail(SA_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
    const size_t bytes = (size_t)g.BH() * g.N * g.d * 2;
    const char* s = (const char*)src;
    const char* d = (const char*)dst;
    if (s < d + bytes && d < s + bytes) return fail(SA_ERR_INVALID_ARG, "src and dst overlap");
    return launch_permute(g, (const uint16_t*)src, (uint16_t*)dst, perm, inverse,
                          (hipStream_t)stream);
}

SA_API sa_status hilbert_permute(const sa_problem* prob, const void* src, void* dst,
                                 const int32_t* perm_dev, void* stream) {
    return permute_common(prob, src, dst, perm_dev, stream, false);
}

SA_API sa_status hilbert_unpermute(const sa_problem* prob, const void* src, void* dst,
                                   const int32_t* perm_dev, void* stream) {
    return permute_common(prob, src, dst, perm_dev, stream, true);
}

namespace sa {

sa_status check_select_args(const Geometry& g, const sa_select_spec* spec, const void* Q,
                            const void* K, const void* V, const int32_t* row_ptr,
                            const int32_t* col_idx, const float* k_mean, const float* v_sum) {
    (void)g;
    const bool scored = spec->rule != SA_RULE_NONE;
    if (scored && (!Q || !K)) return fail(SA_ERR_INVALID_ARG, "Q and K are required by the rule");
    if ((Q && !aligned16(Q)) || (K && !aligned16(K)) || (V && !aligned16(V)))
        return fail(SA_ERR_INVALID_ARG, "Q, K, V must be 16-byte aligned");
    if (!row_ptr || !col_idx) return fail(SA_ERR_INVALID_ARG, "row_ptr and col_idx are required");
    if (spec->want_comp) {
        if (!K || !V) return fail(SA_ERR_INVALID_ARG, "want_comp needs K and V");
        if (!k_mean || !v_sum) return fail(SA_ERR_INVALID_ARG, "want_comp needs k_mean and v_sum");
    }
    return SA_OK;
}

sa_status select_on_workspace(const Geometry& g, const sa_select_spec& spec, const SelectPlan& plan,
                              const void* Q, const void* K, const void* V, int32_t* row_ptr,
                              int32_t* col_idx, float* scores, float* k_mean, float* v_sum,
                              char* ws, hipStream_t stream) {
    // blocks kept per head, resolved on the host
    int32_t k_host[4096];
    int32_t* kh = k_host;
    std::string kbuf;
    if (g.H > 4096) {
        kbuf.resize((size_t)g.H * sizeof(int32_t));
        kh = (int32_t*)&kbuf[0];
    }
    for (int h = 0; h < g.H; ++h) {
        int64_t k = 0;
        if (spec.rule == SA_RULE_TOPK || spec.rule == SA_RULE_ERR) {
            if (spec.topk) {
                k = spec.topk[h];
            } else {
                k = (int64_t)ceil((double)spec.density[h] * (double)g.nb * (1.0 - 1e-6));
            }
            if (k < 1) k = 1;
            if (k > g.nb) k = g.nb;
        }
        kh[h] = (int32_t)k;
    }
    return launch_select(g, plan, kh, (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V,
                         row_ptr, col_idx, scores, k_mean, v_sum, ws, stream);
}

}  // namespace sa

SA_API sa_status sparse_attn_select(const sa_problem* prob, const sa_select_spec* spec,
                                    const void* Q, const void* K, const void* V,
                                    int32_t* row_ptr, int32_t* col_idx, float* scores,
                                    float* k_mean, float* v_sum, void* workspace,
                                    size_t ws_bytes, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = check_spec(g, spec)) != SA_OK) return st;
    if ((st = check_select_args(g, spec, Q, K, V, row_ptr, col_idx, k_mean, v_sum)) != SA_OK)
        return st;
    const SelectPlan plan = make_select_plan(g, *spec);
    if (plan.total > 0) {
        if (!workspace) return fail(SA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", plan.total);
        if (((uintptr_t)workspace & 255u) != 0)
            return fail(SA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
        if (ws_bytes < plan.total)
            return fail(SA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, plan.total);
    }
    return select_on_workspace(g, *spec, plan, Q, K, V, row_ptr, col_idx, scores, k_mean, v_sum,
                               (char*)workspace, (hipStream_t)stream);
}

SA_API sa_status sparse_attn_centroids(const sa_problem* prob, const void* K, const void* V,
                                       float* k_mean, float* v_sum, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if (!K || !V || !k_mean || !v_sum)
        return fail(SA_ERR_INVALID_ARG, "K, V, k_mean and v_sum are required");
    if (!aligned16(K) || !aligned16(V) || !aligned16(k_mean) || !aligned16(v_sum))
        return fail(SA_ERR_INVALID_ARG, "K, V, k_mean, v_sum must be 16-byte aligned");
    return launch_centroids(g, (const uint16_t*)K, (const uint16_t*)V, k_mean, v_sum,
                            (hipStream_t)stream);
}

static sa_status check_fwd_workspace(const Geometry& g, bool comp, const void* workspace,
                                     size_t ws_bytes) {
    const size_t need = fwd_workspace_bytes(g, comp);
    if (!workspace) return fail(SA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (((uintptr_t)workspace & 255u) != 0)
        return fail(SA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
        return fail(SA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    return SA_OK;
}

SA_API sa_status sparse_attn_fwd_prepare(const sa_problem* prob, const void* V,
                                         const int32_t* row_ptr, const float* k_mean,
                                         const float* v_sum, void* workspace, size_t ws_bytes,
                                         void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    // V == NULL: the workspace already starts with V in block layout
    if (V && !aligned16(V)) return fail(SA_ERR_INVALID_ARG, "V must be 16-byte aligned");
    if (!row_ptr) return fail(SA_ERR_INVALID_ARG, "row_ptr is required");
    if ((k_mean == nullptr) != (v_sum == nullptr))
        return fail(SA_ERR_INVALID_ARG, "k_mean and v_sum must be given together");
    if ((st = check_fwd_workspace(g, k_mean != nullptr, workspace, ws_bytes)) != SA_OK) return st;
    return launch_fwd_prepare(g, (const uint16_t*)V, row_ptr, k_mean, v_sum, nullptr,
                              (char*)workspace, (hipStream_t)stream);
}

SA_API sa_status sparse_attn_fwd_run(const sa_problem* prob, const void* Q, const void* K,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int32_t with_comp, void* O, float* lse, void* workspace,
                                     size_t ws_bytes, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if (!Q || !K || !O) return fail(SA_ERR_INVALID_ARG, "Q, K and O are required");
    if (!aligned16(Q) || !aligned16(K) || !aligned16(O))
        return fail(SA_ERR_INVALID_ARG, "Q, K, O must be 16-byte aligned");
    if (!row_ptr || !col_idx) return fail(SA_ERR_INVALID_ARG, "row_ptr and col_idx are required");
    if (with_comp != 0 && with_comp != 1) return fail(SA_ERR_INVALID_ARG, "with_comp must be 0 or 1");
    if ((st = check_fwd_workspace(g, with_comp != 0, workspace, ws_bytes)) != SA_OK) return st;
    return launch_fwd_run(g, with_comp != 0, (const uint16_t*)Q, (const uint16_t*)K, row_ptr,
                          col_idx, (uint16_t*)O, lse, (char*)workspace, (hipStream_t)stream);
}

SA_API sa_status sparse_attn_fwd(const sa_problem* prob, const void* Q, const void* K,
                                 const void* V, const int32_t* row_ptr,
                                 const int32_t* col_idx, const float* k_mean,
                                 const float* v_sum, void* O, float* lse, void* workspace,
                                 size_t ws_bytes, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if (!Q || !K || !V || !O) return fail(SA_ERR_INVALID_ARG, "Q, K, V and O are required");
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
        return fail(SA_ERR_INVALID_ARG, "Q, K, V, O must be 16-byte aligned");
    if (!row_ptr || !col_idx) return fail(SA_ERR_INVALID_ARG, "row_ptr and col_idx are required");
    if ((k_mean == nullptr) != (v_sum == nullptr))
        return fail(SA_ERR_INVALID_ARG, "k_mean and v_sum must be given together");
    const bool comp = k_mean != nullptr;
    if ((st = check_fwd_workspace(g, comp, workspace, ws_bytes)) != SA_OK) return st;
    st = launch_fwd_prepare(g, (const uint16_t*)V, row_ptr, k_mean, v_sum, nullptr,
                            (char*)workspace, (hipStream_t)stream);
    if (st != SA_OK) return st;
    return launch_fwd_run(g, comp, (const uint16_t*)Q, (const uint16_t*)K, row_ptr, col_idx,
                          (uint16_t*)O, lse, (char*)workspace, (hipStream_t)stream);
}

SA_API sa_status sparse_attn_fwd_prepare_counts(const sa_problem* prob, const void* V,
                                                const int32_t* row_ptr, const float* k_mean,
                                                const float* v_sum, const int32_t* kv_count,
                                                void* workspace, size_t ws_bytes, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = no_token_order(g, "sparse_attn_fwd_prepare_counts")) != SA_OK) return st;
    if (!V) return fail(SA_ERR_INVALID_ARG, "V is required");
    if (!aligned16(V)) return fail(SA_ERR_INVALID_ARG, "V must be 16-byte aligned");
    if (!row_ptr) return fail(SA_ERR_INVALID_ARG, "row_ptr is required");
    if (!kv_count) return fail(SA_ERR_INVALID_ARG, "kv_count is required");
    if ((k_mean == nullptr) != (v_sum == nullptr))
        return fail(SA_ERR_INVALID_ARG, "k_mean and v_sum must be given together");
    if ((st = check_fwd_workspace(g, k_mean != nullptr, workspace, ws_bytes)) != SA_OK) return st;
    return launch_fwd_prepare(g, (const uint16_t*)V, row_ptr, k_mean, v_sum, kv_count,
                              (char*)workspace, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// data-dependent block formation
// ---------------------------------------------------------------------------
static sa_status check_cluster(const Geometry& g, const sa_cluster_spec* cs) {
    if (!cs) return fail(SA_ERR_INVALID_ARG, "cspec is NULL");
    if (cs->mode != SA_CLUSTER_COCLUSTER && cs->mode != SA_CLUSTER_KMEANS &&
        cs->mode != SA_CLUSTER_TILES)
        return fail(SA_ERR_INVALID_ARG, "unknown cluster mode %d", cs->mode);
    if (cs->mode == SA_CLUSTER_TILES) {
        if (cs->n_shapes < 1 || cs->n_shapes > 16 || !cs->shapes)
            return fail(SA_ERR_INVALID_ARG, "a menu of 1 to 16 tile shapes is required (got %d)",
                        cs->n_shapes);
        for (int s = 0; s < cs->n_shapes; ++s) {
            const sa_tile_shape sh = cs->shapes[s];
            if (sh.t < 1 || sh.y < 1 || sh.x < 1)
                return fail(SA_ERR_INVALID_ARG, "tile shape %d has a side < 1", s);
            if ((int64_t)sh.t * sh.y * sh.x > g.block)
                return fail(SA_ERR_INVALID_ARG, "tile shape %d holds %lld tokens > block = %d", s,
                            (long long)sh.t * sh.y * sh.x, g.block);
        }
        const int mt = menu_max_tiles(g, *cs);
        if (mt > 1024)
            return fail(SA_ERR_UNSUPPORTED, "the menu cuts the grid into %d tiles (at most 1024)", mt);
        if (cs->n_clusters != mt)
            return fail(SA_ERR_INVALID_ARG, "n_clusters = %d must be the menu's largest tile count %d",
                        cs->n_clusters, mt);
        if (cs->tile_coherence && !(cs->ticket >= -1.f && cs->ticket <= 1.f))
            return fail(SA_ERR_INVALID_ARG, "ticket = %g must be in [-1, 1]", (double)cs->ticket);
        if (((uintptr_t)cs->tile_coherence & 7u) != 0 || ((uintptr_t)cs->shape_idx & 3u) != 0)
            return fail(SA_ERR_INVALID_ARG, "tile_coherence must be 8-byte and shape_idx 4-byte aligned");
    } else {
        const int cmax = g.N < 1024 ? g.N : 1024;
        if (cs->n_clusters < 1 || cs->n_clusters > cmax)
            return fail(SA_ERR_INVALID_ARG, "n_clusters = %d must be in [1, %d]", cs->n_clusters, cmax);
        if (cs->iters < 1 || cs->iters > 64)
            return fail(SA_ERR_INVALID_ARG, "iters = %d must be in [1, 64]", cs->iters);
    }
    const int64_t nbp = padded_block_count(g, *cs);
    if (nbp > 4096)
        return fail(SA_ERR_UNSUPPORTED, "padded layout of %lld blocks (attention supports <= 4096)",
                    (long long)nbp);
    if (g.BH() * nbp * nbp > (int64_t)INT32_MAX)
        return fail(SA_ERR_UNSUPPORTED, "B*H*nbp*nbp exceeds the int32 range of row_ptr");
    return SA_OK;
}

static sa_status check_ws(size_t need, const void* workspace, size_t ws_bytes) {
    if (need == 0) return SA_OK;
    if (!workspace) return fail(SA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (((uintptr_t)workspace & 255u) != 0)
        return fail(SA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (ws_bytes < need)
        return fail(SA_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
    return SA_OK;
}

SA_API sa_status sparse_attn_cluster_size(const sa_problem* prob, const sa_cluster_spec* cspec,
                                          int32_t* nb_padded, size_t* ws_cluster,
                                          size_t* ws_select) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = no_token_order(g, "sparse_attn_cluster_size")) != SA_OK) return st;
    if ((st = check_cluster(g, cspec)) != SA_OK) return st;
    if (nb_padded) *nb_padded = padded_block_count(g, *cspec);
    if (ws_cluster) *ws_cluster = cluster_workspace_bytes(g, *cspec);
    if (ws_select) *ws_select = cluster_select_workspace_bytes(g, *cspec);
    return SA_OK;
}

SA_API sa_status sparse_attn_cluster(const sa_problem* prob, const sa_cluster_spec* cspec,
                                     const void* Q, const void* K, const void* V,
                                     int32_t* q_order, int32_t* k_order, int32_t* q_blk,
                                     int32_t* k_blk, int32_t* q_cnt, int32_t* k_cnt,
                                     float* q_cent, float* k_cent, float* v_cent,
                                     int32_t* q_count, int32_t* k_count, void* workspace,
                                     size_t ws_bytes, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = no_token_order(g, "sparse_attn_cluster")) != SA_OK) return st;
    if ((st = check_cluster(g, cspec)) != SA_OK) return st;
    if (!Q || !K) return fail(SA_ERR_INVALID_ARG, "Q and K are required");
    if (!aligned16(Q) || !aligned16(K) || (V && !aligned16(V)))
        return fail(SA_ERR_INVALID_ARG, "Q, K, V must be 16-byte aligned");
    if ((V == nullptr) != (v_cent == nullptr))
        return fail(SA_ERR_INVALID_ARG, "V and v_cent must be given together");
    if (!q_order || !k_order || !q_blk || !k_blk || !q_cnt || !k_cnt || !q_cent || !k_cent ||
        !q_count || !k_count)
        return fail(SA_ERR_INVALID_ARG, "every output except v_cent is required");
    if (cspec->mode == SA_CLUSTER_TILES && !cspec->shape_idx)
        return fail(SA_ERR_INVALID_ARG, "SA_CLUSTER_TILES needs shape_idx");
    if ((st = check_ws(cluster_workspace_bytes(g, *cspec), workspace, ws_bytes)) != SA_OK)
        return st;
    ClusterOut o{q_order, k_order, q_blk, k_blk, q_cnt, k_cnt, q_cent, k_cent, v_cent,
                 q_count, k_count};
    return launch_cluster(g, *cspec, (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V,
                          o, (char*)workspace, (hipStream_t)stream);
}

SA_API sa_status sparse_attn_sics(const sa_problem* prob, const sa_cluster_spec* cspec,
                                  const void* Q, const void* K, double* scores,
                                  int32_t* shape_idx, void* workspace, size_t ws_bytes,
                                  void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = no_token_order(g, "sparse_attn_sics")) != SA_OK) return st;
    if ((st = check_cluster(g, cspec)) != SA_OK) return st;
    if (cspec->mode != SA_CLUSTER_TILES)
        return fail(SA_ERR_INVALID_ARG, "sparse_attn_sics needs mode SA_CLUSTER_TILES");
    if (!Q || !K || !shape_idx) return fail(SA_ERR_INVALID_ARG, "Q, K and shape_idx are required");
    if (!aligned16(Q) || !aligned16(K)) return fail(SA_ERR_INVALID_ARG, "Q, K must be 16-byte aligned");
    if ((st = check_ws(sics_workspace_bytes(g, *cspec), workspace, ws_bytes)) != SA_OK) return st;
    return launch_sics(g, *cspec, (const uint16_t*)Q, (const uint16_t*)K, scores, shape_idx,
                       (char*)workspace, (hipStream_t)stream);
}

static sa_status check_rows(const Geometry& g, const void* src, void* dst, int64_t src_rows,
                            int64_t dst_rows) {
    if (!src || !dst) return fail(SA_ERR_INVALID_ARG, "src and dst are required");
    if (!aligned16(src) || !aligned16(dst))
        return fail(SA_ERR_INVALID_ARG, "src and dst must be 16-byte aligned");
    const char* s = (const char*)src;
    const char* d = (const char*)dst;
    const size_t sb = (size_t)g.BH() * src_rows * g.d * 2, db = (size_t)g.BH() * dst_rows * g.d * 2;
    if (s < d + db && d < s + sb) return fail(SA_ERR_INVALID_ARG, "src and dst overlap");
    return SA_OK;
}

SA_API sa_status sparse_attn_cluster_gather(const sa_problem* prob, const sa_cluster_spec* cspec,
                                            const int32_t* order, const void* src, void* dst,
                                            void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = no_token_order(g, "sparse_attn_cluster_gather")) != SA_OK) return st;
    if ((st = check_cluster(g, cspec)) != SA_OK) return st;
    if (!order) return fail(SA_ERR_INVALID_ARG, "order is required");
    const int64_t np = (int64_t)padded_block_count(g, *cspec) * g.block;
    if ((st = check_rows(g, src, dst, g.N, np)) != SA_OK) return st;
    return launch_cluster_gather(g, *cspec, order, (const uint16_t*)src,
                                 (uint16_t*)dst, (hipStream_t)stream);
}

SA_API sa_status sparse_attn_cluster_scatter(const sa_problem* prob, const sa_cluster_spec* cspec,
                                             const int32_t* order, const void* src, void* dst,
                                             const float* lse_src, float* lse_dst, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = no_token_order(g, "sparse_attn_cluster_scatter")) != SA_OK) return st;
    if ((st = check_cluster(g, cspec)) != SA_OK) return st;
    if (!order) return fail(SA_ERR_INVALID_ARG, "order is required");
    if ((lse_src == nullptr) != (lse_dst == nullptr))
        return fail(SA_ERR_INVALID_ARG, "lse_src and lse_dst must be given together");
    const int64_t np = (int64_t)padded_block_count(g, *cspec) * g.block;
    if ((st = check_rows(g, src, dst, np, g.N)) != SA_OK) return st;
    return launch_cluster_scatter(g, *cspec, order, (const uint16_t*)src,
                                  (uint16_t*)dst, lse_src, lse_dst, (hipStream_t)stream);
}

SA_API sa_status sparse_attn_cluster_fwd_prepare(const sa_problem* prob,
                                                 const sa_cluster_spec* cspec,
                                                 const int32_t* k_order, const void* V,
                                                 const int32_t* row_ptr, const float* k_mean,
                                                 const float* v_sum, const int32_t* kv_count,
                                                 void* workspace, size_t ws_bytes, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = no_token_order(g, "sparse_attn_cluster_fwd_prepare")) != SA_OK) return st;
    if ((st = check_cluster(g, cspec)) != SA_OK) return st;
    if (!k_order || !V) return fail(SA_ERR_INVALID_ARG, "k_order and V are required");
    if (!aligned16(V)) return fail(SA_ERR_INVALID_ARG, "V must be 16-byte aligned");
    if (!row_ptr) return fail(SA_ERR_INVALID_ARG, "row_ptr is required");
    if (!kv_count) return fail(SA_ERR_INVALID_ARG, "kv_count is required");
    if ((k_mean == nullptr) != (v_sum == nullptr))
        return fail(SA_ERR_INVALID_ARG, "k_mean and v_sum must be given together");
    sa_problem pp = *prob;
    pp.N = padded_block_count(g, *cspec) * g.block;
    pp.T = 1;
    pp.Hg = 1;
    pp.W = pp.N;
    pp.token_order = nullptr;
    Geometry gp;
    if ((st = check_problem(&pp, &gp)) != SA_OK) return st;
    if ((st = check_fwd_workspace(gp, k_mean != nullptr, workspace, ws_bytes)) != SA_OK) return st;
    return launch_fwd_prepare(gp, (const uint16_t*)V, row_ptr, k_mean, v_sum, kv_count,
                              (char*)workspace, (hipStream_t)stream, k_order, g.N);
}

SA_API sa_status sparse_attn_cluster_fwd_run(const sa_problem* prob, const sa_cluster_spec* cspec,
                                             const int32_t* q_order, const void* Q, const void* Kp,
                                             const int32_t* row_ptr, const int32_t* col_idx,
                                             int32_t with_comp, void* O, float* lse,
                                             void* workspace, size_t ws_bytes, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = no_token_order(g, "sparse_attn_cluster_fwd_run")) != SA_OK) return st;
    if ((st = check_cluster(g, cspec)) != SA_OK) return st;
    if (!q_order || !Q || !Kp || !O) return fail(SA_ERR_INVALID_ARG, "q_order, Q, Kp and O are required");
    if (!aligned16(Q) || !aligned16(Kp) || !aligned16(O))
        return fail(SA_ERR_INVALID_ARG, "Q, Kp, O must be 16-byte aligned");
    if (!row_ptr || !col_idx) return fail(SA_ERR_INVALID_ARG, "row_ptr and col_idx are required");
    if (with_comp != 0 && with_comp != 1) return fail(SA_ERR_INVALID_ARG, "with_comp must be 0 or 1");
    // the attention problem of the padded layout: one flat frame of nbp blocks
    sa_problem pp = *prob;
    pp.N = padded_block_count(g, *cspec) * g.block;
    pp.T = 1;
    pp.Hg = 1;
    pp.W = pp.N;
    pp.token_order = nullptr;
    Geometry gp;
    if ((st = check_problem(&pp, &gp)) != SA_OK) return st;
    if ((st = check_fwd_workspace(gp, with_comp != 0, workspace, ws_bytes)) != SA_OK) return st;
    return launch_fwd_run_mapped(gp, with_comp != 0, (const uint16_t*)Q, (const uint16_t*)Kp, row_ptr,
                                 col_idx, q_order, g.N, (uint16_t*)O, lse, (char*)workspace,
                                 (hipStream_t)stream);
}

SA_API sa_status sparse_attn_cluster_select(const sa_problem* prob, const sa_cluster_spec* cspec,
                                            const sa_select_spec* spec, const float* q_cent,
                                            const float* k_cent, const float* v_cent,
                                            const int32_t* k_count, const int32_t* q_blk,
                                            const int32_t* k_blk, const int32_t* k_cnt,
                                            int32_t* row_ptr, int32_t* col_idx, float* scores,
                                            float* k_mean, float* v_sum, void* workspace,
                                            size_t ws_bytes, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = no_token_order(g, "sparse_attn_cluster_select")) != SA_OK) return st;
    if ((st = check_cluster(g, cspec)) != SA_OK) return st;
    if (!spec) return fail(SA_ERR_INVALID_ARG, "spec is NULL");
    if (spec->rule != SA_RULE_TOPK && spec->rule != SA_RULE_MASS)
        return fail(SA_ERR_UNSUPPORTED, "cluster selection supports SA_RULE_TOPK and SA_RULE_MASS");
    if (spec->sub_block != 0 || spec->window_frames != -1 || spec->n_anchors != 0)
        return fail(SA_ERR_UNSUPPORTED,
                    "cluster selection has no sub-blocks, windows or anchors (sub_block = 0, "
                    "window_frames = -1, n_anchors = 0)");
    if (spec->diag != 0 && spec->diag != 1) return fail(SA_ERR_INVALID_ARG, "diag must be 0 or 1");
    if (spec->want_comp != 0 && spec->want_comp != 1)
        return fail(SA_ERR_INVALID_ARG, "want_comp must be 0 or 1");
    if (spec->rule == SA_RULE_TOPK) {
        if (spec->topk) return fail(SA_ERR_UNSUPPORTED, "cluster top-k takes density, not topk");
        if (!spec->density) return fail(SA_ERR_INVALID_ARG, "SA_RULE_TOPK needs density");
        for (int h = 0; h < g.H; ++h)
            if (!(spec->density[h] > 0.f && spec->density[h] <= 1.f))
                return fail(SA_ERR_INVALID_ARG, "density[%d] = %g must be in (0, 1]", h,
                            (double)spec->density[h]);
    } else if (!(spec->mass > 0.f && spec->mass <= 1.f)) {
        return fail(SA_ERR_INVALID_ARG, "mass = %g must be in (0, 1]", (double)spec->mass);
    }
    if (cspec->mode == SA_CLUSTER_TILES && cspec->tile_coherence && !cspec->shape_idx)
        return fail(SA_ERR_INVALID_ARG, "a SICS ticket needs shape_idx (the chosen shapes)");
    if (!q_cent || !k_cent || !k_count || !q_blk || !k_blk || !k_cnt || !row_ptr || !col_idx)
        return fail(SA_ERR_INVALID_ARG, "q_cent, k_cent, k_count, q_blk, k_blk, k_cnt, row_ptr "
                                        "and col_idx are required");
    if (spec->want_comp && (!v_cent || !k_mean || !v_sum))
        return fail(SA_ERR_INVALID_ARG, "want_comp needs v_cent, k_mean and v_sum");
    const int C = cspec->n_clusters;
    if ((st = check_ws(cluster_select_workspace_bytes(g, *cspec), workspace, ws_bytes)) != SA_OK)
        return st;
    std::string bbuf((size_t)g.H * sizeof(int64_t), '\0');
    int64_t* budget = (int64_t*)&bbuf[0];
    for (int h = 0; h < g.H; ++h) {
        int64_t b = 0;
        if (spec->rule == SA_RULE_TOPK)
            b = (int64_t)ceil((double)spec->density[h] * (double)g.N * (1.0 - 1e-6));
        budget[h] = b < 1 ? 1 : b;
    }
    ClusterSel a{};
    a.q_cent = q_cent; a.k_cent = k_cent; a.v_cent = v_cent;
    a.k_count = k_count; a.q_blk = q_blk; a.k_blk = k_blk; a.k_cnt = k_cnt;
    a.row_ptr = row_ptr; a.col_idx = col_idx; a.scores = scores;
    a.k_mean = spec->want_comp ? k_mean : nullptr;
    a.v_sum = spec->want_comp ? v_sum : nullptr;
    a.rule = spec->rule; a.diag = spec->diag; a.mass = spec->mass;
    return launch_cluster_select(g, *cspec, a, budget, (char*)workspace, (hipStream_t)stream);
}

SA_API sa_status sparse_attn_cluster_centroids(const sa_problem* prob, const sa_cluster_spec* cspec,
                                               const void* Kp, const void* Vp,
                                               const int32_t* k_count, const int32_t* k_blk,
                                               const int32_t* k_cnt, float* k_cent, float* v_cent,
                                               float* k_mean, float* v_sum, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = no_token_order(g, "sparse_attn_cluster_centroids")) != SA_OK) return st;
    if ((st = check_cluster(g, cspec)) != SA_OK) return st;
    if (!Kp || !Vp || !k_count || !k_blk || !k_cnt || !k_cent || !v_cent || !k_mean || !v_sum)
        return fail(SA_ERR_INVALID_ARG, "every argument is required");
    if (!aligned16(Kp) || !aligned16(Vp))
        return fail(SA_ERR_INVALID_ARG, "Kp and Vp must be 16-byte aligned");
    return launch_cluster_centroids(g, *cspec, (const uint16_t*)Kp, (const uint16_t*)Vp,
                                    k_count, k_blk, k_cnt, k_cent, v_cent, k_mean, v_sum,
                                    (hipStream_t)stream);
}

SA_API const char* sparse_attn_last_error(void) { return g_last_error.c_str(); }
