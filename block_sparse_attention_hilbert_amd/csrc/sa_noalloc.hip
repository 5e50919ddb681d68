// sparse_attn_select_noalloc: the block selection of sparse_attn_select with
// its scratch (pooled means, scores, keep bitmap, per-row counts) taken from a
// fixed device array of this library instead of a caller's workspace, for
// callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  The array is kScratchBytes per
// GPU, reserved when the library's code object is loaded on that GPU and
// held until the process ends.
#include <mutex>

#include "sa_internal.h"

#define SA_API extern "C" __attribute__((visibility("default")))

namespace sa {
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;     // 64 MiB per GPU
constexpr int kMaxDevices = 64;

// The scratch itself.  In host code this name is only a stand-in for the
// device symbol: its device address comes from hipGetSymbolAddress, once per
// device (each GPU holds its own copy at its own address).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array, looked up on the first call on
// the device (with that device current) and kept.
sa_status scratch_for_current_device(char** out) {
    int dev = 0;
    sa_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
    if (st != SA_OK) return st;
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        st = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch symbol address");
        if (st != SA_OK) return st;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<char*>(g_scratch_ptr[dev]);
    return SA_OK;
}

}  // namespace
}  // namespace sa

using namespace sa;

SA_API sa_status sparse_attn_select_noalloc(const sa_problem* prob, const sa_select_spec* spec,
                                            const void* Q, const void* K, const void* V,
                                            int32_t* row_ptr, int32_t* col_idx, float* scores,
                                            float* k_mean, float* v_sum, void* stream) {
    clear_error();
    Geometry g;
    sa_status st = check_problem(prob, &g);
    if (st != SA_OK) return st;
    if ((st = check_spec(g, spec)) != SA_OK) return st;
    if ((st = check_select_args(g, spec, Q, K, V, row_ptr, col_idx, k_mean, v_sum)) != SA_OK)
        return st;
    const SelectPlan plan = make_select_plan(g, *spec);
    if (plan.total > kScratchBytes)
        return fail(SA_ERR_UNSUPPORTED,
                    "this selection needs %zu bytes of scratch; the allocation-free entry point "
                    "holds at most %zu (use sparse_attn_select with a workspace)",
                    plan.total, kScratchBytes);
    char* ws = nullptr;
    if ((st = scratch_for_current_device(&ws)) != SA_OK) return st;
    return select_on_workspace(g, *spec, plan, Q, K, V, row_ptr, col_idx, scores, k_mean, v_sum,
                               ws, (hipStream_t)stream);
}
