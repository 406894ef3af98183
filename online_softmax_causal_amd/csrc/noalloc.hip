// paged_decode_noalloc (declared in include/osc_attn.h): paged decode whose
// segment states live in a fixed array of this library instead of a caller's
// workspace, for callers that cannot allocate device memory.  Validation and
// kernels are those of paged_decode.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.hpp"
#include "osc_attn.h"
#include "validate.hpp"

// Segment states (partial o, then (m, l)) of paged_decode_noalloc.  Every
// device the library runs on holds its own copy for the life of the process.
// Host code never passes this name to a kernel or a copy: on the host it is
// a stand-in, not a device address.  The address comes from
// hipGetSymbolAddress, once per device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[PAGED_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's `scratch`, looked up on the first
// call on that device (with the device current) and kept.
hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

attn_status_t paged_decode_noalloc(const void* q, const void* cache, const int32_t* block_table,
                                   const int32_t* lengths, float* o, float* lse, int64_t B,
                                   int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                                   int64_t num_pages, int64_t max_pages, attn_dtype_t dtype,
                                   int num_splits, hipStream_t stream) {
    attn_status_t st = ATTN_OK;
    int lp = 0;
    osc::DecodePlan plan;
    int64_t need = 0;
    if (!osc::paged_decode_plan_checked(B, Hq, Hkv, D, page_size, num_pages, max_pages,
                                        num_splits, &st, &lp, &plan, &need)) {
        if (!q || !cache || !block_table || !lengths || !o || !lse) return ATTN_ERR_NULL;
        return st;
    }
    st = osc::validate_paged(q, cache, block_table, lengths, o, lse, B, Hq, Hkv, D, page_size,
                             num_pages, max_pages, dtype);
    if (st != ATTN_OK) return st;
    if (need > PAGED_NOALLOC_SCRATCH_BYTES) return ATTN_ERR_WORKSPACE;
    void* base = nullptr;
    if (scratch_address(&base) != hipSuccess) return ATTN_ERR_LAUNCH;
    // Each segment's kernel workgroup writes its whole state (an empty
    // segment writes m = -inf, l = 0, o = 0) before the merge reads it, so
    // nothing needs clearing between calls.
    float* part_o = static_cast<float*>(base);
    float2* part_ml =
        plan.nseg > 1 ? reinterpret_cast<float2*>(part_o + (int64_t)plan.nseg * B * Hq * D) : nullptr;
    const hipError_t e = osc::launch_paged_decode(
        q, cache, block_table, lengths, o, lse, (int)B, (int)Hq, (int)Hkv, (int)D, lp,
        (int)num_pages, (int)max_pages, dtype == ATTN_BF16, plan, part_o, part_ml, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // extern "C"
