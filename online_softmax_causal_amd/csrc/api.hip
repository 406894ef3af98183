// C ABI of libosc_attn.so (declared in include/osc_attn.h): argument
// validation, then one asynchronous kernel launch on the caller's stream.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "osc_attn.h"
#include "validate.hpp"

namespace osc {

// Decode split plan and segment-state bytes for valid sizes; false (with the
// status to report) if they are not.
bool paged_decode_plan_checked(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                               int64_t num_pages, int64_t max_pages, int num_splits,
                               attn_status_t* status, int* log2_page, DecodePlan* plan,
                               int64_t* bytes) {
    if (!paged_sizes_ok(B, Hq, Hkv, D, page_size, num_pages, max_pages, status, log2_page))
        return false;
    *status = ATTN_ERR_SHAPE;
    if (num_splits < 0 || num_splits > PAGED_MAX_SPLITS) return false;
    *plan = paged_decode_plan(B, Hkv, max_pages * page_size, num_splits);
    if (B * Hkv * plan->nseg >= (int64_t(1) << 31)) return false;
    int64_t words = 0;
    if (!mul_below_2_62(B * Hq * (D + 2), plan->nseg, &words) || words >= (int64_t(1) << 60))
        return false;
    *bytes = plan->nseg > 1 ? words * 4 : 0;
    return true;
}

}  // namespace osc

extern "C" {

static attn_status_t attn_fwd_impl(const void* q, const void* k, const void* v, float* o,
                                   float* lse, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                                   int64_t D, int causal, attn_dtype_t dtype, hipStream_t stream) {
    const attn_status_t st = osc::validate_attn(q, k, v, o, lse, B, H, Hkv, N, D, dtype);
    if (st != ATTN_OK) return st;
    const int waves = osc::attn_pick_waves(B * H, N);
    const hipError_t e = osc::launch_attn_fwd(q, k, v, o, lse, (int)B, (int)H, (int)Hkv, (int)N,
                                              (int)D, causal != 0, dtype == ATTN_BF16, waves,
                                              nullptr, nullptr, nullptr, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

// Split plan and workspace size for valid sizes; false if they are not.
static bool splitkv_plan(int64_t B, int64_t H, int64_t N, int64_t D, int causal, int num_splits,
                         osc::SplitPlan* plan, int64_t* bytes) {
    if (B < 1 || H < 1 || N < 1 || (D != 64 && D != 128)) return false;
    if (num_splits < 0 || num_splits > ATTN_MAX_SPLITS) return false;
    int64_t bh = 0, bhn = 0, total = 0;
    if (!osc::mul_below_2_62(B, H, &bh) || !osc::mul_below_2_62(bh, N, &bhn) ||
        !osc::mul_below_2_62(bhn, D + 2, &total) || N * D >= (int64_t(1) << 31) ||
        bh >= (int64_t(1) << 31))
        return false;
    *plan = osc::attn_plan_split(bh, N, causal != 0, num_splits);
    int64_t words = 0;
    if (!osc::mul_below_2_62(total, plan->nseg, &words) || words >= (int64_t(1) << 60)) return false;
    // One workgroup per (query tile of at least 128 rows, head, segment).
    if (bh * ((N + 127) / 128) * plan->nseg >= (int64_t(1) << 31)) return false;
    *bytes = osc::splitkv_workspace_bytes(*plan, bh, N, D);
    return true;
}

int64_t attn_fwd_splitkv_workspace(int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                                   int num_splits) {
    osc::SplitPlan plan;
    int64_t bytes = 0;
    return splitkv_plan(B, H, N, D, causal, num_splits, &plan, &bytes) ? bytes : -1;
}

attn_status_t attn_fwd_splitkv(const void* q, const void* k, const void* v, float* o, float* lse,
                               int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal,
                               attn_dtype_t dtype, int num_splits, void* workspace,
                               int64_t workspace_bytes, hipStream_t stream) {
    attn_status_t st = osc::validate_attn(q, k, v, o, lse, B, H, Hkv, N, D, dtype);
    if (st != ATTN_OK) return st;
    osc::SplitPlan plan;
    int64_t need = 0;
    if (!splitkv_plan(B, H, N, D, causal, num_splits, &plan, &need)) return ATTN_ERR_SHAPE;
    st = osc::validate_workspace(workspace, workspace_bytes, need, q, k, v, o, lse, B, H, Hkv, N, D);
    if (st != ATTN_OK) return st;
    float* part_o = static_cast<float*>(workspace);
    float2* part_ml = plan.nseg > 1 ? reinterpret_cast<float2*>(part_o + plan.nseg * B * H * N * D)
                                    : nullptr;
    const hipError_t e = osc::launch_attn_fwd(q, k, v, o, lse, (int)B, (int)H, (int)Hkv, (int)N,
                                              (int)D, causal != 0, dtype == ATTN_BF16, plan.waves,
                                              &plan, part_o, part_ml, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                       int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                       attn_dtype_t dtype, hipStream_t stream) {
    return attn_fwd_impl(q, k, v, o, lse, B, H, H, N, D, causal, dtype, stream);
}

attn_status_t attn_fwd_gqa(const void* q, const void* k, const void* v, float* o, float* lse,
                           int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal,
                           attn_dtype_t dtype, hipStream_t stream) {
    return attn_fwd_impl(q, k, v, o, lse, B, H, Hkv, N, D, causal, dtype, stream);
}

int64_t attn_bwd_workspace(int64_t B, int64_t H, int64_t N) {
    int64_t bh = 0, rows = 0;
    if (B < 1 || H < 1 || N < 1 || !osc::mul_below_2_62(B, H, &bh) ||
        !osc::mul_below_2_62(bh, N, &rows) || rows >= (int64_t(1) << 58))
        return -1;
    return 8 * rows;
}

attn_status_t attn_bwd_gqa(const void* q, const void* k, const void* v, const float* o,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal,
                           attn_dtype_t dtype, void* workspace, int64_t workspace_bytes,
                           hipStream_t stream) {
    // validate_attn checks q, k, v and the FP32 pair (o, lse) as inputs here.
    attn_status_t st = osc::validate_attn(q, k, v, o, lse, B, H, Hkv, N, D, dtype);
    if (st != ATTN_OK) return st;
    st = osc::validate_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, B, H,
                           Hkv, N, D);
    if (st != ATTN_OK) return st;
    const hipError_t e = osc::launch_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv,
                                              static_cast<float*>(workspace), (int)B, (int)H,
                                              (int)Hkv, (int)N, (int)D, causal != 0,
                                              dtype == ATTN_BF16, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t attn_bwd(const void* q, const void* k, const void* v, const float* o,
                       const float* lse, const void* dout, float* dq, float* dk, float* dv,
                       int64_t B, int64_t H, int64_t N, int64_t D, int causal, attn_dtype_t dtype,
                       void* workspace, int64_t workspace_bytes, hipStream_t stream) {
    return attn_bwd_gqa(q, k, v, o, lse, dout, dq, dk, dv, B, H, H, N, D, causal, dtype, workspace,
                        workspace_bytes, stream);
}


int64_t paged_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                               int64_t max_pages, int num_splits) {
    attn_status_t st;
    int lp = 0;
    osc::DecodePlan plan;
    int64_t bytes = 0;
    // The cache size does not enter the plan; one page stands in for it.
    return osc::paged_decode_plan_checked(B, Hq, Hkv, D, page_size, 1, max_pages, num_splits, &st,
                                           &lp, &plan, &bytes)
               ? bytes
               : -1;
}

attn_status_t paged_decode(const void* q, const void* cache, const int32_t* block_table,
                           const int32_t* lengths, float* o, float* lse, int64_t B, int64_t Hq,
                           int64_t Hkv, int64_t D, int64_t page_size, int64_t num_pages,
                           int64_t max_pages, attn_dtype_t dtype, int num_splits, void* workspace,
                           int64_t workspace_bytes, hipStream_t stream) {
    attn_status_t st = ATTN_OK;
    int lp = 0;
    osc::DecodePlan plan;
    int64_t need = 0;
    if (!osc::paged_decode_plan_checked(B, Hq, Hkv, D, page_size, num_pages, max_pages,
                                        num_splits, &st, &lp, &plan, &need)) {
        // A null pointer is reported before a size problem, as for attention.
        if (!q || !cache || !block_table || !lengths || !o || !lse) return ATTN_ERR_NULL;
        return st;
    }
    st = osc::validate_paged(q, cache, block_table, lengths, o, lse, B, Hq, Hkv, D, page_size,
                             num_pages, max_pages, dtype);
    if (st != ATTN_OK) return st;
    st = osc::validate_paged_workspace(workspace, workspace_bytes, need, q, cache, block_table,
                                       lengths, o, lse, B, Hq, Hkv, D, page_size, num_pages,
                                       max_pages);
    if (st != ATTN_OK) return st;
    float* part_o = static_cast<float*>(workspace);
    float2* part_ml =
        plan.nseg > 1 ? reinterpret_cast<float2*>(part_o + (int64_t)plan.nseg * B * Hq * D) : nullptr;
    const hipError_t e = osc::launch_paged_decode(
        q, cache, block_table, lengths, o, lse, (int)B, (int)Hq, (int)Hkv, (int)D, lp,
        (int)num_pages, (int)max_pages, dtype == ATTN_BF16, plan, part_o, part_ml, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

attn_status_t row_softmax(const float* x, float* y, int64_t M, int64_t N, hipStream_t stream) {
    const attn_status_t st = osc::validate_softmax(x, y, M, N);
    if (st != ATTN_OK) return st;
    const hipError_t e = osc::launch_row_softmax(x, y, M, N, stream);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

const char* attn_status_str(attn_status_t status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "a size is < 1 or the sizes exceed the supported limits";
        case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
        case ATTN_ERR_ALIGN: return "a pointer is not aligned as required";
        case ATTN_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
        case ATTN_ERR_ALIAS: return "an output buffer overlaps an input buffer";
        case ATTN_ERR_WORKSPACE: return "the workspace is smaller than the call needs";
    }
    return "unknown status";
}

}  // extern "C"
