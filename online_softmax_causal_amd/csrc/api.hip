// C ABI of libosc_attn.so (declared in include/osc_attn.h): argument
// validation, then one asynchronous kernel launch on the caller's stream.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "osc_attn.h"
#include "validate.hpp"

extern "C" {

static attn_status_t attn_fwd_impl(const void* q, const void* k, const void* v, float* o,
                                   float* lse, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                                   int64_t D, int causal, attn_dtype_t dtype, hipStream_t stream) {
    const attn_status_t st = osc::validate_attn(q, k, v, o, lse, B, H, Hkv, N, D, dtype);
    if (st != ATTN_OK) return st;
    const int waves = osc::attn_pick_waves(B * H, N);
    const hipError_t e = osc::launch_attn_fwd(q, k, v, o, lse, (int)B, (int)H, (int)Hkv, (int)N,
                                              (int)D, causal != 0, dtype == ATTN_BF16, waves, stream);
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
    }
    return "unknown status";
}

}  // extern "C"
