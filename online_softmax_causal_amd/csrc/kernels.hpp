// Launch entry points of the HIP kernels, called by the C ABI layer after it
// has validated the arguments.  Each returns the status of hipLaunchKernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace osc {

// Waves per workgroup (4 or 8) for a problem of BH heads of N rows.
int attn_pick_waves(int64_t BH, int64_t N);

// q, o, lse: B*H heads; k, v: B*Hkv heads, query head h reads K/V head h / (H / Hkv).
hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                           int B, int H, int Hkv, int N, int D, bool causal, bool bf16, int waves,
                           hipStream_t stream);

hipError_t launch_row_softmax(const float* x, float* y, int64_t M, int64_t N, hipStream_t stream);

}  // namespace osc
