// Launch entry points of the HIP kernels, called by the C ABI layer after it
// has validated the arguments.  Each returns the status of hipLaunchKernel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "osc_attn.h"

namespace osc {

// Waves per workgroup (4 or 8) for a problem of BH heads of N rows.
int attn_pick_waves(int64_t BH, int64_t N);

// A split of every head's keys into nseg segments of seg_tiles 64-key tiles.
struct SplitPlan {
    int nseg;       // segments (1: no split)
    int seg_tiles;  // tiles per segment, a multiple of 4
    int waves;      // waves per workgroup of the attention kernel
};

// Segments for a key split; requested = 0 chooses automatically.
SplitPlan attn_plan_split(int64_t BH, int64_t N, bool causal, int requested);

// Bytes of workspace a split needs: the partial output and (m, l) per segment.
inline int64_t splitkv_workspace_bytes(const SplitPlan& p, int64_t BH, int64_t N, int64_t D) {
    return p.nseg <= 1 ? 0 : (int64_t)p.nseg * BH * N * (D + 2) * 4;
}

// q, o, lse: B*H heads; k, v: B*Hkv heads, query head h reads K/V head h / (H / Hkv).
// With split->nseg > 1, part_o [nseg, B*H, N, D] and part_ml [nseg, B*H, N]
// receive the segments' states and a second kernel merges them into o, lse.
hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                           int B, int H, int Hkv, int N, int D, bool causal, bool bf16, int waves,
                           const SplitPlan* split, float* part_o, float2* part_ml,
                           hipStream_t stream);

// o, lse of every row from the states of its live segments (key segments of
// seg_rows keys; with causal masking row i has floor(i / seg_rows) + 1).
hipError_t launch_splitkv_merge(const float* part_o, const float2* part_ml, float* o, float* lse,
                                int BH, int N, int D, int nseg, int seg_rows, bool causal,
                                hipStream_t stream);

// Attention backward: D_i and lse_i log2(e) into workspace [2, B*H*N] (FP32),
// then the dK/dV and dQ kernels.  K, V, dK, dV have Hkv heads (Hkv divides H).
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const float* o,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* workspace, int B, int H, int Hkv, int N, int D, bool causal,
                           bool bf16, hipStream_t stream);

// Paged decode: tokens per tile, and the most tokens one segment may hold
// (its page ids are staged in LDS, one slot per page).
constexpr int kDecTile = 32;
constexpr int kDecMaxSegTokens = 2048;

// Split of every request's token range [0, max_pages * T) into nseg segments
// of seg_tokens tokens (a multiple of kDecTile).
struct DecodePlan {
    int nseg;
    int seg_tokens;
};

// requested = 0 chooses automatically; cap = max_pages * T.
DecodePlan paged_decode_plan(int64_t B, int64_t Hkv, int64_t cap, int requested);

// The plan of a paged decode call after checking its sizes, and the bytes of
// segment states it needs (0 for one segment); false, with the status to
// report, if the sizes are invalid.  Host computation only (api.hip).
bool paged_decode_plan_checked(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                               int64_t num_pages, int64_t max_pages, int num_splits,
                               attn_status_t* status, int* log2_page, DecodePlan* plan,
                               int64_t* bytes);

// With plan.nseg > 1, part_o [nseg, B*Hq, D] and part_ml [nseg, B*Hq] receive
// the segments' states and the split-KV merge kernel combines them.
hipError_t launch_paged_decode(const void* q, const void* cache, const int* block_table,
                               const int* lengths, float* o, float* lse, int B, int Hq, int Hkv,
                               int D, int log2_page, int P, int max_pages, bool bf16,
                               const DecodePlan& plan, float* part_o, float2* part_ml,
                               hipStream_t stream);

hipError_t launch_row_softmax(const float* x, float* y, int64_t M, int64_t N, hipStream_t stream);

}  // namespace osc
