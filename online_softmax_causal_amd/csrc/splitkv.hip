// Second kernel of split-KV attention: merge the per-segment states of each
// query row into O and LSE (gfx950).
//
// Segment s of a row holds (m_s, l_s, o_s): m_s is the reference maximum of
// its scaled logits in base-2 units, l_s = sum_j 2^(x_j - m_s) and
// o_s = sum_j 2^(x_j - m_s) v_j over the segment's visible keys.  The row's
// result follows the split-KV merge of "CUDA KV Cache: paged storage and
// long-context decode" (chengzipai.xyz), section 6.4:
//     m = max_s m_s,  l = sum_s l_s 2^(m_s - m),  O = sum_s o_s 2^(m_s - m) / l,
// the same law as the tile recurrence (FA page, section 4).  The maximum is
// taken first over all live segments, then every segment is rescaled to it
// with the shared online_rescale (an empty segment, m_s = -inf, contributes
// 0), so all loads of a row are independent and issue together.
// LSE = (m + log2 l) ln 2.
//
// The kernel is bound by HBM: per row it reads nseg * (D + 2) * 4 bytes and
// writes (D + 1) * 4.  D / 4 lanes cover one row with 16-byte accesses.  Few
// rows (decode: one per request and query head) use 64-thread workgroups so
// that the rows spread over more CUs.
#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "online_merge.hpp"

namespace osc {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D, int THREADS>
__global__ void __launch_bounds__(THREADS)
splitkv_merge_kernel(const float* __restrict__ part_o, const float2* __restrict__ part_ml,
                     float* __restrict__ o, float* __restrict__ lse, int64_t rows, int N, int nseg,
                     int seg_rows, bool causal) {
    constexpr int TPR = D / 4;            // lanes per row
    constexpr int RPB = THREADS / TPR;    // rows per workgroup
    const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = (threadIdx.x % TPR) * 4;
    if (r >= rows) return;
    const int i = (int)(r % N);
    // Segments with a visible key: all of them, or with causal masking those
    // starting at or before row i.
    const int live = causal ? min(nseg, i / seg_rows + 1) : nseg;
    float m = -INFINITY;
#pragma unroll 8
    for (int s = 0; s < live; ++s) m = fmaxf(m, part_ml[(int64_t)s * rows + r].x);
    float l = 0.0f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
    for (int s = 0; s < live; ++s) {
        const int64_t pr = (int64_t)s * rows + r;
        const float2 ml = part_ml[pr];
        const f32x4 os = *reinterpret_cast<const f32x4*>(part_o + pr * D + c);
        const float w = online_rescale(ml.x, m);
        l += ml.y * w;
        acc += os * w;
    }
    const float inv = 1.0f / l;
    *reinterpret_cast<f32x4*>(o + r * D + c) = acc * inv;
    if (c == 0) lse[r] = (m + log2f(l)) * kLn2;
}

}  // namespace

hipError_t launch_splitkv_merge(const float* part_o, const float2* part_ml, float* o, float* lse,
                                int BH, int N, int D, int nseg, int seg_rows, bool causal,
                                hipStream_t stream) {
    const int64_t rows = (int64_t)BH * N;
    const bool small = rows < 16384;
    const int threads = small ? 64 : 256;
    const int rpb = threads / (D / 4);
    const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
    int64_t rows_a = rows;
    void* params[] = {(void*)&part_o, (void*)&part_ml, (void*)&o, (void*)&lse, (void*)&rows_a,
                      (void*)&N, (void*)&nseg, (void*)&seg_rows, (void*)&causal};
    const void* fn;
    if (D == 128)
        fn = small ? reinterpret_cast<const void*>(&splitkv_merge_kernel<128, 64>)
                   : reinterpret_cast<const void*>(&splitkv_merge_kernel<128, 256>);
    else
        fn = small ? reinterpret_cast<const void*>(&splitkv_merge_kernel<64, 64>)
                   : reinterpret_cast<const void*>(&splitkv_merge_kernel<64, 256>);
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), params, 0, stream);
}

}  // namespace osc
