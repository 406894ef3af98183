// Row softmax on gfx950: y[r,:] = softmax(x[r,:]) for an FP32 [M, N] matrix.
//
// Method: the softmax kernel study (lpnh.cn/news/2830604).  Each lane keeps
// the online (m, d) state of its elements (section 4.4), lane states are
// merged in two levels, wave then workgroup (section 4.6, with the empty
// state (-inf, 0) guarded), and the row is read from memory once and kept in
// registers across the reduction (section 4.8), so HBM sees one read of x and
// one write of y.  Short rows get one wave per row with no barrier (section
// 4.9); long rows get a whole workgroup per row.  Rows that do not start on a
// 16-byte boundary (N = 257 makes three rows in four misaligned, section 4.7)
// use 16-byte loads for every aligned quad that lies inside the row and single
// loads for the quads that straddle its ends.
//
// The merge law and the wave reductions are the ones the attention kernel
// uses (online_merge.hpp); the state is kept in base-2 units, m2 = max(x) *
// log2(e), and every exponential is 2^(x*log2(e) - m2) taken with one FMA.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"
#include "online_merge.hpp"

namespace osc {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Quads are 16-byte aligned groups of 4 floats.  A row that starts `off`
// floats past a 16-byte boundary covers quads 0 .. nq-1 of the aligned base
// pointer pb = row - off; quad j holds row elements 4j - off + t, t = 0..3.
// NT: the kernels that keep the row in registers read x and write y exactly
// once, so their whole quads carry the non-temporal hint; the streaming
// kernel reads each row twice and keeps the default policy.
template <bool NT>
__device__ __forceinline__ void load_quad(const float* pb, int off, int n, int j, float (&v)[4]) {
    const int e0 = 4 * j - off;
    if (e0 >= 0 && e0 + 3 < n) {
        const f32x4* p = reinterpret_cast<const f32x4*>(pb + 4 * j);
        const f32x4 q = NT ? __builtin_nontemporal_load(p) : *p;
        v[0] = q[0];
        v[1] = q[1];
        v[2] = q[2];
        v[3] = q[3];
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int e = e0 + t;
            v[t] = (e >= 0 && e < n) ? pb[4 * j + t] : -INFINITY;
        }
    }
}

// Store the elements of quad j (x-aligned numbering) into the y row.  When y
// has the same 16-byte phase as x the quad maps onto one aligned y quad.
template <bool NT>
__device__ __forceinline__ void store_quad(float* yrow, int xoff, bool same_phase, int n, int j,
                                           const float (&v)[4]) {
    const int e0 = 4 * j - xoff;
    if (same_phase && e0 >= 0 && e0 + 3 < n) {
        const f32x4 q = {v[0], v[1], v[2], v[3]};
        if constexpr (NT)
            __builtin_nontemporal_store(q, reinterpret_cast<f32x4*>(yrow + e0));
        else
            *reinterpret_cast<f32x4*>(yrow + e0) = q;
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int e = e0 + t;
            if (e >= 0 && e < n) yrow[e] = v[t];
        }
    }
}

__host__ __device__ __forceinline__ int phase_of(const float* p) {
    return (int)((reinterpret_cast<uintptr_t>(p) >> 2) & 3);
}

// Lane state of cached values: m2 = max * log2(e); values are replaced by
// 2^(x*log2(e) - m2) and l is their sum.  Empty slots hold -inf.
template <int ITEMS>
__device__ __forceinline__ OnlineState lane_state(float (&v)[ITEMS][4]) {
    float mx = -INFINITY;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it)
#pragma unroll
        for (int t = 0; t < 4; ++t) mx = fmaxf(mx, v[it][t]);
    const float m2 = mx * kLog2e;
    const float pivot = online_pivot(m2);
    float l = 0.0f;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            v[it][t] = fast_exp2(fmaf(v[it][t], kLog2e, -pivot));
            l += v[it][t];
        }
    return {m2, l};
}

// One wave per row, 4 rows per 256-thread workgroup; row length <= 256*ITEMS - 3.
template <int ITEMS>
__global__ void __launch_bounds__(256)
softmax_wave_rows(const float* __restrict__ x, float* __restrict__ y, int M, int N) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;  // whole wave leaves; this kernel has no barrier
    const float* xrow = x + (int64_t)row * N;
    float* yrow = y + (int64_t)row * N;
    const int off = phase_of(xrow);
    const bool same = phase_of(yrow) == off;
    const float* pb = xrow - off;
    const int nq = (N + off + 3) / 4;

    float v[ITEMS][4];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int j = lane + 64 * it;
        if (j < nq) {
            load_quad<true>(pb, off, N, j, v[it]);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) v[it][t] = -INFINITY;
        }
    }
    const OnlineState mine = lane_state<ITEMS>(v);
    const OnlineState row_state = wave_merge(mine);
    const float f = online_rescale(mine.m, row_state.m) / row_state.l;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int j = lane + 64 * it;
        if (j < nq) {
            float r[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) r[t] = v[it][t] * f;
            store_quad<true>(yrow, off, same, N, j, r);
        }
    }
}

constexpr int kBlockThreads = 1024;
constexpr int kBlockWaves = kBlockThreads / 64;

// Merge of per-wave states through LDS; every thread merges the waves in the
// same order, so all threads hold identical bits.
__device__ __forceinline__ OnlineState block_merge(OnlineState s, float* sm, float* sl) {
    const OnlineState ws = wave_merge(s);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        sm[w] = ws.m;
        sl[w] = ws.l;
    }
    __syncthreads();
    OnlineState r{sm[0], sl[0]};
#pragma unroll
    for (int i = 1; i < kBlockWaves; ++i) r = online_merge(r, OnlineState{sm[i], sl[i]});
    return r;
}

// One 1024-thread workgroup per row, the row cached in registers;
// row length <= 4096*ITEMS - 3.
template <int ITEMS>
__global__ void __launch_bounds__(kBlockThreads)
softmax_block_row(const float* __restrict__ x, float* __restrict__ y, int N) {
    __shared__ float sm[kBlockWaves], sl[kBlockWaves];
    const int row = blockIdx.x;
    const float* xrow = x + (int64_t)row * N;
    float* yrow = y + (int64_t)row * N;
    const int off = phase_of(xrow);
    const bool same = phase_of(yrow) == off;
    const float* pb = xrow - off;
    const int nq = (N + off + 3) / 4;

    float v[ITEMS][4];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int j = threadIdx.x + kBlockThreads * it;
        if (j < nq) {
            load_quad<true>(pb, off, N, j, v[it]);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) v[it][t] = -INFINITY;
        }
    }
    const OnlineState mine = lane_state<ITEMS>(v);
    const OnlineState row_state = block_merge(mine, sm, sl);
    const float f = online_rescale(mine.m, row_state.m) / row_state.l;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
        const int j = threadIdx.x + kBlockThreads * it;
        if (j < nq) {
            float r[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) r[t] = v[it][t] * f;
            store_quad<true>(yrow, off, same, N, j, r);
        }
    }
}

// Rows too long to cache: pass 1 folds every quad into the lane's online
// state (section 4.4 of the study), pass 2 reads x again and writes y.
__global__ void __launch_bounds__(kBlockThreads)
softmax_block_row_stream(const float* __restrict__ x, float* __restrict__ y, int N) {
    __shared__ float sm[kBlockWaves], sl[kBlockWaves];
    const int row = blockIdx.x;
    const float* xrow = x + (int64_t)row * N;
    float* yrow = y + (int64_t)row * N;
    const int off = phase_of(xrow);
    const bool same = phase_of(yrow) == off;
    const float* pb = xrow - off;
    const int nq = (N + off + 3) / 4;

    OnlineState s{-INFINITY, 0.0f};
    for (int j = threadIdx.x; j < nq; j += kBlockThreads) {
        float v[4];
        load_quad<false>(pb, off, N, j, v);
        const float qmax = fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3]));
        const float m_new = fmaxf(s.m, qmax * kLog2e);
        const float pivot = online_pivot(m_new);
        float add = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) add += fast_exp2(fmaf(v[t], kLog2e, -pivot));
        s.l = s.l * online_rescale(s.m, m_new) + add;
        s.m = m_new;
    }
    const OnlineState row_state = block_merge(s, sm, sl);
    const float inv = 1.0f / row_state.l;
    for (int j = threadIdx.x; j < nq; j += kBlockThreads) {
        float v[4];
        load_quad<false>(pb, off, N, j, v);
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = fast_exp2(fmaf(v[t], kLog2e, -row_state.m)) * inv;
        store_quad<false>(yrow, off, same, N, j, v);
    }
}

template <typename K, typename... Args>
hipError_t launch(K kernel, unsigned grid, unsigned block, hipStream_t stream, Args... args) {
    void* ptrs[] = {(void*)&args...};
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(block), ptrs, 0,
                           stream);
}

}  // namespace

hipError_t launch_row_softmax(const float* x, float* y, int64_t M64, int64_t N64, hipStream_t stream) {
    const int M = (int)M64, N = (int)N64;
    // Quads a row can touch: exact when every row starts 16-byte aligned.
    const bool all_aligned = (N % 4 == 0) && phase_of(x) == 0;
    const int64_t nq = all_aligned ? N64 / 4 : (N64 + 3 + 3) / 4;
    if (nq <= 64 * 8) {
        const unsigned grid = (unsigned)((M64 + 3) / 4);
        if (nq <= 64) return launch(softmax_wave_rows<1>, grid, 256, stream, x, y, M, N);
        if (nq <= 128) return launch(softmax_wave_rows<2>, grid, 256, stream, x, y, M, N);
        if (nq <= 256) return launch(softmax_wave_rows<4>, grid, 256, stream, x, y, M, N);
        return launch(softmax_wave_rows<8>, grid, 256, stream, x, y, M, N);
    }
    const unsigned grid = (unsigned)M64;
    if (nq <= kBlockThreads * 1) return launch(softmax_block_row<1>, grid, kBlockThreads, stream, x, y, N);
    if (nq <= kBlockThreads * 2) return launch(softmax_block_row<2>, grid, kBlockThreads, stream, x, y, N);
    if (nq <= kBlockThreads * 4) return launch(softmax_block_row<4>, grid, kBlockThreads, stream, x, y, N);
    if (nq <= kBlockThreads * 8) return launch(softmax_block_row<8>, grid, kBlockThreads, stream, x, y, N);
    if (nq <= kBlockThreads * 16) return launch(softmax_block_row<16>, grid, kBlockThreads, stream, x, y, N);
    return launch(softmax_block_row_stream, grid, kBlockThreads, stream, x, y, N);
}

}  // namespace osc
