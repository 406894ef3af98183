// Online-softmax state and its merge law, shared by the attention kernel and
// the row-softmax kernels (gfx950, wave64).
//
// The state of a partially reduced row is (m, l): m is the running maximum of
// the logits seen so far and l = sum_j 2^(x_j - m) over those logits.  Two
// states merge by rescaling both sums to the larger maximum:
//     m = max(m1, m2),  l = l1 * 2^(m1 - m) + l2 * 2^(m2 - m).
// This is the tile recurrence of "CUDA FlashAttention: from online softmax to
// long-sequence IO limits" (chengzipai.xyz), section 4 (alpha and beta are
// the two rescale factors), and the two-level (m, d) merge of the softmax
// kernel study (lpnh.cn/news/2830604), section 4.6.  The state is kept in the
// base-2 domain: callers pre-multiply logits by log2(e) (and by any softmax
// scale), so every exponential is the hardware's v_exp_f32.
//
// The empty state is (-inf, 0).  Merging with it must not produce
// -inf - (-inf) = NaN (FA page section 6, softmax study section 4.6): the
// rescale factor of an empty side is defined as 0.
#pragma once

#include <hip/hip_runtime.h>

namespace osc {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct OnlineState {
    float m;  // running maximum, base-2 logit units
    float l;  // sum of 2^(x - m) over the logits folded in so far
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^(m_old - m_new): the factor that moves a sum taken relative to m_old onto
// m_new (m_new >= m_old).  An empty old state (m_old = -inf) contributes 0.
__device__ __forceinline__ float online_rescale(float m_old, float m_new) {
    return m_old == -INFINITY ? 0.0f : fast_exp2(m_old - m_new);
}

// The point exponentials are taken against.  A row with no logit yet keeps
// m = -inf; subtracting 0 instead makes every masked 2^(-inf - 0) = 0.
__device__ __forceinline__ float online_pivot(float m) { return m == -INFINITY ? 0.0f : m; }

__device__ __forceinline__ OnlineState online_merge(OnlineState a, OnlineState b) {
    const float m = fmaxf(a.m, b.m);
    return {m, a.l * online_rescale(a.m, m) + b.l * online_rescale(b.m, m)};
}

// ----------------------------------------------------------------------------
// Cross-lane exchange primitives.
//
// DPP moves within rows of 16 lanes (quad_perm, row_half_mirror, row_mirror),
// ds_swizzle swaps the two 16-lane halves of each 32-lane group, and
// v_permlane32_swap swaps the two 32-lane halves of the wave.

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, true));
}

// DPP control codes (GFX9 encoding).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

// Value of lane (l ^ 16).
__device__ __forceinline__ float swap16_f32(float x) {
    // BitMode swizzle: and_mask = 0x1f, or_mask = 0, xor_mask = 0x10.
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401f));
}

// Value of lane (l ^ 32).
__device__ __forceinline__ float swap32_f32(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // Lanes 0..31 find lane l+32's value in r[1], lanes 32..63 find lane l-32's in r[0].
    const unsigned lo = r[1], hi = r[0];
    return __builtin_bit_cast(float, (threadIdx.x & 32) ? hi : lo);
}

// Maximum over all 64 lanes, returned in every lane.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_f32<kDppXor1>(x));
    x = fmaxf(x, dpp_f32<kDppXor2>(x));
    x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
    x = fmaxf(x, dpp_f32<kDppMirror>(x));
    x = fmaxf(x, swap16_f32(x));
    x = fmaxf(x, swap32_f32(x));
    return x;
}

template <int kCtrl>
__device__ __forceinline__ OnlineState dpp_merge(OnlineState s) {
    return online_merge(s, OnlineState{dpp_f32<kCtrl>(s.m), dpp_f32<kCtrl>(s.l)});
}

// Merge of the 64 lane states of a wave, returned in every lane.  The tree
// has the same shape in every lane, so every lane ends with the same bits.
__device__ __forceinline__ OnlineState wave_merge(OnlineState s) {
    s = dpp_merge<kDppXor1>(s);
    s = dpp_merge<kDppXor2>(s);
    s = dpp_merge<kDppHalfMirror>(s);
    s = dpp_merge<kDppMirror>(s);
    s = online_merge(s, OnlineState{swap16_f32(s.m), swap16_f32(s.l)});
    s = online_merge(s, OnlineState{swap32_f32(s.m), swap32_f32(s.l)});
    return s;
}

}  // namespace osc
