// Attention forward on gfx950: O = softmax(Q K^T / sqrt(D) + M) V with the
// tiled online-softmax recurrence.
//
// Method: "CUDA FlashAttention: from online softmax to long-sequence IO
// limits" (chengzipai.xyz).  Section 4 gives the recurrence (per K/V tile:
// tile max, new running max, rescale of the old sum and of the unnormalised
// output, exponentials against the new max, P V accumulated in FP32; O = o/l
// at the end) and Figure 1 the dataflow (Q resident on chip, K/V tiles
// streamed through double-buffered on-chip memory, only FP32 m/l/O kept).
// Section 5 adds: a workgroup owns Br query rows so one K/V tile read serves
// all of them (5.1); both products on the matrix cores with FP32 accumulation
// (5.2); parallelism along the query direction of each head (5.2); copy of the
// next K/V tile overlapped with compute, padded on-chip layouts against bank
// conflicts (5.3); 128-bit loads and masked tails (5.4).  Section 7: causal
// tiles wholly above the diagonal are skipped and only diagonal tiles are
// masked element by element.
//
// gfx950 mapping (one workgroup = 4 waves = 256 threads):
//   * A wave owns QB blocks of 32 query rows.  It computes S^T = K Q^T on the
//     32x32x16 MFMA, so a lane holds the scores of ONE query (its column) for
//     16 of every 32 keys; lane l and lane l^32 share a query.  Row max and
//     row sum are in-lane plus one exchange with lane l^32.
//   * Q fragments (the MFMA B operand) sit in VGPRs for the whole K/V loop.
//   * K and V tiles of BC keys are double-buffered in LDS, row-major with
//     padded pitches, filled with 16-byte global loads staged in VGPRs while
//     the previous tile is being consumed.
//   * O^T += V^T P^T on the same MFMA: P^T comes straight from the S^T
//     accumulators (converted to 16-bit), V^T fragments are read from the
//     row-major V tile with ds_read_b64_tr_b16 (LDS transpose read).
//   * Exponentials are base 2 with log2(e)/sqrt(D) folded into one FMA.
//   * Workgroups are ordered longest-first for causal load balance; with
//     the hardware's round-robin dispatch over the 8 XCDs, consecutive
//     workgroups are different heads of the same query tile, so each XCD keeps
//     a fixed subset of heads and their K/V stays in that XCD's L2.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"
#include "online_merge.hpp"

namespace osc {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;

template <bool BF16>
struct Mma;

template <>
struct Mma<false> {
    __device__ __forceinline__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    // Round-to-nearest-even conversion of two FP32 values into one packed dword.
    __device__ __forceinline__ static unsigned pack(float lo, float hi) {
        f16x2 r;
        r[0] = (_Float16)lo;
        r[1] = (_Float16)hi;
        return __builtin_bit_cast(unsigned, r);
    }
};

template <>
struct Mma<true> {
    __device__ __forceinline__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ __forceinline__ static unsigned pack(float lo, float hi) {
        bf16x2 r;
        r[0] = (__bf16)lo;
        r[1] = (__bf16)hi;
        return __builtin_bit_cast(unsigned, r);
    }
};

// Compile-time geometry of one kernel instance.
template <int D_, int QB_, int NW_>
struct Geo {
    static constexpr int D = D_;
    static constexpr int QB = QB_;              // 32-row query blocks per wave
    static constexpr int NW = NW_;              // waves per workgroup
    static constexpr int THREADS = 64 * NW;
    static constexpr int BR = 32 * QB * NW;     // query rows per workgroup
    static constexpr int BC = D == 128 ? 64 : 128;  // keys per LDS tile
    static constexpr int SUB = 64;              // keys per compute step
    // LDS pitches in 16-bit elements.  K: pitch = D/2 + 4 dwords, an odd
    // multiple of 4 modulo 64 banks, so the 16 lanes of one ds_read_b128
    // phase (16 consecutive key rows) hit 16 distinct 4-bank groups.  V:
    // pitch = D/2 + 16 dwords, 16 or 48 modulo 64, so the four key rows that
    // each 16-lane group of a ds_read_b64_tr_b16 touches land in disjoint
    // banks, also across the two d-halves of a 32-lane phase.
    static constexpr int KP = D + 8;
    static constexpr int VP = D + 32;
    static constexpr int KT = BC * KP;
    static constexpr int VT = BC * VP;
    static constexpr int STAGE = KT + VT;
    static constexpr int CHUNKS = BC * D / 8;   // 16-byte chunks per K (or V) tile
    static constexpr int CPT = CHUNKS / THREADS;
    static_assert(CHUNKS % THREADS == 0, "tile fill must divide evenly");
    static_assert(BC % SUB == 0, "compute step must divide the tile");
};

template <int D, int QB>
struct WaveState {
    u32x4 qf[QB][D / 16];     // Q^T fragments (MFMA B operand), one per 16-wide d step
    f32x16 acc[QB][D / 32];   // O^T accumulators, 32 d-rows each
    float m[QB];              // running max of this lane's query, log2 units
    float l[QB];              // this lane's share of the running sum
};

__device__ __forceinline__ u32x4 tr16_b64x2(const u16* p0, const u16* p1) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
    const auto a = __builtin_bit_cast(unsigned long long, r0);
    const auto b = __builtin_bit_cast(unsigned long long, r1);
    return u32x4{(unsigned)a, (unsigned)(a >> 32), (unsigned)b, (unsigned)(b >> 32)};
}

// One compute step over SUB = 64 keys of the LDS tile for the query blocks in
// ACT (bit b set = block b has visible keys in this step).  `kl`/`vl` point at
// the first key of the step inside the K / V tile; `key0` is that key's index
// in the sequence.  Bit b of `need_mask` asks for element masking of block b
// (diagonal tile or ragged key tail).
template <bool BF16, int D, int QB, int NW, bool CAUSAL, unsigned ACT>
__device__ __forceinline__ void attend_step(WaveState<D, QB>& st, const u16* kl, const u16* vl,
                                            int lane, int key0, const int (&row0)[QB],
                                            unsigned need_mask, int N, float scale_log2) {
    using G = Geo<D, QB, NW>;
    using M = Mma<BF16>;
    const int g = lane >> 5;
    const int col = lane & 31;

    // S^T[key][query] = sum_d K[key][d] Q[query][d] for two 32-key blocks.
    f32x16 s[QB][2];
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[b][kb] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const u16* kp = kl + (kb * 32 + col) * G::KP + 8 * g;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(kp + ks * 16);
#pragma unroll
            for (int b = 0; b < QB; ++b)
                if (ACT & (1u << b)) s[b][kb] = M::run(a, st.qf[b][ks], s[b][kb]);
        }
    }

    // Online softmax update per query block; P^T packed as the next B operand.
    u32x4 pf[QB][4];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        if (!(ACT & (1u << b))) continue;
        if (need_mask & (1u << b)) {
            const int qrow = row0[b] + col;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = key0 + kb * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
                    if ((CAUSAL && key > qrow) || key >= N) s[b][kb][i] = -INFINITY;
                }
        }
        float mx = s[b][0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][kb][i]);
        mx = fmaxf(mx, swap32_f32(mx));
        const float m_new = fmaxf(st.m[b], mx * scale_log2);
        const float alpha = online_rescale(st.m[b], m_new);
        const float pivot = online_pivot(m_new);
        float rs = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(fmaf(s[b][kb][i], scale_log2, -pivot));
                s[b][kb][i] = p;
                rs += p;
            }
        st.l[b] = st.l[b] * alpha + rs;
        st.m[b] = m_new;
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) st.acc[b][mt] *= alpha;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kb = u >> 1, h = (u & 1) * 8;
            pf[b][u] = u32x4{M::pack(s[b][kb][h + 0], s[b][kb][h + 1]),
                             M::pack(s[b][kb][h + 2], s[b][kb][h + 3]),
                             M::pack(s[b][kb][h + 4], s[b][kb][h + 5]),
                             M::pack(s[b][kb][h + 6], s[b][kb][h + 7])};
        }
    }

    // O^T[d][query] += sum_key V^T[d][key] P^T[key][query].  B-operand slot
    // 8g+j of MFMA u holds key 16u + 8(j/4) + 4g + j%4 (the S^T accumulator
    // order); the transpose reads fetch V^T in exactly that key order: each
    // 16-lane group reads 4 key rows x 16 d, lane l ends with d = l%32.
    const int tr_key = 4 * g + ((lane >> 2) & 3);
    const int tr_d = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u16* vp = vl + (u * 16 + tr_key) * G::VP + mt * 32 + tr_d;
            const u32x4 a = tr16_b64x2(vp, vp + 8 * G::VP);
#pragma unroll
            for (int b = 0; b < QB; ++b)
                if (ACT & (1u << b)) st.acc[b][mt] = M::run(a, pf[b][u], st.acc[b][mt]);
        }
}

template <class G, int CPT>
__device__ __forceinline__ void load_tile(u32x4 (&kr)[CPT], u32x4 (&vr)[CPT],
                                          const u16* __restrict__ k, const u16* __restrict__ v,
                                          int tile, int N, int tid) {
    constexpr int D = G::D;
#pragma unroll
    for (int c = 0; c < G::CPT; ++c) {
        const int id = tid + c * G::THREADS;
        const int r = id / (D / 8), cc = id % (D / 8);
        const int key = tile * G::BC + r;
        if (key < N) {
            const int64_t off = (int64_t)key * D + cc * 8;
            kr[c] = *reinterpret_cast<const u32x4*>(k + off);
            vr[c] = *reinterpret_cast<const u32x4*>(v + off);
        } else {
            kr[c] = u32x4{0u, 0u, 0u, 0u};
            vr[c] = u32x4{0u, 0u, 0u, 0u};
        }
    }
}

template <class G, int CPT>
__device__ __forceinline__ void store_tile(u16* stage, const u32x4 (&kr)[CPT],
                                           const u32x4 (&vr)[CPT], int tid) {
    constexpr int D = G::D;
#pragma unroll
    for (int c = 0; c < G::CPT; ++c) {
        const int id = tid + c * G::THREADS;
        const int r = id / (D / 8), cc = id % (D / 8);
        *reinterpret_cast<u32x4*>(stage + r * G::KP + cc * 8) = kr[c];
        *reinterpret_cast<u32x4*>(stage + G::KT + r * G::VP + cc * 8) = vr[c];
    }
}

template <bool BF16, int D, bool CAUSAL, int QB, int NW>
__global__ void __launch_bounds__(64 * NW)
attn_fwd_kernel(const u16* __restrict__ q, const u16* __restrict__ k, const u16* __restrict__ v,
                float* __restrict__ o, float* __restrict__ lse, int BH, int N, int T,
                float scale_log2) {
    using G = Geo<D, QB, NW>;
    __shared__ __attribute__((aligned(16))) u16 lds[2 * G::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

    // Work item: longest causal tiles first; consecutive workgroups are
    // different heads of one query tile.
    const int bid = blockIdx.x;
    const int t = CAUSAL ? (T - 1 - bid / BH) : (bid / BH);
    const int bh = bid % BH;
    const int64_t head = (int64_t)bh * N * D;
    q += head;
    k += head;
    v += head;
    o += head;
    lse += (int64_t)bh * N;

    const int row_base = t * G::BR;
    int row0[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) row0[b] = row_base + (b * G::NW + w) * 32;
    const int kv_end = CAUSAL ? min(row_base + G::BR, N) : N;
    const int ntiles = (kv_end + G::BC - 1) / G::BC;

    WaveState<D, QB> st;
    const int col = lane & 31, g = lane >> 5;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const int row = row0[b] + col;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            st.qf[b][ks] = row < N ? *reinterpret_cast<const u32x4*>(q + (int64_t)row * D + ks * 16 + 8 * g)
                                   : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt) st.acc[b][mt] = f32x16{};
        st.m[b] = -INFINITY;
        st.l[b] = 0.0f;
    }

    u32x4 kr[G::CPT], vr[G::CPT];
    load_tile<G>(kr, vr, k, v, 0, N, tid);
    store_tile<G>(lds, kr, vr, tid);
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const bool more = it + 1 < ntiles;
        if (more) load_tile<G>(kr, vr, k, v, it + 1, N, tid);
        const u16* kl = lds + (it & 1) * G::STAGE;
        const u16* vl = kl + G::KT;
#pragma unroll
        for (int sub = 0; sub < G::BC / G::SUB; ++sub) {
            const int key0 = it * G::BC + sub * G::SUB;
            unsigned act = 0, need = 0;
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                const bool live = row0[b] < N && key0 < N && (!CAUSAL || key0 <= row0[b] + 31);
                const bool mask = (CAUSAL && key0 + G::SUB - 1 > row0[b]) || key0 + G::SUB > N;
                act |= live ? (1u << b) : 0u;
                need |= mask ? (1u << b) : 0u;
            }
            const u16* ks = kl + sub * G::SUB * G::KP;
            const u16* vs = vl + sub * G::SUB * G::VP;
            if constexpr (QB == 2) {
                if (act == 3u)
                    attend_step<BF16, D, QB, NW, CAUSAL, 3u>(st, ks, vs, lane, key0, row0, need, N, scale_log2);
                else if (act == 2u)
                    attend_step<BF16, D, QB, NW, CAUSAL, 2u>(st, ks, vs, lane, key0, row0, need, N, scale_log2);
                else if (act == 1u)
                    attend_step<BF16, D, QB, NW, CAUSAL, 1u>(st, ks, vs, lane, key0, row0, need, N, scale_log2);
            } else {
                if (act == 1u)
                    attend_step<BF16, D, QB, NW, CAUSAL, 1u>(st, ks, vs, lane, key0, row0, need, N, scale_log2);
            }
        }
        if (more) store_tile<G>(lds + ((it + 1) & 1) * G::STAGE, kr, vr, tid);
        __syncthreads();
    }

    // Epilogue: combine the two lane halves of each query, normalise, store.
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const float l_tot = st.l[b] + swap32_f32(st.l[b]);
        const int row = row0[b] + col;
        if (row < N) {
            const float inv = 1.0f / l_tot;
            float* orow = o + (int64_t)row * D;
#pragma unroll
            for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x4 r = {st.acc[b][mt][4 * i4 + 0] * inv, st.acc[b][mt][4 * i4 + 1] * inv,
                                     st.acc[b][mt][4 * i4 + 2] * inv, st.acc[b][mt][4 * i4 + 3] * inv};
                    *reinterpret_cast<f32x4*>(orow + mt * 32 + 8 * i4 + 4 * g) = r;
                }
            if (g == 0) lse[row] = (st.m[b] + log2f(l_tot)) * kLn2;
        }
    }
}

template <bool BF16, int D, bool CAUSAL, int QB, int NW>
hipError_t launch_one(const void* q, const void* k, const void* v, float* o, float* lse, int BH,
                      int N, hipStream_t stream) {
    using G = Geo<D, QB, NW>;
    const int T = (N + G::BR - 1) / G::BR;
    const float scale_log2 = kLog2e / __builtin_sqrtf((float)D);
    const u16* qq = static_cast<const u16*>(q);
    const u16* kk = static_cast<const u16*>(k);
    const u16* vv = static_cast<const u16*>(v);
    void* args[] = {(void*)&qq, (void*)&kk, (void*)&vv, (void*)&o, (void*)&lse,
                    (void*)&BH, (void*)&N, (void*)const_cast<int*>(&T), (void*)const_cast<float*>(&scale_log2)};
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_kernel<BF16, D, CAUSAL, QB, NW>),
                           dim3((unsigned)(T * BH)), dim3(G::THREADS), args, 0, stream);
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch_qb(const void* q, const void* k, const void* v, float* o, float* lse, int BH,
                     int N, int qb, hipStream_t stream) {
    return qb == 1 ? launch_one<BF16, D, CAUSAL, 1, 4>(q, k, v, o, lse, BH, N, stream)
                   : launch_one<BF16, D, CAUSAL, 1, 8>(q, k, v, o, lse, BH, N, stream);
}

}  // namespace

// Rows per workgroup: 256 (two 32-row blocks per wave) when that still gives
// at least one workgroup per CU, else 128.
int attn_pick_qb(int64_t BH, int64_t N) {
    const int64_t wgs_big = BH * ((N + 255) / 256);
    return wgs_big >= 256 ? 2 : 1;
}

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                           int BH, int N, int D, bool causal, bool bf16, int qb, hipStream_t stream) {
    if (D == 128) {
        if (bf16)
            return causal ? launch_qb<true, 128, true>(q, k, v, o, lse, BH, N, qb, stream)
                          : launch_qb<true, 128, false>(q, k, v, o, lse, BH, N, qb, stream);
        return causal ? launch_qb<false, 128, true>(q, k, v, o, lse, BH, N, qb, stream)
                      : launch_qb<false, 128, false>(q, k, v, o, lse, BH, N, qb, stream);
    }
    if (bf16)
        return causal ? launch_qb<true, 64, true>(q, k, v, o, lse, BH, N, qb, stream)
                      : launch_qb<true, 64, false>(q, k, v, o, lse, BH, N, qb, stream);
    return causal ? launch_qb<false, 64, true>(q, k, v, o, lse, BH, N, qb, stream)
                  : launch_qb<false, 64, false>(q, k, v, o, lse, BH, N, qb, stream);
}

}  // namespace osc
