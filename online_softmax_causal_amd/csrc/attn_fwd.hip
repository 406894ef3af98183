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
// gfx950 mapping, common to both kernels below:
//   * A wave owns blocks of 32 query rows.  It computes S^T = K Q^T on the
//     32x32x16 MFMA, so a lane holds the scores of ONE query (its column) for
//     16 of every 32 keys; lane l and lane l^32 share a query.  Row max and
//     row sum are in-lane plus one exchange with lane l^32.
//   * Q fragments (the MFMA B operand) sit in VGPRs for the whole K/V loop.
//   * K and V tiles of 64 keys are copied global -> LDS with
//     global_load_lds_dwordx4 (no VGPR staging) into unpadded rows whose
//     16-byte chunks are XOR-swizzled against bank conflicts, several tiles
//     ahead of their use.
//   * O^T += V^T P^T on the same MFMA: P^T comes straight from the S^T
//     accumulators (converted to 16-bit), V^T fragments are read from the
//     row-major V tile with ds_read_b64_tr_b16 (LDS transpose read).
//   * Exponentials are base 2 with log2(e)/sqrt(D) folded into one FMA.
//   * Workgroups are ordered longest-first for causal load balance; with
//     the hardware's round-robin dispatch over the 8 XCDs, consecutive
//     workgroups are different heads of the same query tile, so each XCD keeps
//     a fixed subset of heads and their K/V stays in that XCD's L2.
// Three kernels: the tile-lagged pipeline kernel (D = 128) and the key-half
// unit kernel (D = 64), both 8 waves and 256 query rows per workgroup (512
// for the unit kernel with two row blocks per wave), one workgroup per CU,
// used when there are enough workgroups of 256 rows and for every key split;
// and the ring kernel (4 waves, 128 rows, two workgroups per CU) for grids too
// small for those.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>
#include <utility>

#include "kernels.hpp"
#include "mfma_tile.hpp"
#include "online_merge.hpp"

namespace osc {
namespace {

// Compile-time loop: f(integral_constant<int, i>) for i = 0 .. N-1, always
// fully unrolled (a #pragma unroll loop over a large body may be left rolled,
// which turns register arrays into scratch memory).
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Compile-time geometry of one kernel instance.
//
// LDS holds STAGES stages; a stage is one K tile followed by one V tile, each
// BC = 64 key rows of D 16-bit values, unpadded (a row is D/8 chunks of 16
// bytes).  Tiles are written straight from global memory by
// global_load_lds_dwordx4, which puts lane i's 16 bytes at 16*i past a
// wave-uniform LDS address, so one wave instruction fills one 1 KiB block
// (RPB rows).  Bank conflicts are avoided by storing logical chunk c of row r
// at chunk position c ^ chunk_swizzle(r): the swizzle gives the 16
// consecutive rows read by one ds_read_b128 phase 16 distinct 16-byte bank
// groups, and the 4 rows x 4 chunks of one 32-lane ds_read_b64_tr_b16 phase
// 16 distinct bank groups as well.
template <int D_, int NW_, int STAGES_, int DIST_, int DMAW_>
struct Geo {
    static constexpr int D = D_;
    static constexpr int NW = NW_;              // waves per workgroup
    static constexpr int DMAW = DMAW_;          // waves that issue the tile copies
    static constexpr int STAGES = STAGES_;      // LDS stages
    static constexpr int DIST = DIST_;          // tiles copied ahead of the one being computed
    static constexpr int THREADS = 64 * NW;
    static constexpr int BC = 64;               // keys per tile
    static constexpr int MT = D / 32;           // 32-row d blocks of O^T
    static constexpr int KS = D / 16;           // 16-wide d steps of Q K^T
    static constexpr int CPR = D / 8;           // 16-byte chunks per row
    static constexpr int RPB = 1024 / (2 * D);  // rows per 1 KiB block
    static constexpr int TILE = BC * D;         // 16-bit elements per K (or V) tile
    static constexpr int STAGE = 2 * TILE;
    static constexpr int BPW = BC / RPB / DMAW; // 1 KiB blocks per copying wave per tile
    static_assert(BPW >= 1 && BPW * RPB * DMAW == BC, "tile fill must divide evenly");
    static_assert(DIST == 1 || DIST == 2, "prefetch distance");
};

// Kernel arguments (one struct, passed by value).
struct AttnArgs {
    const u16* q;   // [B, H, N, D]
    const u16* k;   // [B, Hkv, N, D]
    const u16* v;   // [B, Hkv, N, D]
    float* o;       // [B, H, N, D]
    float* lse;     // [B, H, N]
    int BH;         // B * H
    int H;          // query heads
    int Hkv;        // key/value heads (divides H)
    int N;          // sequence length
    int T;          // query tiles per head
    int fold;       // causal order folded: the grid's second half runs shortest first
    float scale_log2;  // log2(e) / sqrt(D)
    // Split along the keys (split-KV): segment s of every head covers the
    // 64-key tiles [s * seg_tiles, (s + 1) * seg_tiles).  With part_o set,
    // each workgroup stores its segment's unnormalised state instead of O
    // and LSE, for splitkv_merge_kernel to combine.
    int nseg;          // segments per head (1: no split)
    int seg_tiles;     // tiles per segment, a multiple of 4 (256 keys)
    float* part_o;     // [nseg, B*H, N, D]: sum_j 2^(s_j - m) v_j over the segment
    float2* part_ml;   // [nseg, B*H, N]: (m, l) of the segment, base-2 units
};

template <int D, int QB>
struct WaveState {
    u32x4 qf[QB][D / 16];     // Q^T fragments (MFMA B operand), one per 16-wide d step
    f32x16 acc[QB][D / 32];   // O^T accumulators, 32 d-rows each
    float m[QB];              // reference max of this lane's query, log2 units
    float l[QB];              // this lane's share of the running sum (relative to m)
};

// Per-lane LDS offsets (16-bit elements, relative to a tile) of the MFMA
// operand fragments, swizzle included; fixed for the whole kernel.
template <int D>
struct FragOffsets {
    int k[D / 16];        // K fragment of d step ks for key row (lane % 32); + 32*D for keys 32..63
    int v[D / 32][2];     // V^T fragment halves of d block mt; + 16*D per 16-key group
};

template <class G>
__device__ __forceinline__ FragOffsets<G::D> frag_offsets(int lane) {
    constexpr int D = G::D;
    FragOffsets<D> fo;
    const int col = lane & 31, g = lane >> 5;
    const int sw = chunk_swizzle<D>(col);
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks) fo.k[ks] = col * D + (((2 * ks + g) ^ sw) << 3);
    // ds_read_b64_tr_b16: each 16-lane group reads 4 key rows x 16 d; lane l
    // supplies row tr_key (+8 for the second read), d = 32 mt + 16 dh + 4 (l % 4).
    const int tr_key = 4 * g + ((lane >> 2) & 3);
    const int dh = (lane >> 4) & 1;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = tr_key + 8 * r;
            const int c = 4 * mt + 2 * dh + ((lane & 3) >> 1);
            fo.v[mt][r] = row * D + ((c ^ chunk_swizzle<D>(row)) << 3) + 4 * (lane & 1);
        }
    return fo;
}

// S^T[key][query] = sum_d K[key][d] Q[query][d] for the 64 keys of one K
// tile (two 32-key accumulators per query block).  The 2*KS A-operand
// fragments stream through a 4-deep register ring so each LDS read is issued
// four fragments ahead of its use (enforced with scheduling groups); each
// fragment feeds the MFMAs of all QB query blocks, and consecutive MFMAs
// alternate accumulators.
template <bool BF16, class G, int QB>
__device__ __forceinline__ void qk_tile(const WaveState<G::D, QB>& st, const FragOffsets<G::D>& fo,
                                        const u16* kt, f32x16 (&s)[QB][2]) {
    using M = Mma<BF16>;
    constexpr int NF = 2 * G::KS;
    auto kfrag = [&](int f) {
        return *reinterpret_cast<const u32x4*>(kt + fo.k[f >> 1] + (f & 1) * 32 * G::D);
    };
    __builtin_amdgcn_sched_barrier(0);
    u32x4 ring[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) ring[f] = kfrag(f);
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        s[b][0] = f32x16{};
        s[b][1] = f32x16{};
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const u32x4 a = ring[f & 3];
        if (f + 4 < NF) ring[f & 3] = kfrag(f + 4);
#pragma unroll
        for (int b = 0; b < QB; ++b) s[b][f & 1] = M::run(a, st.qf[b][f >> 1], s[b][f & 1]);
    }
    // Keep the ring: without these groups the scheduler, tight on registers,
    // issued each read right before its MFMA and waited for it there.
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 0);
#pragma unroll
    for (int f = 0; f < NF - 4; ++f) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, QB, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 4 * QB, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// Online-softmax update and O^T += V^T P^T for one 64-key tile whose raw
// scores are in `s`.  Lane (col, g) holds keys 8(i/4) + 4g + i%4 of each
// 32-key block for query row0[b] + col of query block b.  MASKED (diagonal
// tile or ragged key tail) sets the scores of keys after the query or past N
// to -inf first.
template <bool BF16, class G, bool CAUSAL, bool MASKED, int QB>
__device__ __forceinline__ void softmax_pv_tile(WaveState<G::D, QB>& st, const FragOffsets<G::D>& fo,
                                                f32x16 (&s)[QB][2], const u16* vt, int lane,
                                                int key0, const int (&row0)[QB], int N,
                                                float scale_log2) {
    using M = Mma<BF16>;
    const int g = lane >> 5;
    const int col = lane & 31;

    if constexpr (MASKED) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            // key0 + c + 4g is masked iff it is > row0 + col (causal) or >= N,
            // i.e. iff the compile-time offset c exceeds lim.
            const int lim = min(CAUSAL ? row0[b] + col - key0 : (1 << 30), N - 1 - key0) - 4 * g;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int c = kb * 32 + 8 * (i >> 2) + (i & 3);
                    s[b][kb][i] = c > lim ? -INFINITY : s[b][kb][i];
                }
        }
    }
    float tile_m[QB];
    bool grow[QB];
    bool any_grow = false;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        float mx = s[b][0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][kb][i]);
        mx = fmaxf(mx, swap32_f32(mx));
        tile_m[b] = mx * scale_log2;
        grow[b] = tile_m[b] > st.m[b] + rescale_slack<BF16>();
        any_grow = any_grow || grow[b];
    }
    // Each query decides for itself (so a row's result never depends on
    // another row's data); the wave branches if any query needs to move, and
    // the others multiply by exactly 1.
    if (__builtin_amdgcn_ballot_w64(any_grow) != 0) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            const float m_new = grow[b] ? tile_m[b] : st.m[b];
            const float alpha = grow[b] ? online_rescale(st.m[b], m_new) : 1.0f;
            st.l[b] *= alpha;
#pragma unroll
            for (int mt = 0; mt < G::MT; ++mt) st.acc[b][mt] *= alpha;
            st.m[b] = m_new;
        }
    }

    u32x4 pf[QB][4];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const float pivot = online_pivot(st.m[b]);
        float rs0 = 0.0f, rs1 = 0.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kb = u >> 1, h = (u & 1) * 8;
            float p[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) p[j] = fast_exp2(fmaf(s[b][kb][h + j], scale_log2, -pivot));
            pf[b][u] = u32x4{M::pack(p[0], p[1]), M::pack(p[2], p[3]), M::pack(p[4], p[5]),
                             M::pack(p[6], p[7])};
            if constexpr (M::kSumRounded) {
                rs0 = M::sum2(pf[b][u][0], rs0);
                rs1 = M::sum2(pf[b][u][1], rs1);
                rs0 = M::sum2(pf[b][u][2], rs0);
                rs1 = M::sum2(pf[b][u][3], rs1);
            } else {
#pragma unroll
                for (int j = 0; j < 8; j += 2) {
                    rs0 += p[j];
                    rs1 += p[j + 1];
                }
            }
        }
        st.l[b] += rs0 + rs1;
    }

    // O^T[d][query] += sum_key V^T[d][key] P^T[key][query].  B-operand slot
    // 8g+j of MFMA u holds key 16u + 8(j/4) + 4g + j%4 (the S^T accumulator
    // order); the transpose reads fetch V^T in exactly that key order, lane l
    // ending with d = 32 mt + l % 32.  Each fragment feeds all query blocks.
    constexpr int NV = 4 * G::MT;
    auto vfrag = [&](int f) {
        const u16* base = vt + (f / G::MT) * 16 * G::D;
        return tr16_b64x2(base + fo.v[f % G::MT][0], base + fo.v[f % G::MT][1]);
    };
    u32x4 vring[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) vring[f] = vfrag(f);
#pragma unroll
    for (int f = 0; f < NV; ++f) {
        const u32x4 a = vring[f & 3];
        if (f + 4 < NV) vring[f & 3] = vfrag(f + 4);
#pragma unroll
        for (int b = 0; b < QB; ++b)
            st.acc[b][f % G::MT] = M::run(a, pf[b][f / G::MT], st.acc[b][f % G::MT]);
    }
}

// Issue the direct global->LDS copy of rows [tile*BC, tile*BC + BC) of one
// head's K (or V) into an LDS tile.  Rows past N are clamped to row N-1: they
// only feed keys that are masked (score -inf, weight exactly 0).
template <class G>
__device__ __forceinline__ void dma_block(const u16* __restrict__ src, u16* dst, int tile, int N,
                                          int w, int lane, int j) {
    constexpr int D = G::D;
    const int blk = w * G::BPW + j;
    const int r = blk * G::RPB + lane / G::CPR;
    const int c = (lane % G::CPR) ^ chunk_swizzle<D>(r);
    const int key = min(tile * G::BC + r, N - 1);
    copy_to_lds16(src, (unsigned)((key * D + c * 8) * 2), dst + blk * 512);
}

// The same for a tile wholly below N: nothing to clamp, so each lane's offset
// within the tile is loop invariant and the tile's position goes into the
// scalar base address (no vector instructions per copy).
template <class G>
__device__ __forceinline__ void dma_block_full(const u16* __restrict__ src, u16* dst, int tile, int w,
                                               int lane, int j) {
    constexpr int D = G::D;
    const int blk = w * G::BPW + j;
    const int r = blk * G::RPB + lane / G::CPR;
    const int c = (lane % G::CPR) ^ chunk_swizzle<D>(r);
    copy_to_lds16(src + (int64_t)tile * G::BC * D, (unsigned)((r * D + c * 8) * 2), dst + blk * 512);
}

template <class G>
__device__ __forceinline__ void dma_tile(const u16* __restrict__ src, u16* dst, int tile, int N,
                                         int w, int lane) {
#pragma unroll
    for (int j = 0; j < G::BPW; ++j) dma_block<G>(src, dst, tile, N, w, lane, j);
}

// Epilogue: combine the two lane halves of each query's sum; store O = o/l
// and LSE = (m + log2 l) ln 2 for rows below N, or, for one segment of a key
// split, the unnormalised o and the (m, l) pair.  Lane (col, g) holds d
// values 32 mt + 8 i4 + 4 g .. + 3 of query row0[b] + col.
template <int D, int QB>
__device__ __forceinline__ void store_rows(const WaveState<D, QB>& st, const AttnArgs& args, int seg,
                                           int bh, const int* row0, int col, int g) {
    constexpr int MT = D / 32;
    const int N = args.N;
    const bool split = args.part_o != nullptr;
    const int64_t part = (int64_t)seg * args.BH + bh;
    float* __restrict__ obase = split ? args.part_o + part * N * D : args.o + (int64_t)bh * N * D;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const float l_tot = st.l[b] + swap32_f32(st.l[b]);
        const int row = row0[b] + col;
        if (row >= N) continue;
        const float inv = split ? 1.0f : 1.0f / l_tot;
        float* orow = obase + (int64_t)row * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const f32x4 r = {st.acc[b][mt][4 * i4 + 0] * inv, st.acc[b][mt][4 * i4 + 1] * inv,
                                 st.acc[b][mt][4 * i4 + 2] * inv, st.acc[b][mt][4 * i4 + 3] * inv};
                *reinterpret_cast<f32x4*>(orow + mt * 32 + 8 * i4 + 4 * g) = r;
            }
        if (g == 0) {
            if (split)
                args.part_ml[part * N + row] = float2{st.m[b], l_tot};
            else
                args.lse[(int64_t)bh * N + row] = (st.m[b] + log2f(l_tot)) * kLn2;
        }
    }
}

// Ring kernel: NW waves of 32 * QB query rows; MINWG workgroups must fit on
// one CU at once (this bounds the registers per wave).  Tile t lives in stage
// t % STAGES; during iteration t the copy of tile t + DIST is in flight, and
// before the iteration's one barrier each wave waits until its own part of
// tile t + 1 has landed.  Used with 4 waves and two workgroups per CU, where
// the two waves on a SIMD belong to different workgroups.
template <bool BF16, int D, bool CAUSAL, int NW, int MINWG, int STAGES, int DIST, int QB>
__global__ void __launch_bounds__(64 * NW, MINWG)
attn_fwd_kernel(AttnArgs args) {
    using G = Geo<D, NW, STAGES, DIST, NW>;
    static_assert(STAGES >= DIST + 1, "a stage still being read would be overwritten");
    constexpr int BR = 32 * QB * NW;   // query rows per workgroup
    __shared__ __attribute__((aligned(1024))) u16 lds[STAGES * G::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int block = w;

    const int N = args.N;
    const float scale_log2 = args.scale_log2;
    // Work item: longest causal tiles first; consecutive workgroups are
    // different heads of one query tile.  Workgroups are dealt round-robin
    // to the 8 XCDs (workgroup i to XCD i % 8), each with its own L2.  When
    // BH is a multiple of 8, XCD x takes the contiguous heads
    // [x BH/8, (x+1) BH/8) of every query tile, so all query tiles of a head,
    // and the query heads that share a K/V head, meet in one L2.
    // With a key split the segments of one query tile follow each other.
    const int bid = blockIdx.x;
    const int per_tile = args.BH * args.nseg;
    const int tt = bid / per_tile;
    // When the whole grid is resident at once (one round, more workgroups
    // than CUs), the first half of the grid takes the longest query tiles and
    // the second half the shortest first: workgroups are placed one per CU
    // before any CU takes a second, so the two that share a CU get
    // complementary amounts of causal work (causal bf16 B1 H32 N2048 D128:
    // +5%).
    const int half = (args.T + 1) / 2;
    const int t = !CAUSAL ? tt : (args.fold && tt >= half) ? tt - half : args.T - 1 - tt;
    const int seg = (bid - tt * per_tile) / args.BH;
    const int j = bid % args.BH;
    const int bh = (args.BH & 7) ? j : (j & 7) * (args.BH >> 3) + (j >> 3);
    // Query head h of batch b reads K/V head h / (H / Hkv) of the same batch
    // (grouped-query attention; Hkv = H is ordinary multi-head attention).
    const int kvh = (bh / args.H) * args.Hkv + (bh % args.H) / (args.H / args.Hkv);
    const u16* __restrict__ q = args.q + (int64_t)bh * N * D;
    const u16* __restrict__ k = args.k + (int64_t)kvh * N * D;
    const u16* __restrict__ v = args.v + (int64_t)kvh * N * D;
    const int row_base = t * BR;
    // Query block b of this wave starts at row0[b]; with QB = 2 the two
    // blocks are adjacent and share their diagonal 64-key tile.
    int row0[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) row0[b] = row_base + (QB * block + b) * 32;
    // Key tiles of this workgroup: kt0 .. ntiles-1.  Segments hold a whole
    // number of query tiles' worth of keys (seg_tiles * 64 is a multiple of
    // BR), so a segment either starts at or before the first row of the query
    // tile, and every row sees at least one of its keys, or lies entirely in
    // the masked future of the tile and the workgroup has nothing to do.
    const int kt0 = seg * args.seg_tiles;
    const int kv_end = min(CAUSAL ? min(row_base + BR, N) : N, (kt0 + args.seg_tiles) * G::BC);
    const int ntiles = (kv_end + G::BC - 1) / G::BC;
    if (kt0 >= ntiles) return;
    // Tiles this wave attends to: kt0 .. last_live (none if its rows are past N).
    const int last_live = row0[0] >= N ? kt0 - 1
                        : min(ntiles - 1, CAUSAL ? (row0[QB - 1] + 31) / G::BC : ntiles - 1);

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
        for (int mt = 0; mt < G::MT; ++mt) st.acc[b][mt] = f32x16{};
        st.m[b] = -INFINITY;
        st.l[b] = 0.0f;
    }
    const FragOffsets<D> fo = frag_offsets<G>(lane);

    auto stage = [&](int it) { return lds + (it % STAGES) * G::STAGE; };
    auto issue = [&](int it) {
        if (it < ntiles && w < G::DMAW) {
            dma_tile<G>(k, stage(it), it, N, w, lane);
            dma_tile<G>(v, stage(it) + G::TILE, it, N, w, lane);
        }
    };
    // End of iteration `it`: tile it+1 complete for this wave (a copy issued
    // later may stay in flight), then the barrier makes it complete for all.
    auto finish = [&](int it) {
        if constexpr (DIST == 2) {
            if (it + 2 < ntiles)
                wait_vmcnt<2 * G::BPW>();
            else
                wait_vmcnt<0>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();
    };
    auto qk = [&](int it, f32x16 (&s)[QB][2]) { qk_tile<BF16, G, QB>(st, fo, stage(it), s); };
    // Finish tile `it`; a wave's diagonal or ragged-tail tile is its last
    // live tile (blocks start at multiples of 32 rows and a wave's blocks lie
    // in one 64-row span, tiles hold 64 keys), so only that one can need
    // masking.
    auto smpv_last = [&](int it, f32x16 (&s)[QB][2]) {
        const int key0 = it * G::BC;
        if ((CAUSAL && key0 + G::BC - 1 > row0[0]) || key0 + G::BC > N)
            softmax_pv_tile<BF16, G, CAUSAL, true, QB>(st, fo, s, stage(it) + G::TILE, lane, key0,
                                                       row0, N, scale_log2);
        else
            softmax_pv_tile<BF16, G, CAUSAL, false, QB>(st, fo, s, stage(it) + G::TILE, lane, key0,
                                                        row0, N, scale_log2);
    };
    auto smpv = [&](int it, f32x16 (&s)[QB][2]) {
        softmax_pv_tile<BF16, G, CAUSAL, false, QB>(st, fo, s, stage(it) + G::TILE, lane, it * G::BC,
                                                    row0, N, scale_log2);
    };

    // Prologue: the first DIST tiles are copied while the Q fragments arrive;
    // one full wait covers both (and tells the compiler Q is ready).
#pragma unroll
    for (int i = 0; i < DIST; ++i) issue(kt0 + i);
    wait_vmcnt<0>();
    __syncthreads();

    // All waves run all ntiles iterations (copies and barriers), whatever
    // they compute; the loops are split so each holds one code variant.
    f32x16 s[QB][2];
    int it = kt0;
    for (; it < last_live; ++it) {
        issue(it + DIST);
        qk(it, s);
        smpv(it, s);
        finish(it);
    }
    if (it == last_live) {
        issue(it + DIST);
        qk(it, s);
        smpv_last(it, s);
        finish(it);
        ++it;
    }
    for (; it < ntiles; ++it) {
        issue(it + DIST);
        finish(it);
    }

    store_rows<D, QB>(st, args, seg, bh, row0, col, g);
}

// ---------------------------------------------------------------------------
// Key-split kernel: for grids of at most one workgroup per CU, where the
// longest workgroup's walk over its key tiles is the critical path.  NW
// waves, one per SIMD with NW = 4: the first NW/2 take 32-row blocks and the
// even key tiles of the workgroup, the other NW/2 the same rows and the odd
// key tiles, each with its own (m, l, o) (the ring kernel's per-tile steps,
// FA page section 4), so a SIMD walks half the keys.  Step j holds tiles 2j
// and 2j+1 in one LDS stage (K and V of each; two stages, the copies of step
// j+1 in flight during step j).  At the end each odd-tile wave hands its
// state to its partner through LDS and the partner merges the two with the
// split-KV law (m = max, each part rescaled to it; "CUDA KV Cache: paged
// storage and long-context decode" (chengzipai.xyz), section 6.4) before
// storing the rows.
// With one wave per SIMD a wave may use 512 registers, and by default the
// compiler then gives every MFMA AGPR accumulators and copies the scores out
// to VGPRs for the softmax; this file is built with VGPR-form MFMAs (build.py),
// which keeps them in VGPRs (222 registers, no copies).  The other kernels
// of the file compile to the same instructions either way.
template <bool BF16, int D, bool CAUSAL, int NW>
__global__ void __launch_bounds__(64 * NW) attn_fwd_ksplit_kernel(AttnArgs args) {
    constexpr int QB = 1;
    using G = Geo<D, NW, 2, 1, NW>;
    constexpr int TILE = G::TILE;
    constexpr int SLOT = 2 * TILE;     // K then V of one tile
    constexpr int STAGE = 2 * SLOT;    // the two tiles of one step
    constexpr int NB = NW / 2;         // 32-row blocks
    constexpr int BR = 32 * NB;        // query rows per workgroup
    constexpr int MT = G::MT;
    __shared__ __attribute__((aligned(1024))) u16 lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int block = w % NB;          // 32-row block
    const int kg = w / NB;             // key group: even (0) or odd (1) tiles

    const int N = args.N;
    const float scale_log2 = args.scale_log2;
    // Work item: longest causal query tiles first; consecutive workgroups
    // are different heads of one query tile, dealt to the 8 XCDs so each XCD
    // keeps a fixed set of heads in its L2.
    const int bid = blockIdx.x;
    const int tt = bid / args.BH;
    const int t_q = CAUSAL ? (args.T - 1 - tt) : tt;
    const int jh = bid % args.BH;
    const int bh = (args.BH & 7) ? jh : (jh & 7) * (args.BH >> 3) + (jh >> 3);
    const int kvh = (bh / args.H) * args.Hkv + (bh % args.H) / (args.H / args.Hkv);
    const u16* __restrict__ q = args.q + (int64_t)bh * N * D;
    const u16* __restrict__ k = args.k + (int64_t)kvh * N * D;
    const u16* __restrict__ v = args.v + (int64_t)kvh * N * D;

    const int row_base = t_q * BR;
    int row0[QB];
    row0[0] = row_base + 32 * block;
    const int kv_end = CAUSAL ? min(row_base + BR, N) : N;
    const int ntiles = (kv_end + G::BC - 1) / G::BC;
    const int nsteps = (ntiles + 1) / 2;
    // The wave's last tile with a visible key (none if its rows are past N).
    const int last_live = row0[0] >= N ? -1
                        : min(ntiles - 1, CAUSAL ? (row0[0] + 31) / G::BC : ntiles - 1);

    WaveState<D, QB> st;
    const int col = lane & 31, g = lane >> 5;
    {
        const int row = row0[0] + col;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            st.qf[0][ks] = row < N ? *reinterpret_cast<const u32x4*>(q + (int64_t)row * D + ks * 16 + 8 * g)
                                   : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) st.acc[0][mt] = f32x16{};
        st.m[0] = -INFINITY;
        st.l[0] = 0.0f;
    }
    const FragOffsets<D> fo = frag_offsets<G>(lane);

    auto stage = [&](int j) { return lds + (j & 1) * STAGE; };
    // Copies of step j (tiles 2j and 2j+1), shared by all 8 waves.
    auto issue = [&](int j) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int tile = 2 * j + s2;
            if (tile < ntiles) {
                u16* dst = stage(j) + s2 * SLOT;
#pragma unroll
                for (int c = 0; c < G::BPW; ++c) {
                    if ((tile + 1) * G::BC <= N) {
                        dma_block_full<G>(k, dst, tile, w, lane, c);
                        dma_block_full<G>(v, dst + TILE, tile, w, lane, c);
                    } else {
                        dma_block<G>(k, dst, tile, N, w, lane, c);
                        dma_block<G>(v, dst + TILE, tile, N, w, lane, c);
                    }
                }
            }
        }
    };
    // End of step j: the copies of step j+1 complete for this wave, then for all.
    auto finish = [&]() {
        wait_vmcnt<0>();
        __syncthreads();
    };

    issue(0);
    finish();
    // Every wave runs all nsteps steps (copies and barriers), whatever it
    // computes; the loops are split so each holds one code variant.  Stage
    // (j+1) & 1, which step j's copies fill, held step j-1.
    f32x16 s[QB][2];
    int j = 0;
    for (; 2 * j + kg < last_live; ++j) {
        issue(j + 1);
        const u16* kt = stage(j) + kg * SLOT;
        qk_tile<BF16, G, QB>(st, fo, kt, s);
        softmax_pv_tile<BF16, G, CAUSAL, false, QB>(st, fo, s, kt + TILE, lane, (2 * j + kg) * G::BC,
                                                    row0, N, scale_log2);
        finish();
    }
    if (j < nsteps && 2 * j + kg == last_live) {
        issue(j + 1);
        const u16* kt = stage(j) + kg * SLOT;
        const int key0 = (2 * j + kg) * G::BC;
        qk_tile<BF16, G, QB>(st, fo, kt, s);
        if ((CAUSAL && key0 + G::BC - 1 > row0[0]) || key0 + G::BC > N)
            softmax_pv_tile<BF16, G, CAUSAL, true, QB>(st, fo, s, kt + TILE, lane, key0, row0, N,
                                                       scale_log2);
        else
            softmax_pv_tile<BF16, G, CAUSAL, false, QB>(st, fo, s, kt + TILE, lane, key0, row0, N,
                                                        scale_log2);
        finish();
        ++j;
    }
    for (; j < nsteps; ++j) {
        issue(j + 1);
        finish();
    }

    // Merge: the odd-tile wave of each row block passes (o, m, l) to its
    // partner through LDS (free after the last barrier), lane to lane, as
    // 16-byte vectors (a lane's record is padded to 68 floats: a multiple of
    // four, and lanes 4 banks apart).
    constexpr int NR = MT * 16 + 4;
    f32x4* xch = reinterpret_cast<f32x4*>(reinterpret_cast<float*>(lds) + (block * 64 + lane) * NR);
    if (kg == 1) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                xch[mt * 4 + i4] = f32x4{st.acc[0][mt][4 * i4], st.acc[0][mt][4 * i4 + 1],
                                         st.acc[0][mt][4 * i4 + 2], st.acc[0][mt][4 * i4 + 3]};
        xch[MT * 4] = f32x4{st.m[0], st.l[0], 0.0f, 0.0f};
    }
    __syncthreads();
    if (kg == 1) return;
    const f32x4 ml = xch[MT * 4];
    const float m = fmaxf(st.m[0], ml[0]);
    const float a0 = online_rescale(st.m[0], m);
    const float a1 = online_rescale(ml[0], m);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 o1 = xch[mt * 4 + i4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                st.acc[0][mt][4 * i4 + e] = st.acc[0][mt][4 * i4 + e] * a0 + o1[e] * a1;
        }
    st.l[0] = st.l[0] * a0 + ml[1] * a1;
    st.m[0] = m;
    store_rows<D, QB>(st, args, 0, bh, row0, col, g);
}

// ---------------------------------------------------------------------------
// Key-half unit kernel: 8 waves of 32 query rows (256 rows per workgroup, one
// workgroup per CU), two waves per SIMD, all computing.
//
// Work is cut into units of one key half (32 keys) of one product:
// QKa(t), QKb(t) compute S^T for key half 0 / 1 of tile t, and PVa(t), PVb(t)
// accumulate O^T += V^T P^T for key half 0 / 1.  A wave runs them in the order
//     X(t) = QKa(t), PVb(t-1)        Y(t) = QKb(t), PVa(t)
// so the exponentials of a key half are spread over the two units that follow
// its QK unit: one value per MFMA (fma and exp; every other MFMA a 16-bit pack
// and a pair sum).  That is three VALU instructions per MFMA, which issue
// while the wave's own MFMA executes; the work is software-pipelined over the
// MFMA steps (a value's exp one step after its fma, the pack two steps after,
// the sum three steps after) so that no instruction waits on one issued
// beside the same MFMA.  (FA page, section 4: the recurrence; the order of
// its steps within a tile is unchanged, only their interleaving is.)
//
// Reference max and bound.  The exponentials of a key half are taken against
// the query's current reference max m before that half's scores are
// examined; the half's sum of P then decides: if every lane's sum is at most
// 2^8 (so every P is), nothing else is done.  Otherwise each query whose two
// lanes include such a lane moves m to max(m, the half's max), rescales o and
// l, and the half's exponentials are taken again.  A query's decision uses
// only its own scores, so rows never influence each other's bits.  Before the
// first half no reference exists and the check always fails.
//
// Operands stream from LDS through a 4-deep register ring over the fragments
// of an iteration (K(t) half 0, V(t-1) half 1, K(t) half 1, V(t) half 0).
// Tile t's V is still read in X(t+1), so a copy may only overwrite a tile two
// iterations old: K and V each have four stages, copies run two tiles ahead,
// one barrier per tile.  LDS holds the four K stages, then the four V stages;
// tile t uses stage (t - kt0) % 4, a compile-time value in the loop unrolled
// by four, so every fragment address is a per-lane base plus an immediate.
// Every wave computes every tile of its workgroup: a tile wholly above a
// wave's rows is fully masked (P = 0 leaves o and l unchanged) and runs while
// the SIMDs of later rows work on the same tile.

// A key half's P sum at most 2^8 keeps every P of it at most 2^8.
constexpr float kSumBound = 256.0f;

// P = 2^(s * scale_log2 - m) for the 16 scores of one key half held by this
// lane, packed to 16-bit MFMA operands (p0: values 0-7, p1: values 8-15);
// returns the lane's share of the half's sum.  The unit kernel's pipelined
// exponentials compute exactly this, in this order.
template <bool BF16>
__device__ __forceinline__ float half_exp(const f32x16& s, float m, float scale_log2, u32x4& p0,
                                          u32x4& p1) {
    using M = Mma<BF16>;
    float p[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) p[j] = fast_exp2(fmaf(s[j], scale_log2, -m));
    p0 = u32x4{M::pack(p[0], p[1]), M::pack(p[2], p[3]), M::pack(p[4], p[5]), M::pack(p[6], p[7])};
    p1 = u32x4{M::pack(p[8], p[9]), M::pack(p[10], p[11]), M::pack(p[12], p[13]),
               M::pack(p[14], p[15])};
    float r0 = 0.0f, r1 = 0.0f;
    if constexpr (M::kSumRounded) {
        r0 = M::sum2(p0[0], r0);
        r1 = M::sum2(p0[1], r1);
        r0 = M::sum2(p0[2], r0);
        r1 = M::sum2(p0[3], r1);
        r0 = M::sum2(p1[0], r0);
        r1 = M::sum2(p1[1], r1);
        r0 = M::sum2(p1[2], r0);
        r1 = M::sum2(p1[3], r1);
    } else {
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            r0 += p[j];
            r1 += p[j + 1];
        }
    }
    return r0 + r1;
}

template <bool BF16, int D, bool CAUSAL, int QB, int NWV>
__global__ void __launch_bounds__(64 * NWV, 1) attn_fwd_units_kernel(AttnArgs args) {
    using G = Geo<D, NWV, 4, 2, NWV>;
    using M = Mma<BF16>;
    constexpr int KS = G::KS;       // K fragments per key half (d steps)
    constexpr int MT = G::MT;
    constexpr int NHV = 2 * MT;     // V fragments per key half
    static_assert(KS == NHV, "QK and PV units have the same number of MFMAs");
    constexpr int NU = KS;          // operand fragments per unit (each feeds QB MFMAs)
    constexpr int VPQ = 8 / KS;     // hosted values per MFMA step
    constexpr int HV = 8 * QB;      // hosted values per unit
    constexpr int RW = 32 * QB * NWV;   // query rows per workgroup
    constexpr int TILE = G::TILE;
    constexpr int BPW = G::BPW;
    constexpr int NST = 4;          // stages of K and of V
    constexpr int RING = 4;         // operand fragments in flight
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    typedef __attribute__((address_space(3))) u16 lds_u16;
    __shared__ __attribute__((aligned(1024))) u16 lds[2 * NST * TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Waves w and w + 4 share a SIMD; they take adjacent row spans so their
    // causal work is equal.  A wave owns QB adjacent 32-row blocks.
    const int block = NWV == 8 ? 2 * (w & 3) + (w >> 2) : w;

    const int N = args.N;
    const float scale_log2 = args.scale_log2;
    // Work item: as in the ring kernel (longest causal tiles first; heads of
    // one query tile dealt to the 8 XCDs so each XCD keeps a fixed set).
    const int bid = blockIdx.x;
    const int per_tile = args.BH * args.nseg;
    const int tt = bid / per_tile;
    const int t_q = CAUSAL ? (args.T - 1 - tt) : tt;
    const int seg = (bid - tt * per_tile) / args.BH;
    const int j = bid % args.BH;
    const int bh = (args.BH & 7) ? j : (j & 7) * (args.BH >> 3) + (j >> 3);
    const int kvh = (bh / args.H) * args.Hkv + (bh % args.H) / (args.H / args.Hkv);
    const u16* __restrict__ q = args.q + (int64_t)bh * N * D;
    const u16* __restrict__ k = args.k + (int64_t)kvh * N * D;
    const u16* __restrict__ v = args.v + (int64_t)kvh * N * D;

    const int row_base = t_q * RW;
    int row0[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) row0[b] = row_base + (QB * block + b) * 32;
    const int kt0 = seg * args.seg_tiles;
    const int kv_end = min(CAUSAL ? min(row_base + RW, N) : N, (kt0 + args.seg_tiles) * G::BC);
    const int ntiles = (kv_end + G::BC - 1) / G::BC;
    if (kt0 >= ntiles) return;
    const int T = ntiles - 1;       // last tile

    WaveState<D, QB> st;
    const int col = lane & 31, g = lane >> 5;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const int row = row0[b] + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            st.qf[b][ks] = row < N ? *reinterpret_cast<const u32x4*>(q + (int64_t)row * D + ks * 16 + 8 * g)
                                   : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) st.acc[b][mt] = f32x16{};
        st.m[b] = -INFINITY;
        st.l[b] = 0.0f;
    }
    // Bound on a key half's P sum; negative until the first reference max.
    float lim = -1.0f;

    // Per-lane LDS fragment bases of stage 0 (pinned so the compiler keeps
    // base + offset sums out of registers: every offset fits the immediate).
    const FragOffsets<D> fo = frag_offsets<G>(lane);
    const lds_u32x4* kp[KS];
    const lds_s16x4* vp[MT][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        kp[ks] = (const lds_u32x4*)((const lds_u16*)lds + fo.k[ks]);
        asm volatile("" : "+v"(kp[ks]));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            vp[mt][r] = (const lds_s16x4*)((const lds_u16*)lds + NST * TILE + fo.v[mt][r]);
            asm volatile("" : "+v"(vp[mt][r]));
        }
    auto k_stage = [&](int s_) __attribute__((always_inline)) { return lds + s_ * TILE; };
    auto v_stage = [&](int s_) __attribute__((always_inline)) { return lds + (NST + s_) * TILE; };
    auto issue = [&](int t) __attribute__((always_inline)) {
        if (t <= T) {
            const int s_ = (t - kt0) % NST;
            dma_tile<G>(k, k_stage(s_), t, N, w, lane);
            dma_tile<G>(v, v_stage(s_), t, N, w, lane);
        }
    };
    // The same copies spread over the four units of an iteration (copy i of
    // the wave's 2 * BPW goes with unit 4 i / (2 BPW)): issued together after
    // the barrier, the copies of all waves queued behind each other and held
    // the waves' first MFMAs back.
    // Tiles below TF lie wholly below N (all but a ragged last tile) and take
    // the unclamped copy.
    const int TF = (T + 1) * G::BC <= N ? T + 1 : T;
    auto issue_part = [&](int t, int u) __attribute__((always_inline)) {
        if (__builtin_expect(t < TF, 1)) {
            const int s_ = (t - kt0) % NST;
#pragma unroll
            for (int i = 0; i < 2 * BPW; ++i) {
                if ((4 * i) / (2 * BPW) != u) continue;
                if (i < BPW)
                    dma_block_full<G>(k, k_stage(s_), t, w, lane, i);
                else
                    dma_block_full<G>(v, v_stage(s_), t, w, lane, i - BPW);
            }
        } else if (t <= T) {
            const int s_ = (t - kt0) % NST;
#pragma unroll
            for (int i = 0; i < 2 * BPW; ++i) {
                if ((4 * i) / (2 * BPW) != u) continue;
                if (i < BPW)
                    dma_block<G>(k, k_stage(s_), t, N, w, lane, i);
                else
                    dma_block<G>(v, v_stage(s_), t, N, w, lane, i - BPW);
            }
        }
    };
    // Fragment e of the operand stream of an iteration whose tile is in stage
    // par: units 0..3 = K(t) half 0, V(t-1) half 1, K(t) half 1, V(t) half 0.
    // V fragment f of key half kb covers key group 2 kb + f / MT, d block f % MT.
    auto frag = [&](int par, int e) __attribute__((always_inline)) {
        const int unit = e / NU, f = e % NU;
        if (unit == 0 || unit == 2) return kp[f][(par * TILE + (unit / 2) * 32 * D) / 8];
        const int sp = unit == 1 ? (par + NST - 1) % NST : par;
        const int kb = unit == 1 ? 1 : 0;
        const int o = (sp * TILE + (2 * kb + f / MT) * 16 * D) / 4;
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp[f % MT][0] + o));
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp[f % MT][1] + o));
        const auto lo = __builtin_bit_cast(unsigned long long, x0);
        const auto hi = __builtin_bit_cast(unsigned long long, x1);
        return u32x4{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi, (unsigned)(hi >> 32)};
    };

    f32x16 s[2][QB];    // S^T of key half 0 and 1, per row block
    u32x4 pf[QB][4];    // 16-bit P^T of the four 16-key groups, per row block
    float r0[QB], r1[QB];   // the lane's half sums (even / odd pairs)
#pragma unroll
    for (int b = 0; b < QB; ++b) r0[b] = r1[b] = 0.0f;
    float hx[HV], hp[HV];
    unsigned hk[HV / 2];
    // Hosted work: values hi0 .. hi0+7 of key half hkb of each row block
    // (value vv: row block vv / 8), VP per MFMA step; step jstep runs value
    // vv's fma when jstep == vv / VP, its exp one step later, the pack of an
    // odd vv and its predecessor two steps later and the pair's sum three
    // steps later.  Steps past the unit's last MFMA drain after it.  Same
    // arithmetic and order as half_exp.  The empty asm statements anchor each
    // result where it is computed: the work is pure and would otherwise sink
    // out of the MFMA stream it fills.
    auto host_step = [&](int hkb, int hi0, int VP, int jstep) __attribute__((always_inline)) {
#pragma unroll
        for (int vv = 0; vv < HV; ++vv) {
            const int b = vv / 8, idx = hi0 + vv % 8;
            const int s0 = vv / VP;
            if (jstep == s0 + 1) {
                hp[vv] = fast_exp2(hx[vv]);
                asm volatile("" ::"v"(hp[vv]));
            }
            if (jstep == s0) {
                hx[vv] = fmaf(s[hkb][b][idx], scale_log2, -st.m[b]);
                asm volatile("" ::"v"(hx[vv]));
            }
            if ((vv & 1) && jstep == s0 + 2) {
                hk[vv >> 1] = M::pack(hp[vv - 1], hp[vv]);
                asm volatile("" ::"v"(hk[vv >> 1]));
            }
            if ((vv & 1) && jstep == s0 + 3) {
                const int pk_i = idx >> 1;   // pair index within the half
                if constexpr (M::kSumRounded) {
                    if (pk_i & 1)
                        r1[b] = M::sum2(hk[vv >> 1], r1[b]);
                    else
                        r0[b] = M::sum2(hk[vv >> 1], r0[b]);
                } else {
                    r0[b] += hp[vv - 1];
                    r1[b] += hp[vv];
                }
                asm volatile("" ::"v"(r0[b]), "v"(r1[b]));
                pf[b][2 * hkb + pk_i / 4][pk_i % 4] = hk[vv >> 1];
            }
        }
    };
    auto host_drain = [&](int hkb, int hi0, int VP, int from) __attribute__((always_inline)) {
#pragma unroll
        for (int jstep = from; jstep < HV / VP + 3; ++jstep) host_step(hkb, hi0, VP, jstep);
    };
    // Scores of keys after the query (causal) or past N set to -inf.  Lane
    // (col, g) holds keys 8(i/4) + 4g + i%4 of key half kb for query
    // row0[b] + col.
    auto mask_half = [&](int kb, int key0) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            const int lim_c = min(CAUSAL ? row0[b] + col - key0 : (1 << 30), N - 1 - key0) - 4 * g;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int c = kb * 32 + 8 * (i >> 2) + (i & 3);
                s[kb][b][i] = c > lim_c ? -INFINITY : s[kb][b][i];
            }
        }
    };
    auto is_masked = [&](int t) __attribute__((always_inline)) {
        const int key0 = t * G::BC;
        return (CAUSAL && key0 + G::BC - 1 > row0[0]) || key0 + G::BC > N;
    };
    // Key half kb's exponentials are complete: the bound check, the rare
    // move of the reference max, and the half's sum into l.
    auto settle = [&](int kb) __attribute__((always_inline)) {
        float rs[QB];
        bool bad = false;
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            rs[b] = r0[b] + r1[b];
            r0[b] = 0.0f;
            r1[b] = 0.0f;
            bad = bad || !(rs[b] <= lim);
        }
        if (__builtin_amdgcn_ballot_w64(bad) != 0) {
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                // Both lanes of a query take the same decision; the exchanges
                // run in every lane (under a partial EXEC mask they would read
                // stale values).
                const float rs_pair = swap32_f32(rs[b]);
                const bool need = !(rs[b] <= lim && rs_pair <= lim);
                float hm = s[kb][b][0];
#pragma unroll
                for (int i = 1; i < 16; ++i) hm = fmaxf(hm, s[kb][b][i]);
                hm = fmaxf(hm, swap32_f32(hm)) * scale_log2;
                const float m_new = need ? fmaxf(st.m[b], hm) : st.m[b];
                const float alpha = need ? online_rescale(st.m[b], m_new) : 1.0f;
                st.l[b] *= alpha;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) st.acc[b][mt] *= alpha;
                st.m[b] = m_new;
                rs[b] = half_exp<BF16>(s[kb][b], m_new, scale_log2, pf[b][2 * kb], pf[b][2 * kb + 1]);
            }
            lim = kSumBound;
        }
#pragma unroll
        for (int b = 0; b < QB; ++b) st.l[b] += rs[b];
    };

    // One iteration: the fragment stream through the ring, one loop per
    // unit, with the settle and mask steps between units.  HEAD (t = kt0):
    // there is no PVb(t-1); half 0's first exponentials run alone.
    auto iteration = [&](auto par_c, auto head_c, int t) __attribute__((always_inline)) {
        constexpr int par = decltype(par_c)::value;
        constexpr bool HEAD = decltype(head_c)::value;
        u32x4 ring[RING];
        // Stream position i fragments after (unit u, fragment f); HEAD skips
        // unit 1.  At or past 4 * NU: beyond this iteration.
        auto ahead = [&](int u, int f, int i) __attribute__((always_inline)) {
            int uu = u, ff = f + i;
            while (ff >= NU && uu < 4) {
                ff -= NU;
                uu = (HEAD && uu == 0) ? 2 : uu + 1;
            }
            return uu * NU + ff;
        };
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < RING; ++i) ring[i] = frag(par, ahead(0, 0, i));
        int rslot = 0;
        auto unit_loop = [&](auto u_c) __attribute__((always_inline)) {
            constexpr int u = decltype(u_c)::value;
#pragma unroll
            for (int f = 0; f < NU; ++f) {
                const u32x4 a = ring[(rslot + f) % RING];
#pragma unroll
                for (int b = 0; b < QB; ++b) {
                    if constexpr (u == 0 || u == 2) {
                        if (f == 0) s[u / 2][b] = f32x16{};
                        s[u / 2][b] = M::run(a, st.qf[b][f], s[u / 2][b]);
                    } else {
                        const int kb = u == 1 ? 1 : 0;
                        st.acc[b][f % MT] = M::run(a, pf[b][2 * kb + f / MT], st.acc[b][f % MT]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (b == 0) {
                        const int e = ahead(u, f, RING);
                        if (e < 4 * NU) ring[(rslot + f) % RING] = frag(par, e);
                        if (!HEAD && f == 0) issue_part(t + 2, u);
                    }
                    // X: QKa hosts values 8..15 of half 1 (tile t-1), PVb
                    // values 0..7 of half 0; Y: QKb hosts values 8..15 of
                    // half 0, PVa values 0..7 of half 1.
                    const int js = f * QB + b;
                    if constexpr (u == 0) {
                        if (!HEAD) host_step(1, 8, VPQ, js);
                    } else if constexpr (u == 1) {
                        host_step(0, 0, VPQ, js);
                    } else if constexpr (u == 2) {
                        host_step(0, 8, VPQ, js);
                    } else {
                        host_step(1, 0, VPQ, js);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            rslot = (rslot + NU) % RING;
        };
        unit_loop(std::integral_constant<int, 0>{});
        if (!HEAD) {
            host_drain(1, 8, VPQ, NU * QB);
            settle(1);
        }
        if (is_masked(t)) mask_half(0, t * G::BC);
        if (HEAD) {
            host_drain(0, 0, 1, 0);
        } else {
            unit_loop(std::integral_constant<int, 1>{});
            host_drain(0, 0, VPQ, NU * QB);
        }
        __builtin_amdgcn_sched_barrier(0);
        unit_loop(std::integral_constant<int, 2>{});
        host_drain(0, 8, VPQ, NU * QB);
        settle(0);
        if (is_masked(t)) mask_half(1, t * G::BC);
        __builtin_amdgcn_sched_barrier(0);
        unit_loop(std::integral_constant<int, 3>{});
        host_drain(1, 0, VPQ, NU * QB);
        __builtin_amdgcn_sched_barrier(0);
    };
    // End of iteration t: tile t+1 complete for this wave (the copy of t+2
    // may still fly), then the barrier makes it complete for all.
    auto finish = [&](int t) __attribute__((always_inline)) {
        if (t + 2 <= T)
            wait_vmcnt<2 * BPW>();
        else
            wait_vmcnt<0>();
        __syncthreads();
    };

    // Prologue: the first two tiles are copied while the Q fragments arrive;
    // one full wait covers both (and tells the compiler Q is ready).
    issue(kt0);
    issue(kt0 + 1);
    wait_vmcnt<0>();
    __syncthreads();
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    issue(kt0 + 2);
    iteration(P0{}, std::true_type{}, kt0);
    finish(kt0);
    auto step = [&](auto par_c, int t) __attribute__((always_inline)) {
        iteration(par_c, std::false_type{}, t);
        finish(t);
    };
    // Tiles kt0+1 .. T (stages 1, 2, 3, 0, ...) in groups of four, then the
    // remainder: the loop keeps a single exit (a second exit gave the O
    // accumulators two register homes).
    const int nmain = T - kt0;
    const int nq = nmain / 4;
    int t = kt0 + 1;
    for (int i = 0; i < nq; ++i, t += 4) {
        step(P1{}, t);
        step(P2{}, t + 1);
        step(P3{}, t + 2);
        step(P0{}, t + 3);
    }
    const int nr = nmain - 4 * nq;
    if (nr >= 1) step(P1{}, t++);
    if (nr >= 2) step(P2{}, t++);
    if (nr >= 3) step(P3{}, t++);
    // Tail: half 1 of tile T (exponentials, settle, PVb(T)).
    {
        host_drain(1, 8, 1, 0);
        settle(1);
        const u16* vt = v_stage((T - kt0) % NST);
#pragma unroll
        for (int f = 0; f < NHV; ++f) {
            const u16* base = vt + (2 + f / MT) * 16 * D;
            const u32x4 a = tr16_b64x2(base + fo.v[f % MT][0], base + fo.v[f % MT][1]);
#pragma unroll
            for (int b = 0; b < QB; ++b)
                st.acc[b][f % MT] = M::run(a, pf[b][2 + f / MT], st.acc[b][f % MT]);
        }
    }

    store_rows<D, QB>(st, args, seg, bh, row0, col, g);
}

// ---------------------------------------------------------------------------
// Tile-lagged pipeline kernel: 8 waves of 32 query rows (256 rows per
// workgroup, one workgroup per CU), two waves per SIMD.
//
// Iteration i of a wave issues, one after the other, the MFMAs of QK (S^T =
// K Q^T) for key half 1 of tile i and key half 0 of tile i+1, alternating
// with those of PV(i-1) (O^T += V^T P^T of the tile before), and hosts under
// them the softmax of tile i, key half 0 in the first half of the iteration
// and key half 1 in the second:
// per MFMA one score's fma and exp (two at D = 64), the FP32 sum of the
// exponentials and every other value one 16-bit pack.  P(i) is complete at
// the end of iteration i and first read by PV(i) in iteration i+1, so no MFMA
// ever waits on the exponentials, and the check that accepts P(i) (below)
// runs once per tile, at the iteration end, before the barrier.  Each key
// half's scores are consumed before the next tile's scores of that half are
// written, so one buffer of scores suffices.  (FA page,
// section 4: the recurrence is unchanged; only the order in which its steps
// of different tiles interleave is.)
//
// Reference max and bound.  The first tile's scores set the reference max m
// of each query (its exact maximum).  Every later tile's exponentials are
// taken against the current m; if a lane's sum over the tile exceeds 2^8
// (so some P might exceed it) or is NaN, each query whose two lanes include
// such a lane moves m to max(m, tile max), rescales o and l, and takes the
// tile's exponentials again (half 0's scores, overwritten by then, are
// recomputed from K of the tile, still in LDS).  A query's decision depends only on its own
// scores.  Between moves every P is at most 2^8, exact in fp16 and bf16
// range, and numerator and denominator share m, so O = o / l is unchanged.
//
// LDS holds four K stages then four V stages.  Iteration i reads K(i),
// K(i+1) and V(i-1) and copies K(i+3) and V(i+2) (direct global -> LDS
// copies, issued early in the iteration); the barrier that ends iteration i
// certifies the copies issued in iteration i-1, i.e. the data iteration i+2
// reads first, so the operand ring runs across iteration boundaries and the
// next iteration's first fragments are read before the barrier.  Tile t's K and V use stage
// (t - kt0) mod 4; the loop is unrolled by four so every LDS address is a
// per-lane base plus an immediate.
//
// Causal masking (and the ragged key tail) is applied in place to S(i), key
// half 0 at the start of iteration i and key half 1 once its QK is done, only
// for tiles that need it: the four diagonal tiles
// of the workgroup and a ragged last tile.  A tile wholly above a wave's rows
// is fully masked (P = 0); the wave still computes it while it has other work
// in the same iteration, and skips every iteration from the one where none is
// left (it then only copies and meets the barriers).
template <bool BF16, int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) attn_fwd_pipe_kernel(AttnArgs args) {
    constexpr int QB = 1;             // 32-row blocks per wave
    constexpr int NW = 8;             // waves per workgroup
    using G = Geo<D, NW, 4, 2, NW>;
    using M = Mma<BF16>;
    constexpr int KS = G::KS;         // K fragments per key half
    constexpr int MT = G::MT;         // 32-row d blocks of O^T
    constexpr int NQK = 2 * KS;       // K fragments per tile
    constexpr int NPV = 4 * MT;       // V fragments per tile
    static_assert(NQK == NPV, "QK and PV take the same number of fragments");
    constexpr int NSTEP = NQK + NPV;  // fragments per iteration (each feeds QB MFMAs)
    constexpr int NVAL = 32 * QB;     // scores per lane per tile
    constexpr int VPS = NVAL / NSTEP; // hosted values per fragment step
    constexpr int TILE = G::TILE;
    constexpr int BPW = G::BPW;       // 1 KiB copies per wave per K (or V) tile
    constexpr int NST = 4;            // stages of K and of V
    constexpr int RING = 4;           // operand fragments in flight
    constexpr int RW = 256;           // query rows per workgroup
    constexpr float kBound = 256.0f;  // a lane's tile sum at most 2^8 keeps every P at most 2^8
    typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    typedef __attribute__((address_space(3))) u16 lds_u16;
    __shared__ __attribute__((aligned(1024))) u16 lds[2 * NST * TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Waves w and w + 4 share a SIMD (w mod 4) and take 32-row blocks w mod 4
    // and 7 - w mod 4: on the causal diagonal the waves of the early blocks
    // run out of work first, and each SIMD then keeps one busy wave.
    const int block0 = w < 4 ? w : 11 - w;

    const int N = args.N;
    const float scale_log2 = args.scale_log2;
    // Work item: longest causal query tiles first; the heads of one query
    // tile are dealt to the 8 XCDs so each XCD keeps a fixed set of heads
    // (and of shared K/V heads) in its L2.
    const int bid = blockIdx.x;
    const int per_tile = args.BH * args.nseg;
    const int tt = bid / per_tile;
    const int t_q = CAUSAL ? (args.T - 1 - tt) : tt;
    const int seg = (bid - tt * per_tile) / args.BH;
    const int jh = bid % args.BH;
    const int bh = (args.BH & 7) ? jh : (jh & 7) * (args.BH >> 3) + (jh >> 3);
    const int kvh = (bh / args.H) * args.Hkv + (bh % args.H) / (args.H / args.Hkv);
    const u16* __restrict__ q = args.q + (int64_t)bh * N * D;
    const u16* __restrict__ k = args.k + (int64_t)kvh * N * D;
    const u16* __restrict__ v = args.v + (int64_t)kvh * N * D;

    const int row_base = t_q * RW;
    int row0[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) row0[b] = row_base + 32 * (block0 + b);
    const int kt0 = seg * args.seg_tiles;
    const int kv_end = min(CAUSAL ? min(row_base + RW, N) : N, (kt0 + args.seg_tiles) * G::BC);
    const int ntiles = (kv_end + G::BC - 1) / G::BC;
    if (kt0 >= ntiles) return;
    const int T = ntiles - 1;   // last key tile
    // Tiles from first_masked on need the causal mask (keys past the
    // workgroup's first row); a tile reaching past N needs the tail mask.
    const int first_masked = CAUSAL ? row_base / G::BC : T + 1;

    WaveState<D, QB> st;
    const int col = lane & 31, g = lane >> 5;
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const int row = row0[b] + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            st.qf[b][ks] = row < N ? *reinterpret_cast<const u32x4*>(q + (int64_t)row * D + ks * 16 + 8 * g)
                                   : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) st.acc[b][mt] = f32x16{};
        st.l[b] = 0.0f;
    }

    // Per-lane LDS fragment bases of stage 0 (pinned so that every fragment
    // address stays a base plus an immediate offset).
    const FragOffsets<D> fo = frag_offsets<G>(lane);
    const lds_u32x4* kp[KS];
    const lds_s16x4* vp[MT][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        kp[ks] = (const lds_u32x4*)((const lds_u16*)lds + fo.k[ks]);
        asm volatile("" : "+v"(kp[ks]));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            vp[mt][r] = (const lds_s16x4*)((const lds_u16*)lds + NST * TILE + fo.v[mt][r]);
            asm volatile("" : "+v"(vp[mt][r]));
        }
    auto k_stage = [&](int s_) __attribute__((always_inline)) { return lds + s_ * TILE; };
    auto v_stage = [&](int s_) __attribute__((always_inline)) { return lds + (NST + s_) * TILE; };
    // K fragment (key half h, d step ks) and V^T fragment (16-key group kg,
    // d block mt) of the tiles in stages sk and sv.
    auto kfrag = [&](int sk, int h, int ks) __attribute__((always_inline)) {
        return kp[ks][(sk * TILE + h * 32 * D) / 8];
    };
    auto vfrag = [&](int sv, int kg, int mt) __attribute__((always_inline)) {
        const int o = (sv * TILE + kg * 16 * D) / 4;
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp[mt][0] + o));
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vp[mt][1] + o));
        const auto lo = __builtin_bit_cast(unsigned long long, x0);
        const auto hi = __builtin_bit_cast(unsigned long long, x1);
        return u32x4{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi, (unsigned)(hi >> 32)};
    };
    // Element e of the operand stream of an iteration of phase PH (tile i
    // with (i - kt0) mod 4 = PH): even e the K fragments, first those of key
    // half 1 of tile i, then those of key half 0 of tile i+1 (d step order);
    // odd e the V^T fragments of tile i-1 in PV order (key group, d block).
    auto frag = [&](int PH, int e) __attribute__((always_inline)) {
        const int n = e >> 1;
        if ((e & 1) == 0) return n < KS ? kfrag(PH, 1, n) : kfrag((PH + 1) % NST, 0, n - KS);
        return vfrag((PH + 3) % NST, n / MT, n % MT);
    };
    // Copy part c (of 2 BPW) of the copies of iteration i (phase PH): K(i+3)
    // into stage PH+3 and V(i+2) into stage PH+2.  A tile wholly below N takes
    // the unclamped copy.
    auto copy_part = [&](int PH, int i, int c) __attribute__((always_inline)) {
        if (c < BPW) {
            const int t = i + 3;
            if (t <= T) {
                if ((t + 1) * G::BC <= N)
                    dma_block_full<G>(k, k_stage((PH + 3) % NST), t, w, lane, c);
                else
                    dma_block<G>(k, k_stage((PH + 3) % NST), t, N, w, lane, c);
            }
        } else {
            const int t = i + 2;
            if (t <= T) {
                if ((t + 1) * G::BC <= N)
                    dma_block_full<G>(v, v_stage((PH + 2) % NST), t, w, lane, c - BPW);
                else
                    dma_block<G>(v, v_stage((PH + 2) % NST), t, N, w, lane, c - BPW);
            }
        }
    };

    // S^T += K Q^T (first: S^T = K Q^T) and O^T += V^T P^T.
    auto mm_qk = [&](f32x16& d, const u32x4& a, const u32x4& bq, auto first_c) __attribute__((always_inline)) {
        d = M::run(a, bq, decltype(first_c)::value ? f32x16{} : d);
    };
    auto mm_pv = [&](f32x16& acc, const u32x4& a, const u32x4& bp) __attribute__((always_inline)) {
        acc = M::run(a, bp, acc);
    };

    f32x16 s[QB][2];       // S^T: [row block][key half]
    u32x4 pf[2][QB][4];    // 16-bit P^T: [buffer][row block][16-key group]
    float x[NVAL], p[NVAL];
    float r0[QB], r1[QB];  // the lane's tile sum per row block (even / odd values)
    u32x4 ring[RING];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        r0[b] = 0.0f;
        r1[b] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pf[0][b][j] = u32x4{0u, 0u, 0u, 0u};
            pf[1][b][j] = u32x4{0u, 0u, 0u, 0u};
        }
    }

    // Scores of keys after the query (causal) or past N set to -inf, in key
    // half h of tile i (sc: that half's scores of each row block).  Lane
    // (col, g) holds keys 8(j/4) + 4g + j%4 of the half for query
    // row0[b] + col.
    auto mask_half = [&](f32x16 (&sc)[QB], int i, int h) __attribute__((always_inline)) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            const int key0 = i * G::BC + 32 * h;
            const int lim = min(CAUSAL ? row0[b] + col - key0 : (1 << 30), N - 1 - key0) - 4 * g;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int c = 8 * (j >> 2) + (j & 3);
                sc[b][j] = c > lim ? -INFINITY : sc[b][j];
            }
        }
    };
    auto mask_s = [&](int i, int h) __attribute__((always_inline)) {
        f32x16 t[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) t[b] = s[b][h];
        mask_half(t, i, h);
#pragma unroll
        for (int b = 0; b < QB; ++b) s[b][h] = t[b];
    };
    auto needs_mask = [&](int i) __attribute__((always_inline)) {
        return i >= first_masked || (i + 1) * G::BC > N;
    };

    // Hosted work of step `step` of an iteration whose scores are in buffer
    // sb and whose P goes to buffer sb: value vv (key half vv / (16 QB), row
    // block (vv / 16) % QB, element vv % 16) has its fma at step vv / VPS,
    // its exp one step later, its sum and (odd vv, with vv - 1) its pack one
    // step after that.  The empty asm statements anchor each result where it
    // is computed, so the work stays spread over the MFMA stream.
    auto host_step = [&](auto sb_c, auto step_c) __attribute__((always_inline)) {
        constexpr int sb = decltype(sb_c)::value;
        constexpr int step = decltype(step_c)::value;
        static_for<NVAL>([&](auto vv_c) __attribute__((always_inline)) {
            constexpr int vv = decltype(vv_c)::value;
            constexpr int s0 = vv / VPS;
            constexpr int h = vv / (16 * QB), b = (vv / 16) % QB, j = vv & 15;
            if constexpr (step == s0 + 2) {
                if constexpr (vv & 1)
                    r1[b] += p[vv];
                else
                    r0[b] += p[vv];
                asm volatile("" ::"v"(r0[b]), "v"(r1[b]));
                if constexpr (vv & 1) {
                    constexpr int kg = 2 * h + (j >> 3), d = (j & 7) >> 1;
                    pf[sb][b][kg][d] = M::pack(p[vv - 1], p[vv]);
                    asm volatile("" ::"v"(pf[sb][b][kg][d]));
                }
            }
            if constexpr (step == s0 + 1) {
                p[vv] = fast_exp2(x[vv]);
                asm volatile("" ::"v"(p[vv]));
            }
            if constexpr (step == s0) {
                x[vv] = fmaf(s[b][h][j], scale_log2, -st.m[b]);
                asm volatile("" ::"v"(x[vv]));
            }
        });
    };

    // End of the softmax of tile i (phase PH; P in buffer sb): the bound
    // check, the rare move of the reference max, and the tile's sum into l.
    // The move recomputes key half 0's scores (their registers hold tile
    // i+1's by now) from K(i), still in stage PH.
    auto settle = [&](int sb, int PH, int i) __attribute__((always_inline)) {
        float ts[QB];
        bool bad = false;
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            ts[b] = r0[b] + r1[b];
            r0[b] = 0.0f;
            r1[b] = 0.0f;
            bad = bad || !(ts[b] <= kBound);
        }
        if (__builtin_amdgcn_ballot_w64(bad) != 0) {
            f32x16 s0[QB];
            static_for<KS>([&](auto ks_c) __attribute__((always_inline)) {
                constexpr int ks = decltype(ks_c)::value;
                const u32x4 a = kfrag(PH, 0, ks);
#pragma unroll
                for (int b = 0; b < QB; ++b) mm_qk(s0[b], a, st.qf[b][ks], std::bool_constant<ks == 0>{});
            });
            if (needs_mask(i)) mask_half(s0, i, 0);
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                // Both lanes of a query take the same decision; the exchanges
                // run in every lane (under a partial EXEC mask they would read
                // stale values).
                const float ts_pair = swap32_f32(ts[b]);
                const bool need = !(ts[b] <= kBound && ts_pair <= kBound);
                float hm = s0[b][0];
#pragma unroll
                for (int j = 0; j < 16; ++j) hm = fmaxf(hm, fmaxf(s0[b][j], s[b][1][j]));
                hm = fmaxf(hm, swap32_f32(hm)) * scale_log2;
                const float m_new = need ? fmaxf(st.m[b], hm) : st.m[b];
                const float alpha = need ? fast_exp2(st.m[b] - m_new) : 1.0f;
                st.l[b] *= alpha;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) st.acc[b][mt] *= alpha;
                st.m[b] = m_new;
                float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int j = 0; j < 16; j += 2) {
                        const float v0 = h == 0 ? s0[b][j] : s[b][1][j];
                        const float v1 = h == 0 ? s0[b][j + 1] : s[b][1][j + 1];
                        const float e0 = fast_exp2(fmaf(v0, scale_log2, -m_new));
                        const float e1 = fast_exp2(fmaf(v1, scale_log2, -m_new));
                        a0 += e0;
                        a1 += e1;
                        pf[sb][b][2 * h + (j >> 3)][(j & 7) >> 1] = M::pack(e0, e1);
                    }
                ts[b] = a0 + a1;
            }
        }
#pragma unroll
        for (int b = 0; b < QB; ++b) st.l[b] += ts[b];
    };

    // One iteration of phase PH for tile i: QK of key half 1 of tile i and of
    // key half 0 of tile i+1 if HQ, PV(i-1) if HP, the softmax of tile i if
    // HOST.  On entry ring holds stream elements 0 .. RING-1; on exit it holds
    // those of the next iteration (phase PH+1).
    auto iteration = [&](auto ph_c, auto hq_c, auto hp_c, auto host_c, int i) __attribute__((always_inline)) {
        constexpr int PH = decltype(ph_c)::value;
        constexpr bool HQ = decltype(hq_c)::value;
        constexpr bool HP = decltype(hp_c)::value;
        constexpr bool HOST = decltype(host_c)::value;
        constexpr int SB = PH & 1;       // buffer of tile i's P
        constexpr int SN = SB ^ 1;       // buffer of tile i-1's P
        const bool masked = HOST && needs_mask(i);
        if (masked) {
            mask_s(i, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        static_for<NSTEP>([&](auto e_c) __attribute__((always_inline)) {
            constexpr int e = decltype(e_c)::value;
            constexpr int n = e >> 1;
            const u32x4 a = ring[e % RING];
#pragma unroll
            for (int b = 0; b < QB; ++b) {
                if constexpr ((e & 1) == 0) {
                    if constexpr (HQ) {
                        // n < KS: key half 1 of tile i; else key half 0 of tile i+1
                        constexpr int h = n < KS ? 1 : 0, ks = n % KS;
                        mm_qk(s[b][h], a, st.qf[b][ks], std::bool_constant<ks == 0>{});
                    }
                } else {
                    if constexpr (HP) {
                        constexpr int kg = n / MT, mt = n % MT;
                        mm_pv(st.acc[b][mt], a, pf[SN][b][kg]);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (e == NSTEP / 2 - 1) {
                // Key half 1 of tile i is complete: mask it before its softmax.
                if (masked) {
                            mask_s(i, 1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (e + RING < NSTEP) ring[e % RING] = frag(PH, e + RING);
            if constexpr (HOST) {
                static_for<2 * BPW>([&](auto c_c) __attribute__((always_inline)) {
                    constexpr int c = decltype(c_c)::value;
                    if constexpr (e == 1 + 2 * c) copy_part(PH, i, c);
                });
                host_step(std::integral_constant<int, SB>{}, e_c);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (HOST) {
            host_step(std::integral_constant<int, SB>{}, std::integral_constant<int, NSTEP>{});
            // The next iteration's first fragments: certified by the barrier
            // that ended the previous iteration.
#pragma unroll
            for (int e = 0; e < RING; ++e) ring[e] = frag((PH + 1) % NST, e);
            host_step(std::integral_constant<int, SB>{}, std::integral_constant<int, NSTEP + 1>{});
            settle(SB, PH, i);
            // Copies issued in this iteration may stay in flight; everything
            // older (the data the iteration after next reads) has landed.
            if (i + 3 <= T)
                wait_vmcnt<2 * BPW>();
            else if (i + 2 <= T)
                wait_vmcnt<BPW>();
            else
                wait_vmcnt<0>();
            __syncthreads();
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    // Prologue: Q, and the copies iterations kt0-3 .. kt0-1 would have
    // issued (K of tiles kt0 .. kt0+2, V of tiles kt0, kt0+1).
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        if (kt0 + t <= T) {
#pragma unroll
            for (int c = 0; c < BPW; ++c) {
                if ((kt0 + t + 1) * G::BC <= N)
                    dma_block_full<G>(k, k_stage(t), kt0 + t, w, lane, c);
                else
                    dma_block<G>(k, k_stage(t), kt0 + t, N, w, lane, c);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        if (kt0 + t <= T) {
#pragma unroll
            for (int c = 0; c < BPW; ++c) {
                if ((kt0 + t + 1) * G::BC <= N)
                    dma_block_full<G>(v, v_stage(t), kt0 + t, w, lane, c);
                else
                    dma_block<G>(v, v_stage(t), kt0 + t, N, w, lane, c);
            }
        }
    }
    wait_vmcnt<0>();
    __syncthreads();
    // S(kt0) and the reference max from its exact row maximum.
    {
        u32x4 fr[NQK];
#pragma unroll
        for (int n = 0; n < NQK; ++n) fr[n] = kfrag(0, n / KS, n % KS);
        static_for<NQK>([&](auto n_c) __attribute__((always_inline)) {
            constexpr int n = decltype(n_c)::value;
            constexpr int h = n / KS, ks = n % KS;
#pragma unroll
            for (int b = 0; b < QB; ++b) mm_qk(s[b][h], fr[n], st.qf[b][ks], std::bool_constant<ks == 0>{});
        });
    }
    if (needs_mask(kt0)) {
        mask_s(kt0, 0);
        mask_s(kt0, 1);
    }
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        float hm = s[b][0][0];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 16; ++j) hm = fmaxf(hm, s[b][h][j]);
        st.m[b] = fmaxf(hm, swap32_f32(hm)) * scale_log2;
    }
#pragma unroll
    for (int e = 0; e < RING; ++e) ring[e] = frag(0, e);

    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    using Y = std::true_type;
    using F = std::false_type;
    // Iteration kt0 has no PV.  (It computes key half 1 of tile kt0 again
    // and masks it again, which changes nothing.)
    iteration(P0{}, Y{}, F{}, Y{}, kt0);
    // Iterations kt0+1 .. T: QK of key half 0 of tile T+1 (in the last one)
    // reads a stage holding no valid tile and its result is never used.
    // With causal masking a wave has no work left from iteration i_idle on:
    // every key of tile i_idle - 1 and later lies after its last row
    // (64 (i_idle - 1) >= row0 + 32), so those tiles' scores are all masked,
    // their P is zero and the PV products add nothing.  From there the wave
    // only issues its share of the copies and meets the barriers.
    const int i_idle = CAUSAL ? (row0[0] + 96 + G::BC - 1) / G::BC : T + 2;
    const int Tw = min(T, i_idle - 1);  // this wave's last iteration with work
    const int nmid = max(Tw - kt0, 0);
    const int nq = nmid / 4;
    int i = kt0 + 1;
    for (int qq = 0; qq < nq; ++qq, i += 4) {
        iteration(P1{}, Y{}, Y{}, Y{}, i);
        iteration(P2{}, Y{}, Y{}, Y{}, i + 1);
        iteration(P3{}, Y{}, Y{}, Y{}, i + 2);
        iteration(P0{}, Y{}, Y{}, Y{}, i + 3);
    }
    const int nr = nmid - 4 * nq;
    if (nr >= 1) iteration(P1{}, Y{}, Y{}, Y{}, i++);
    if (nr >= 2) iteration(P2{}, Y{}, Y{}, Y{}, i++);
    if (nr >= 3) iteration(P3{}, Y{}, Y{}, Y{}, i++);
    // Idle iterations: the copies of iteration i (K(i+3), V(i+2)), then the
    // iteration's wait and barrier.
    for (; i <= T; ++i) {
        const int ph = (i - kt0) & 3;
#pragma unroll
        for (int c = 0; c < 2 * BPW; ++c) copy_part(ph, i, c);
        if (i + 3 <= T)
            wait_vmcnt<2 * BPW>();
        else if (i + 2 <= T)
            wait_vmcnt<BPW>();
        else
            wait_vmcnt<0>();
        __syncthreads();
    }
    // PV(T): the PV half of the iteration after T (nothing for a wave idle there).
    if (i_idle > T + 1) {
        switch (nr) {
            case 0: iteration(P1{}, F{}, Y{}, F{}, i); break;
            case 1: iteration(P2{}, F{}, Y{}, F{}, i); break;
            case 2: iteration(P3{}, F{}, Y{}, F{}, i); break;
            default: iteration(P0{}, F{}, Y{}, F{}, i); break;
        }
    }

    store_rows<D, QB>(st, args, seg, bh, row0, col, g);
}

template <bool BF16, int D, bool CAUSAL, int NW, int MINWG, int STAGES, int DIST, int QB = 1>
hipError_t launch_ring(AttnArgs a, hipStream_t stream) {
    constexpr int BR = 32 * QB * NW;
    a.T = (a.N + BR - 1) / BR;
    a.scale_log2 = kLog2e / __builtin_sqrtf((float)D);
    // Fold when the grid is one round (every workgroup resident at once,
    // MINWG per CU) and larger than the CU count, so CUs are shared.
    const int64_t wgs = (int64_t)a.T * a.BH * a.nseg;
    a.fold = wgs > 256 && wgs <= 256 * MINWG && a.nseg == 1 ? 1 : 0;
    void* params[] = {(void*)&a};
    return hipLaunchKernel(
        reinterpret_cast<const void*>(&attn_fwd_kernel<BF16, D, CAUSAL, NW, MINWG, STAGES, DIST, QB>),
        dim3((unsigned)(a.T * a.BH * a.nseg)), dim3(64 * NW), params, 0, stream);
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch_pipe(AttnArgs a, hipStream_t stream) {
    a.T = (a.N + 255) / 256;
    a.scale_log2 = kLog2e / __builtin_sqrtf((float)D);
    void* params[] = {(void*)&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_pipe_kernel<BF16, D, CAUSAL>),
                           dim3((unsigned)(a.T * a.BH * a.nseg)), dim3(512), params, 0, stream);
}

template <bool BF16, int D, bool CAUSAL, int NW>
hipError_t launch_ksplit(AttnArgs a, hipStream_t stream) {
    constexpr int BR = 16 * NW;
    a.T = (a.N + BR - 1) / BR;
    a.scale_log2 = kLog2e / __builtin_sqrtf((float)D);
    void* params[] = {(void*)&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_ksplit_kernel<BF16, D, CAUSAL, NW>),
                           dim3((unsigned)(a.T * a.BH)), dim3(64 * NW), params, 0, stream);
}

template <bool BF16, int D, bool CAUSAL, int QB, int NWV>
hipError_t launch_units(AttnArgs a, hipStream_t stream) {
    constexpr int RW = 32 * QB * NWV;
    a.T = (a.N + RW - 1) / RW;
    a.scale_log2 = kLog2e / __builtin_sqrtf((float)D);
    void* params[] = {(void*)&a};
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_fwd_units_kernel<BF16, D, CAUSAL, QB, NWV>),
                           dim3((unsigned)(a.T * a.BH * a.nseg)), dim3(64 * NWV), params, 0, stream);
}

// Two 32-row blocks per wave (512 query rows per workgroup) at D = 64 when
// that still gives two workgroups per CU: each K/V fragment read from LDS
// then feeds two MFMAs.  (At D = 128 the two blocks' O accumulators, Q
// fragments and scores exceed the 256 registers a wave has at two waves per
// SIMD.)
inline bool units_qb2(int64_t BH, int64_t N) { return BH * ((N + 511) / 512) >= 512; }

// 8 waves: the key-half unit kernel (256 query rows, one workgroup per CU).
// 4 waves: the ring kernel, two workgroups per CU (LDS for two: copies one
// tile ahead at D = 128, two at D = 64).
template <bool BF16, int D, bool CAUSAL>
hipError_t launch_cfg(const AttnArgs& a, int waves, hipStream_t stream) {
    if (waves == 4) {
        if constexpr (D == 128) {
            // At most two rounds of 64-row workgroups: the key split shortens
            // the longest workgroup's walk over its keys (C2: 15 -> 11 us).
            if (a.nseg == 1 && (int64_t)a.BH * ((a.N + 63) / 64) <= 512)
                return launch_ksplit<BF16, D, CAUSAL, 4>(a, stream);
            return launch_ring<BF16, D, CAUSAL, 4, 2, 2, 1>(a, stream);
        } else {
            return launch_ring<BF16, D, CAUSAL, 4, 2, 3, 2>(a, stream);
        }
    }
    if constexpr (D == 64) {
        if (a.nseg == 1 && units_qb2(a.BH, a.N)) return launch_units<BF16, D, CAUSAL, 2, 8>(a, stream);
        return launch_units<BF16, D, CAUSAL, 1, 8>(a, stream);
    } else {
        return launch_pipe<BF16, D, CAUSAL>(a, stream);
    }
}

}  // namespace

// Waves per workgroup: 8 (256 query rows, one workgroup per CU, each K/V
// tile read serves 256 rows) when that still gives at least two workgroups
// per CU; else 4 (128 rows, two workgroups per CU) for more parallelism.
int attn_pick_waves(int64_t BH, int64_t N) {
    const int64_t wgs_big = BH * ((N + 255) / 256);
    return wgs_big >= 512 ? 8 : 4;
}

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                           int B, int H, int Hkv, int N, int D, bool causal, bool bf16, int waves,
                           const SplitPlan* split, float* part_o, float2* part_ml,
                           hipStream_t stream) {
    AttnArgs a{};
    a.q = static_cast<const u16*>(q);
    a.k = static_cast<const u16*>(k);
    a.v = static_cast<const u16*>(v);
    a.o = o;
    a.lse = lse;
    a.BH = B * H;
    a.H = H;
    a.Hkv = Hkv;
    a.N = N;
    if (split != nullptr && split->nseg > 1) {
        a.nseg = split->nseg;
        a.seg_tiles = split->seg_tiles;
        a.part_o = part_o;
        a.part_ml = part_ml;
    } else {
        a.nseg = 1;
        a.seg_tiles = ((N + 255) / 256) * 4;
    }
    hipError_t e;
    if (D == 128) {
        if (bf16)
            e = causal ? launch_cfg<true, 128, true>(a, waves, stream)
                       : launch_cfg<true, 128, false>(a, waves, stream);
        else
            e = causal ? launch_cfg<false, 128, true>(a, waves, stream)
                       : launch_cfg<false, 128, false>(a, waves, stream);
    } else {
        if (bf16)
            e = causal ? launch_cfg<true, 64, true>(a, waves, stream)
                       : launch_cfg<true, 64, false>(a, waves, stream);
        else
            e = causal ? launch_cfg<false, 64, true>(a, waves, stream)
                       : launch_cfg<false, 64, false>(a, waves, stream);
    }
    if (e != hipSuccess || a.nseg == 1) return e;
    return launch_splitkv_merge(part_o, part_ml, o, lse, a.BH, N, D, a.nseg, a.seg_tiles * 64, causal,
                                stream);
}

// Split-KV plan (KV page, section 6.4: split the keys when the query side
// alone cannot fill the chip; the count depends on B*H, length and the
// number of CUs).  `requested` > 0 asks for that many segments.  With 0 the
// plan keeps one segment when the plain grid has two workgroups per CU or N
// is below 4096 keys (the merge's extra launch and traffic cost more than a
// short head gains).  Otherwise it takes the most segments whose non-empty
// workgroups still fit on the CUs at once (one 8-wave workgroup per CU):
// more would add a second round of workgroups, each paying its own Q load
// and partial-state store, plus merge traffic.  With causal masking, S
// segments leave about (S + 1) / 2 of the grid non-empty.  At most 16.
// Segments are whole multiples of 256 keys (so they align with every
// query-tile size); the count is then the number of such segments N needs.
// A split runs 8-wave workgroups: the segments supply the parallelism, and
// 256 query rows share each K/V tile.
SplitPlan attn_plan_split(int64_t BH, int64_t N, bool causal, int requested) {
    constexpr int kCUs = 256;
    const int64_t tiles = (N + 63) / 64;
    const int64_t quads = (tiles + 3) / 4;     // 256-key units
    const int plain_waves = attn_pick_waves(BH, N);
    const int64_t wgs_plain = BH * ((N + 32 * plain_waves - 1) / (32 * plain_waves));
    const int64_t wgs8 = BH * ((N + 255) / 256);
    int64_t want = requested;
    if (want <= 0) {
        if (wgs_plain >= 2 * kCUs || N < 4096)
            want = 1;
        else
            want = causal ? 2 * kCUs / wgs8 - 1 : kCUs / wgs8;
        want = want > 16 ? 16 : want;
    }
    if (want > quads) want = quads;
    if (want < 1) want = 1;
    const int64_t seg_quads = (quads + want - 1) / want;
    SplitPlan p;
    p.seg_tiles = (int)(seg_quads * 4);
    p.nseg = (int)((quads + seg_quads - 1) / seg_quads);
    p.waves = p.nseg > 1 ? 8 : plain_waves;
    return p;
}

}  // namespace osc
