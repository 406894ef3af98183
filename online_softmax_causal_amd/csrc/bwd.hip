// Attention backward on gfx950: dQ, dK, dV of O = softmax(Q K^T / sqrt(D) + M) V
// for a given dO, from the forward pass's O and log-sum-exp.
//
// The pages keep the log-sum-exp of each row for the backward pass ("CUDA
// FlashAttention: from online softmax to long-sequence IO limits"
// (chengzipai.xyz), section 7) and give no backward algorithm of their own.
// With it the softmax weights are recomputed tile by tile, P_ij =
// exp(s_ij / sqrt(D) - lse_i), so nothing N x N is ever stored, and the
// gradients are those of the definition:
//     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_d dO_id O_id,
//     dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D)
// (D_i = sum_j P_ij dP_ij because O_i = sum_j P_ij v_j).  With grouped K/V
// heads (query head h reads K/V head floor(h / g), "CUDA KV Cache: paged
// storage and long-context decode" (chengzipai.xyz), section 3), dK and dV of
// a K/V head are the sums of these over the g query heads of its group.
//
// Three kernels, all on one stream:
//   attn_bwd_pre_kernel   D_i and the base-2 log-sum-exp lse_i * log2(e) of
//                         every row, into the caller's workspace (HBM-bound);
//   dK/dV kernel          key-major: a workgroup keeps 32 keys per wave of
//                         one K/V head in registers and streams 64-row tiles
//                         of Q and dO (with D and lse of those rows) of every
//                         query head of the group through LDS;
//                         dV^T += dO^T P and dK^T += Q^T dS on the MFMA.
//                         D = 64: attn_bwd_dkdv_kernel, 8 waves (two per
//                         SIMD), one 32-query block after the other;
//                         D = 128: attn_bwd_dkdv_pipe_kernel, 4 waves (one
//                         per SIMD), the blocks software-pipelined;
//   attn_bwd_dq_kernel    query-major, like the forward kernel: a workgroup of
//                         8 waves (two per SIMD) keeps 256 query rows of Q and
//                         dO in registers and streams 64-key tiles of K and V,
//                         taken 32 keys at a time; dQ^T += K^T dS^T.
// Splitting dQ from dK/dV recomputes S and dP once more but needs no atomic
// accumulation, so the result is deterministic.  P and dS are rounded RNE to
// the input dtype as MFMA operands; every accumulation is FP32.
//
// Operand layouts are those of the forward kernel (32x32x16 MFMA, chunk
// swizzle, direct global->LDS copies, transpose reads for X^T operands):
//   dK/dV kernel: S = Q K^T with A = Q rows from LDS and B = K^T in
//   registers, so a lane holds one key (column) and 16 query rows; those
//   accumulators, packed, are the B operand of dV^T = dO^T P whose A operand
//   dO^T is read transposed from the dO tile in the same query order.
//   dQ kernel: S^T = K Q^T exactly as the forward's; dS^T packed is the B
//   operand of dQ^T = K^T dS^T with K^T read transposed from the K tile.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "kernels.hpp"
#include "mfma_tile.hpp"
#include "online_merge.hpp"

namespace osc {
namespace {

constexpr int kBwdWaves = 4;            // waves per workgroup (one per SIMD)
constexpr int kBwdRows = 32 * kBwdWaves; // resident rows (keys or queries) per workgroup
constexpr int kBwdTile = 64;            // streamed rows per tile
constexpr int kBwdStages = 3;           // LDS stages; tile t+2 is copied during tile t

struct BwdArgs {
    const u16* q;       // [B, H, N, D]
    const u16* k;
    const u16* v;
    const float* o;     // [B, H, N, D] forward output
    const float* lse;   // [B, H, N] forward log-sum-exp (natural log)
    const u16* dout;    // [B, H, N, D]
    float* dq;          // [B, H, N, D]
    float* dk;
    float* dv;
    float* dd;          // workspace [B, H, N]: D_i
    float* lse2;        // workspace [B, H, N]: lse_i * log2(e)
    int BH;             // B * H (query heads)
    int H;              // query heads per batch
    int Hkv;            // key/value heads per batch (divides H)
    int BHkv;           // B * Hkv
    int N;
    float scale_log2;   // log2(e) / sqrt(D)
    float scale;        // 1 / sqrt(D)
};

// Workgroup index -> (tile of resident rows, head), longest causal work first
// for the key-major kernel (tile 0 sees every query) and for the query-major
// kernel (the last tile sees every key); heads are spread over the XCDs as in
// the forward kernel.
__device__ __forceinline__ void bwd_work(int bid, int BH, int ntiles, bool reverse, int* tile,
                                         int* bh) {
    const int tt = bid / BH;
    *tile = reverse ? ntiles - 1 - tt : tt;
    const int j = bid % BH;
    *bh = (BH & 7) ? j : (j & 7) * (BH >> 3) + (j >> 3);
}

// Copy rows [row0, row0 + 64) of a [N, D] 16-bit matrix into an LDS tile
// (chunk-swizzled rows); the four waves share the 1 KiB blocks.  Rows past N
// repeat row N - 1 (finite data; the kernels mask them).
template <int D, int NW = kBwdWaves>
__device__ __forceinline__ void copy_tile(const u16* src, u16* dst, int row0, int N, int w,
                                          int lane) {
    constexpr int CPR = D / 8, RPB = 1024 / (2 * D);
    constexpr int BPW = kBwdTile / RPB / NW;
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int blk = w * BPW + j;
        const int r = blk * RPB + lane / CPR;
        const int c = (lane % CPR) ^ chunk_swizzle<D>(r);
        const int row = min(row0 + r, N - 1);
        copy_to_lds16(src, (unsigned)((row * D + c * 8) * 2), dst + blk * 512);
    }
}

template <int D, int NW = kBwdWaves>
constexpr int copies_per_matrix() {
    return kBwdTile / (1024 / (2 * D)) / NW;
}

// dK/dV kernel waves: two per SIMD where K, V and both accumulators fit 256
// registers (D = 64); one per SIMD at D = 128 (8 waves spill heavily there).
template <int D>
constexpr int dkdv_waves() {
    return D == 128 ? 4 : 8;
}
constexpr int kDqWaves = 8;                  // dQ kernel: two waves per SIMD
constexpr int kDqRows = 32 * kDqWaves;       // query rows per dQ workgroup

// One 16-bit value (low bits of b) as FP32, exactly.
template <bool BF16>
__device__ __forceinline__ float bits16_to_float(unsigned b) {
    if constexpr (BF16)
        return __builtin_bit_cast(float, b << 16);
    else
        return (float)__builtin_bit_cast(_Float16, (unsigned short)b);
}

// ---------------------------------------------------------------------------
// D_i = sum_d dO_id O_id and lse2_i = lse_i log2(e).  D / 8 lanes per row,
// each lane 8 values (a 16-byte dO load and two 16-byte O loads).
template <bool BF16, int D>
__global__ void __launch_bounds__(256)
attn_bwd_pre_kernel(BwdArgs a) {
    constexpr int LPR = D / 8;
    const int64_t rows = (int64_t)a.BH * a.N;
    const int64_t r = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
    const int c = (threadIdx.x % LPR) * 8;
    float acc = 0.0f;
    if (r < rows) {
        const u32x4 d16 = *reinterpret_cast<const u32x4*>(a.dout + r * D + c);
        const f32x4 o0 = *reinterpret_cast<const f32x4*>(a.o + r * D + c);
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(a.o + r * D + c + 4);
        const float ov[8] = {o0[0], o0[1], o0[2], o0[3], o1[0], o1[1], o1[2], o1[3]};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const unsigned w = d16[i];
            acc = fmaf(bits16_to_float<BF16>(w & 0xffffu), ov[2 * i], acc);
            acc = fmaf(bits16_to_float<BF16>(w >> 16), ov[2 * i + 1], acc);
        }
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
    if (r < rows && threadIdx.x % LPR == 0) {
        a.dd[r] = acc;
        a.lse2[r] = a.lse[r] * kLog2e;
    }
}

// ---------------------------------------------------------------------------
// LDS pointer types: fragment reads through them are a per-lane base plus an
// immediate offset.
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
typedef __attribute__((address_space(3))) u16 lds_u16;

// acc = the 32-row block at element offset `off` of the tile behind rp (rp[ks]:
// this lane's row fragment of d step ks, lane row lane % 32) times the
// B-operand fragments bf over d: KS MFMAs whose A fragments stream through a
// 4-deep register ring (held by scheduling groups, so each LDS read is
// issued four fragments ahead of its use).
template <bool BF16, int D>
__device__ __forceinline__ void rows_times(const lds_u32x4* const (&rp)[D / 16], int off,
                                           const u32x4 (&bf)[D / 16], f32x16& acc) {
    using M = Mma<BF16>;
    constexpr int KS = D / 16;
    auto frag = [&](int f) { return rp[f][off / 8]; };
    __builtin_amdgcn_sched_barrier(0);
    u32x4 ring[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) ring[f] = frag(f);
#pragma unroll
    for (int f = 0; f < KS; ++f) {
        const u32x4 x = ring[f & 3];
        if (f + 4 < KS) ring[f & 3] = frag(f + 4);
        acc = M::run(x, bf[f], f == 0 ? f32x16{} : acc);
    }
    __builtin_amdgcn_sched_group_barrier(kSgDsRead, 4, 0);
#pragma unroll
    for (int f = 0; f < KS - 4; ++f) {
        __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSgDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
}

// acc[mt] += X^T[d = 32 mt + ..][16 rows of group u] * bf[u] over the NU
// 16-row groups of the block at element offset `off` of the tile behind tp
// (tp[mt][r]: this lane's two transpose reads of group 0): 2 * NU * MT
// transpose reads through a 4-fragment ring.  X^T is read in the
// accumulator's row order (tr_frag_offset).
template <bool BF16, int D, int NU>
__device__ __forceinline__ void trans_times(const lds_s16x4* const (&tp)[D / 32][2], int off,
                                            const u32x4 (&bf)[NU], f32x16 (&acc)[D / 32]) {
    using M = Mma<BF16>;
    constexpr int MT = D / 32, NF = NU * MT;
    auto frag = [&](int f) {
        const int o = (off + (f / MT) * 16 * D) / 4;
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tp[f % MT][0] + o));
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tp[f % MT][1] + o));
        const auto lo = __builtin_bit_cast(unsigned long long, x0);
        const auto hi = __builtin_bit_cast(unsigned long long, x1);
        return u32x4{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi, (unsigned)(hi >> 32)};
    };
    u32x4 ring[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) ring[f] = frag(f);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        const u32x4 x = ring[f & 3];
        if (f + 4 < NF) ring[f & 3] = frag(f + 4);
        acc[f % MT] = M::run(x, bf[f / MT], acc[f % MT]);
    }
}

// Per-lane LDS pointers into the stage of a streamed tile: row fragments
// (rp), transposed reads (tp) and, when the stage holds them, this lane's
// lse2 / D entries (lp).  advance() moves them from the stage of tile fi to
// that of tile fi + 1 (kBwdStages stages of `stage` elements).
template <int D, bool LP>
struct StagePtrs {
    const lds_u32x4* rp[D / 16];
    const lds_s16x4* tp[D / 32][2];
    const lds_f32x4* lp;
    __device__ __forceinline__ void init(const u16* lds, int lane, int lp_off) {
        const int col = lane & 31;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            rp[ks] = (const lds_u32x4*)((const lds_u16*)lds + row_frag_offset<D>(col, ks, lane));
            asm volatile("" : "+v"(rp[ks]));
        }
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                tp[mt][r] = (const lds_s16x4*)((const lds_u16*)lds + tr_frag_offset<D>(lane, mt, r));
                asm volatile("" : "+v"(tp[mt][r]));
            }
        if constexpr (LP) {
            lp = (const lds_f32x4*)((const lds_u16*)lds + lp_off) + (lane >> 5);
            asm volatile("" : "+v"(lp));
        }
    }
    __device__ __forceinline__ void advance(int fi, int stage) {
        const int delta = (fi % kBwdStages == kBwdStages - 1) ? -(kBwdStages - 1) * stage : stage;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
            rp[ks] = (const lds_u32x4*)((const lds_u16*)rp[ks] + delta);
            asm volatile("" : "+v"(rp[ks]));
        }
#pragma unroll
        for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                tp[mt][r] = (const lds_s16x4*)((const lds_u16*)tp[mt][r] + delta);
                asm volatile("" : "+v"(tp[mt][r]));
            }
        if constexpr (LP) {
            lp = (const lds_f32x4*)((const lds_u16*)lp + delta);
            asm volatile("" : "+v"(lp));
        }
    }
};

template <bool BF16, int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * dkdv_waves<D>(), 1)
attn_bwd_dkdv_kernel(BwdArgs a) {
    constexpr int kDkdvWaves = dkdv_waves<D>();
    constexpr int kDkdvRows = 32 * kDkdvWaves;
    using M = Mma<BF16>;
    constexpr int KS = D / 16, MT = D / 32;
    constexpr int TILE = kBwdTile * D;
    constexpr int STAGE = 2 * TILE + 2 * kBwdTile * 2;  // Q, dO (16-bit), lse2, D (FP32)
    constexpr int LPM = copies_per_matrix<D, kDkdvWaves>();
    __shared__ __attribute__((aligned(1024))) u16 lds[kBwdStages * STAGE];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, g = lane >> 5;
    const int N = a.N;
    const int nkt = (N + kDkdvRows - 1) / kDkdvRows;
    // Workgroup: one key tile of one K/V head.  Its dK and dV sum over the
    // g query heads of the group (KV page, section 3: query head h reads K/V
    // head floor(h / g)), whose Q / dO tiles stream through one sequence.
    int kt, bkv;
    bwd_work(blockIdx.x, a.BHkv, nkt, false, &kt, &bkv);
    const int64_t head = (int64_t)bkv * N;   // K/V / dK / dV rows of this head
    const int grp = a.H / a.Hkv;
    const int hq0 = (bkv / a.Hkv) * a.H + (bkv % a.Hkv) * grp;  // first query head
    const int kw = kt * kDkdvRows + 32 * w;  // first key of this wave
    const int key = kw + col;

    // K^T and V^T fragments (B operands): lane (col, g) holds key `key`,
    // d = 16 ks + 8 g .. + 7.
    u32x4 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int64_t off = (head + key) * D + ks * 16 + 8 * g;
        kf[ks] = key < N ? *reinterpret_cast<const u32x4*>(a.k + off) : u32x4{0u, 0u, 0u, 0u};
        vf[ks] = key < N ? *reinterpret_cast<const u32x4*>(a.v + off) : u32x4{0u, 0u, 0u, 0u};
    }
    f32x16 dk_acc[MT], dv_acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        dk_acc[mt] = f32x16{};
        dv_acc[mt] = f32x16{};
    }
    StagePtrs<D, true> sp;
    sp.init(lds, lane, 2 * TILE);

    // Query tiles: with causal masking only rows at or after the workgroup's
    // first key contribute.
    const int nqt = (N + kBwdTile - 1) / kBwdTile;
    const int qt0 = CAUSAL ? (kt * kDkdvRows) / kBwdTile : 0;
    // Streamed tiles, numbered fi = i * nt + (it - qt0) for query head
    // hq0 + i of the group and query tile it.
    const int nt = nqt - qt0;
    const int nflat = grp * nt;
    auto stage = [&](int fi) { return lds + (fi % kBwdStages) * STAGE; };
    // Waves 0 and 1 also copy the tile's lse2 and D rows (one 4-byte copy each).
    auto issue = [&](int fi) {
        if (fi >= nflat) return;
        u16* st = stage(fi);
        const int64_t qhead = (int64_t)(hq0 + fi / nt) * N;
        const int r0 = (qt0 + fi % nt) * kBwdTile;
        copy_tile<D, kDkdvWaves>(a.q + qhead * D, st, r0, N, w, lane);
        copy_tile<D, kDkdvWaves>(a.dout + qhead * D, st + TILE, r0, N, w, lane);
        if (w < 2) {
            const int row = min(r0 + lane, N - 1);
            const float* src = w == 0 ? a.lse2 + qhead : a.dd + qhead;
            copy_to_lds4(src, (unsigned)(row * 4), st + 2 * TILE + w * 2 * kBwdTile);
        }
    };
    // Tile fi+1 complete for this wave (tile fi+2 may stay in flight), then
    // for all waves.
    auto wait_next = [&](int fi) {
        if (fi + 2 < nflat) {
            if (w < 2)
                wait_vmcnt<2 * LPM + 1>();
            else
                wait_vmcnt<2 * LPM>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();
    };

    // One 32-query block at row qb of a staged tile: S = Q K^T and dP = dO V^T
    // (lane (col, g) holds query rows qb + 8(e/4) + 4g + e%4 of key `key`),
    // P from the saved LSE, dS = P (dP - D), then dV^T += dO^T P and
    // dK^T += Q^T dS.  MASKED zeroes P where key > query (causal) or the
    // query row is past N.
    auto block = [&](int b, int qb, auto masked_tag) {
        f32x16 s[1], dp[1];
        rows_times<BF16, D>(sp.rp, 32 * b * D, kf, s[0]);
        rows_times<BF16, D>(sp.rp, TILE + 32 * b * D, vf, dp[0]);
        int lo = 0, hi = 32;
        if constexpr (decltype(masked_tag)::value) {
            // masked iff offset e' = 8(e/4) + e%4 is < key - qb - 4g (causal)
            // or >= N - qb - 4g (rows past N)
            lo = CAUSAL ? key - qb - 4 * g : -1;
            hi = N - qb - 4 * g;
        }
        u32x4 pf[2], dsf[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float p[8], ds[8];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int j4 = 2 * u + h;
                const f32x4 l2 = sp.lp[(32 * b + 8 * j4) / 4];
                const f32x4 dd = sp.lp[(kBwdTile + 32 * b + 8 * j4) / 4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int e = 4 * j4 + i;
                    float pe = fast_exp2(fmaf(s[0][e], a.scale_log2, -l2[i]));
                    if constexpr (decltype(masked_tag)::value) {
                        const int off = 8 * j4 + i;
                        pe = (off < lo || off >= hi) ? 0.0f : pe;
                    }
                    p[4 * h + i] = pe;
                    ds[4 * h + i] = pe * (dp[0][e] - dd[i]);
                }
            }
            pf[u] = u32x4{M::pack(p[0], p[1]), M::pack(p[2], p[3]), M::pack(p[4], p[5]),
                          M::pack(p[6], p[7])};
            dsf[u] = u32x4{M::pack(ds[0], ds[1]), M::pack(ds[2], ds[3]), M::pack(ds[4], ds[5]),
                           M::pack(ds[6], ds[7])};
        }
        trans_times<BF16, D, 2>(sp.tp, TILE + 32 * b * D, pf, dv_acc);
        trans_times<BF16, D, 2>(sp.tp, 32 * b * D, dsf, dk_acc);
    };
    std::integral_constant<bool, false> plain;
    std::integral_constant<bool, true> masked;

    issue(0);
    issue(1);
    if (1 < nflat) {
        if (w < 2)
            wait_vmcnt<2 * LPM + 1>();
        else
            wait_vmcnt<2 * LPM>();
    } else {
        wait_vmcnt<0>();
    }
    __syncthreads();

    for (int fi = 0; fi < nflat; ++fi) {
        issue(fi + 2);
        const int it = qt0 + fi % nt;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int qb = it * kBwdTile + 32 * b;  // first query row of the block
            if (qb >= N || (CAUSAL && qb + 31 < kw)) continue;
            if ((CAUSAL && qb < kw + 31) || qb + 32 > N)
                block(b, qb, masked);
            else
                block(b, qb, plain);
        }
        wait_next(fi);
        sp.advance(fi, STAGE);
    }

    // Lane (col, g) holds d = 32 mt + 8 (i / 4) + 4 g + i % 4 of key `key`.
    if (key >= N) return;
    float* dkr = a.dk + (head + key) * D;
    float* dvr = a.dv + (head + key) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d = mt * 32 + 8 * i4 + 4 * g;
            *reinterpret_cast<f32x4*>(dkr + d) =
                f32x4{dk_acc[mt][4 * i4], dk_acc[mt][4 * i4 + 1], dk_acc[mt][4 * i4 + 2],
                      dk_acc[mt][4 * i4 + 3]} * a.scale;
            *reinterpret_cast<f32x4*>(dvr + d) =
                f32x4{dv_acc[mt][4 * i4], dv_acc[mt][4 * i4 + 1], dv_acc[mt][4 * i4 + 2],
                      dv_acc[mt][4 * i4 + 3]};
        }
}

// ---------------------------------------------------------------------------
template <bool BF16, int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kDqWaves, 1)
attn_bwd_dq_kernel(BwdArgs a) {
    using M = Mma<BF16>;
    constexpr int KS = D / 16, MT = D / 32;
    constexpr int TILE = kBwdTile * D;
    constexpr int STAGE = 2 * TILE;  // K, V
    constexpr int LPM = copies_per_matrix<D, kDqWaves>();
    __shared__ __attribute__((aligned(1024))) u16 lds[kBwdStages * STAGE];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, g = lane >> 5;
    const int N = a.N;
    const int nq = (N + kDqRows - 1) / kDqRows;
    int t, bh;
    bwd_work(blockIdx.x, a.BH, nq, CAUSAL, &t, &bh);
    const int64_t head = (int64_t)bh * N;
    // K/V head of this query head (KV page, section 3).
    const int64_t kvhead = (int64_t)((bh / a.H) * a.Hkv + (bh % a.H) / (a.H / a.Hkv)) * N;
    const int row0 = t * kDqRows + 32 * w;  // first query row of this wave
    const int row = row0 + col;

    u32x4 qf[KS], dof[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int64_t off = (head + row) * D + ks * 16 + 8 * g;
        qf[ks] = row < N ? *reinterpret_cast<const u32x4*>(a.q + off) : u32x4{0u, 0u, 0u, 0u};
        dof[ks] = row < N ? *reinterpret_cast<const u32x4*>(a.dout + off) : u32x4{0u, 0u, 0u, 0u};
    }
    const float l2 = row < N ? a.lse2[head + row] : 0.0f;
    const float dd = row < N ? a.dd[head + row] : 0.0f;
    f32x16 dq_acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) dq_acc[mt] = f32x16{};
    // Per-lane LDS pointers into the stage of the current tile (row
    // fragments of the K tile, transposed reads of its first 16-row group);
    // the V tile, the key half and the group are immediates.
    StagePtrs<D, false> sp;
    sp.init(lds, lane, 0);

    const int kv_end = CAUSAL ? min(t * kDqRows + kDqRows, N) : N;
    const int ntiles = (kv_end + kBwdTile - 1) / kBwdTile;
    // This wave's last key tile, its diagonal or ragged-tail tile (the only
    // one that can need masking); -1 if its rows are past N.
    const int last = row0 >= N ? -1 : min(ntiles - 1, CAUSAL ? (row0 + 31) / kBwdTile : ntiles - 1);
    auto stage = [&](int it) { return lds + (it % kBwdStages) * STAGE; };
    auto issue = [&](int it) {
        if (it >= ntiles) return;
        u16* st = stage(it);
        copy_tile<D, kDqWaves>(a.k + kvhead * D, st, it * kBwdTile, N, w, lane);
        copy_tile<D, kDqWaves>(a.v + kvhead * D, st + TILE, it * kBwdTile, N, w, lane);
    };
    auto finish = [&](int it) {
        if (it + 2 < ntiles)
            wait_vmcnt<2 * LPM>();
        else
            wait_vmcnt<0>();
        __syncthreads();
    };
    // One 64-key tile: S^T = K Q^T and dP^T = V dO^T (lane (col, g) holds
    // keys 32 kb + 8(e/4) + 4g + e%4 of query `row`), P^T from the saved LSE,
    // dS^T = P^T (dP^T - D), dQ^T += K^T dS^T.  MASKED zeroes keys after the
    // query (causal) or past N.
    // The tile is taken as two halves of 32 keys, to keep the live registers
    // within two waves per SIMD.
    auto tile = [&](int it, auto masked_tag) {
        const int key0 = it * kBwdTile;
        int lim = 1 << 30;
        if constexpr (decltype(masked_tag)::value)
            lim = min(CAUSAL ? row - key0 : (1 << 30), N - 1 - key0) - 4 * g;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            f32x16 s[1], dp[1];
            rows_times<BF16, D>(sp.rp, half * 32 * D, qf, s[0]);
            rows_times<BF16, D>(sp.rp, TILE + half * 32 * D, dof, dp[0]);
            u32x4 dsf[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                float ds[8];
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int e = 8 * u + jj;
                    float pe = fast_exp2(fmaf(s[0][e], a.scale_log2, -l2));
                    if constexpr (decltype(masked_tag)::value) {
                        const int c = 32 * half + 8 * (e >> 2) + (e & 3);
                        pe = c > lim ? 0.0f : pe;
                    }
                    ds[jj] = pe * (dp[0][e] - dd);
                }
                dsf[u] = u32x4{M::pack(ds[0], ds[1]), M::pack(ds[2], ds[3]), M::pack(ds[4], ds[5]),
                               M::pack(ds[6], ds[7])};
            }
            trans_times<BF16, D, 2>(sp.tp, half * 32 * D, dsf, dq_acc);
        }
    };
    std::integral_constant<bool, false> plain;
    std::integral_constant<bool, true> masked;

    issue(0);
    issue(1);
    if (1 < ntiles)
        wait_vmcnt<2 * LPM>();
    else
        wait_vmcnt<0>();
    __syncthreads();

    int it = 0;
    for (; it < last; ++it) {
        issue(it + 2);
        tile(it, plain);
        finish(it);
        sp.advance(it, STAGE);
    }
    if (it == last) {
        issue(it + 2);
        tile(it, masked);
        finish(it);
        ++it;
    }
    for (; it < ntiles; ++it) {
        issue(it + 2);
        finish(it);
    }

    if (row >= N) return;
    float* dqr = a.dq + (head + row) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<f32x4*>(dqr + mt * 32 + 8 * i4 + 4 * g) =
                f32x4{dq_acc[mt][4 * i4], dq_acc[mt][4 * i4 + 1], dq_acc[mt][4 * i4 + 2],
                      dq_acc[mt][4 * i4 + 3]} * a.scale;
}

// ---------------------------------------------------------------------------
// dK/dV at D = 128 as a software pipeline over 32-query blocks.  Same layout
// and per-block arithmetic as attn_bwd_dkdv_kernel (one wave per SIMD, 32
// keys per wave with K^T and V^T resident), but the step of block j runs
//   (a) S and dP of block j on the MFMA (16 MFMAs, the two products
//       alternating, A operands through a 4-deep LDS ring that runs on
//       across the steps of a tile);
//   (b) if block j needs the mask: S_j set to -inf where key > query or the
//       query row is past N (a wave-uniform branch);
//   (c) dV^T += dO^T P and dK^T += Q^T dS of block j-1 (16 MFMAs,
//       transposed LDS reads through a 4-deep ring), with block j's weights
//       hosted between them: P = 2^(S scale - lse2), dS = P (dP - D), both
//       packed to 16 bits.
// A block wholly masked for the wave (all its rows before the wave's keys,
// or past N) is computed with P = 0 instead of skipped, which keeps every
// wave's step sequence the same; its dV/dK products add zeros.
// Blocks 0 and 1 of a streamed tile are its two 32-row halves; block 0's
// step finishes block 1 of the previous tile, so four LDS stages hold the
// tile being read, the previous one (its last dV/dK) and two in flight.
// Even and odd blocks keep packed P and dS in separate registers (the loop
// body holds both steps of a tile), so no value moves between iterations.
template <bool BF16, bool CAUSAL>
__global__ void __launch_bounds__(256, 1)
attn_bwd_dkdv_pipe_kernel(BwdArgs a) {
    constexpr int D = 128, NW = 4;
    using M = Mma<BF16>;
    constexpr int KS = D / 16, MT = D / 32;
    constexpr int TILE = kBwdTile * D;
    constexpr int STAGE = 2 * TILE + 2 * kBwdTile * 2;  // Q, dO (16-bit), lse2, D (FP32)
    constexpr int LPM = copies_per_matrix<D, NW>();
    constexpr int NSTG = 4;  // stages: tile t read, t-1 still read by dV/dK, t+1 and t+2 in flight
    __shared__ __attribute__((aligned(1024))) u16 lds[NSTG * STAGE];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 31, g = lane >> 5;
    const int N = a.N;
    constexpr int kRows = 32 * NW;
    const int nkt = (N + kRows - 1) / kRows;
    int kt, bkv;
    bwd_work(blockIdx.x, a.BHkv, nkt, false, &kt, &bkv);
    const int64_t head = (int64_t)bkv * N;   // K/V / dK / dV rows of this head
    const int grp = a.H / a.Hkv;
    const int hq0 = (bkv / a.Hkv) * a.H + (bkv % a.Hkv) * grp;  // first query head
    const int kw = kt * kRows + 32 * w;  // first key of this wave
    const int key = kw + col;

    // K^T and V^T fragments (B operands): lane (col, g) holds key `key`,
    // d = 16 ks + 8 g .. + 7.
    u32x4 kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const int64_t off = (head + key) * D + ks * 16 + 8 * g;
        kf[ks] = key < N ? *reinterpret_cast<const u32x4*>(a.k + off) : u32x4{0u, 0u, 0u, 0u};
        vf[ks] = key < N ? *reinterpret_cast<const u32x4*>(a.v + off) : u32x4{0u, 0u, 0u, 0u};
    }
    f32x16 dk_acc[MT], dv_acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        dk_acc[mt] = f32x16{};
        dv_acc[mt] = f32x16{};
    }
    int rfo[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) rfo[ks] = row_frag_offset<D>(col, ks, lane);
    int tfo[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 2; ++r) tfo[mt][r] = tr_frag_offset<D>(lane, mt, r);

    // Query tiles: with causal masking only rows at or after the workgroup's
    // first key contribute.  Streamed tiles fi = i * nt + (it - qt0) for
    // query head hq0 + i of the group and query tile it.
    const int nqt = (N + kBwdTile - 1) / kBwdTile;
    const int qt0 = CAUSAL ? (kt * kRows) / kBwdTile : 0;
    const int nt = nqt - qt0;
    const int nflat = grp * nt;
    auto stage_off = [&](int fi) { return (fi % NSTG) * STAGE; };
    auto tile_row0 = [&](int fi) { return (qt0 + fi % nt) * kBwdTile; };
    // Waves 0 and 1 also copy the tile's lse2 and D rows (one 4-byte copy each).
    auto issue = [&](int fi) {
        if (fi >= nflat) return;
        u16* st = lds + stage_off(fi);
        const int64_t qhead = (int64_t)(hq0 + fi / nt) * N;
        const int r0 = tile_row0(fi);
        copy_tile<D, NW>(a.q + qhead * D, st, r0, N, w, lane);
        copy_tile<D, NW>(a.dout + qhead * D, st + TILE, r0, N, w, lane);
        if (w < 2) {
            const int row = min(r0 + lane, N - 1);
            const float* src = w == 0 ? a.lse2 + qhead : a.dd + qhead;
            copy_to_lds4(src, (unsigned)(row * 4), st + 2 * TILE + w * 2 * kBwdTile);
        }
    };

    // Per-lane LDS pointers, rebased once per tile: row fragments (read by
    // S and dP; advanced to the next tile at its barrier) and transposed
    // fragments plus this lane's lse2 / D entries (read by the weights and by
    // dV, dK; advanced after a tile's last step).  Every fragment is a
    // pointer plus an immediate.
    const lds_u32x4* rp[KS];
    const lds_s16x4* tp[MT][2];
    const lds_f32x4* lp;
    auto rebase_rows = [&](int fi) {
        const int so = stage_off(fi);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            rp[ks] = (const lds_u32x4*)((const lds_u16*)lds + so + rfo[ks]);
            asm volatile("" : "+v"(rp[ks]));
        }
        lp = (const lds_f32x4*)((const lds_u16*)lds + so + 2 * TILE) + g;
        asm volatile("" : "+v"(lp));
    };
    auto rebase_trans = [&](int fi) {
        const int so = stage_off(fi);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                tp[mt][r] = (const lds_s16x4*)((const lds_u16*)lds + so + tfo[mt][r]);
                asm volatile("" : "+v"(tp[mt][r]));
            }
    };
    // Row fragment ks of block b of the Q (X = 0) or dO (X = 1) tile.
    auto rfrag = [&](int X, int b, int ks) __attribute__((always_inline)) {
        return rp[ks][(X * TILE + b * 32 * D) / 8];
    };
    // Transposed fragment (16-row group u, d block mt) of block b of the Q
    // (X = 0) or dO (X = 1) tile.
    auto tfrag = [&](int X, int b, int u, int mt) __attribute__((always_inline)) {
        const int o = (X * TILE + b * 32 * D + u * 16 * D) / 4;
        const s16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tp[mt][0] + o));
        const s16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tp[mt][1] + o));
        const auto lo = __builtin_bit_cast(unsigned long long, x0);
        const auto hi = __builtin_bit_cast(unsigned long long, x1);
        return u32x4{(unsigned)lo, (unsigned)(lo >> 32), (unsigned)hi, (unsigned)(hi >> 32)};
    };

    // Mask of block rows qb .. qb+31 (lane rows qb + 4g + off, off = 8(e/4) + e%4).
    auto needs_mask = [&](int qb) __attribute__((always_inline)) {
        return (CAUSAL && qb < kw + 31) || qb + 32 > N;
    };
    auto mask_s = [&](f32x16& s, int qb) __attribute__((always_inline)) {
        const int lo = CAUSAL ? key - qb - 4 * g : -1;
        const int hi = N - qb - 4 * g;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int off = 8 * (e >> 2) + (e & 3);
            s[e] = (off < lo || off >= hi) ? -INFINITY : s[e];
        }
    };

    f32x16 sc, dpc;            // S and dP of the current block
    u32x4 pf0[2], dsf0[2], pf1[2], dsf1[2];  // packed P, dS of even / odd blocks
    u32x4 ring[4];

    // Operand streams of the two kinds of step, as functions of the fragment
    // index: row fragments of block b (products) and transposed fragments of
    // block pb (dV/dK).  A step given WARM finds its first four fragments
    // already in the ring; a step given a `next` stream reads that stream's
    // first four fragments into the slots its last four MFMAs free, so the
    // ring runs on from step to step within a tile.
    auto rhead = [&](int b) __attribute__((always_inline)) {
        return [&, b](int j) __attribute__((always_inline)) { return rfrag(j & 1, b, j >> 1); };
    };
    auto thead = [&](int pb) __attribute__((always_inline)) {
        return [&, pb](int j) __attribute__((always_inline)) {
            return tfrag(1 - (j & 1), pb, (j >> 1) / MT, (j >> 1) % MT);
        };
    };
    // S and dP of block b of the tile behind rp: fragment f is the S product
    // (ks = f/2) for even f, the dP product for odd f.
    auto products = [&](int b, auto warm_c, auto next) __attribute__((always_inline)) {
        constexpr bool WARM = decltype(warm_c)::value;
        constexpr bool NEXT = !std::is_same_v<decltype(next), std::nullptr_t>;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!WARM) {
#pragma unroll
            for (int f = 0; f < 4; ++f) ring[f] = rfrag(f & 1, b, f >> 1);
        }
#pragma unroll
        for (int f = 0; f < 2 * KS; ++f) {
            const u32x4 x = ring[f & 3];
            if (f + 4 < 2 * KS) ring[f & 3] = rfrag((f + 4) & 1, b, (f + 4) >> 1);
            else if constexpr (NEXT) ring[f & 3] = next(f + 4 - 2 * KS);
            if (f & 1)
                dpc = M::run(x, vf[f >> 1], f < 2 ? f32x16{} : dpc);
            else
                sc = M::run(x, kf[f >> 1], f < 2 ? f32x16{} : sc);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Weights of the current block b (rows qb.., lse2 / D behind lp) into
    // (pf, dsf); with PREV, hosted between the 16 MFMAs of dV^T += dO^T P and
    // dK^T += Q^T dS of the previous block pb (tile behind tp) from (pfp,
    // dsfp): fragment f is dV (even) or dK (odd) of pair (u, mt) =
    // ((f/2) / MT, (f/2) % MT); element e of the weights runs after MFMA e.
    auto weights = [&](auto prev_c, int b, int qb, u32x4 (&pf)[2], u32x4 (&dsf)[2], int pb,
                       const u32x4 (&pfp)[2], const u32x4 (&dsfp)[2], auto warm_c, auto next) __attribute__((always_inline)) {
        constexpr bool PREV = decltype(prev_c)::value;
        constexpr bool WARM = decltype(warm_c)::value;
        constexpr bool NEXT = !std::is_same_v<decltype(next), std::nullptr_t>;
        if (needs_mask(qb)) mask_s(sc, qb);
        float p[16], ds[16];
        f32x4 l2, dd;
        auto host = [&](int e) __attribute__((always_inline)) {
            const int j4 = e >> 2, i = e & 3;
            if (i == 0) {
                l2 = lp[(32 * b + 8 * j4) / 4];
                dd = lp[(kBwdTile + 32 * b + 8 * j4) / 4];
            }
            p[e] = fast_exp2(fmaf(sc[e], a.scale_log2, -l2[i]));
            ds[e] = p[e] * (dpc[e] - dd[i]);
            // Anchor each result where it is computed, so the work stays
            // spread over the MFMA stream instead of sinking to its use.
            asm volatile("" ::"v"(p[e]), "v"(ds[e]));
            if (e & 1) {
                const int u = e >> 3, q = (e & 7) >> 1;
                pf[u][q] = M::pack(p[e - 1], p[e]);
                dsf[u][q] = M::pack(ds[e - 1], ds[e]);
                asm volatile("" ::"v"(pf[u][q]), "v"(dsf[u][q]));
            }
        };
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PREV) {
            if constexpr (!WARM) {
#pragma unroll
                for (int f = 0; f < 4; ++f) ring[f] = tfrag(1 - (f & 1), pb, (f >> 1) / MT, (f >> 1) % MT);
            }
#pragma unroll
            for (int f = 0; f < 4 * MT; ++f) {
                const u32x4 x = ring[f & 3];
                const int nf = f + 4;
                if (nf < 4 * MT) ring[f & 3] = tfrag(1 - (nf & 1), pb, (nf >> 1) / MT, (nf >> 1) % MT);
                else if constexpr (NEXT) ring[f & 3] = next(nf - 4 * MT);
                const int u = (f >> 1) / MT, mt = (f >> 1) % MT;
                if (f & 1)
                    dk_acc[mt] = M::run(x, dsfp[u], dk_acc[mt]);
                else
                    dv_acc[mt] = M::run(x, pfp[u], dv_acc[mt]);
                host(f);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) host(e);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    // dV, dK of block pb alone (the last block).
    auto finish = [&](int pb, const u32x4 (&pfp)[2], const u32x4 (&dsfp)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int f = 0; f < 4; ++f) ring[f] = tfrag(1 - (f & 1), pb, (f >> 1) / MT, (f >> 1) % MT);
#pragma unroll
        for (int f = 0; f < 4 * MT; ++f) {
            const u32x4 x = ring[f & 3];
            const int nf = f + 4;
            if (nf < 4 * MT) ring[f & 3] = tfrag(1 - (nf & 1), pb, (nf >> 1) / MT, (nf >> 1) % MT);
            const int u = (f >> 1) / MT, mt = (f >> 1) % MT;
            if (f & 1)
                dk_acc[mt] = M::run(x, dsfp[u], dk_acc[mt]);
            else
                dv_acc[mt] = M::run(x, pfp[u], dv_acc[mt]);
        }
    };
    std::integral_constant<bool, true> prev;
    std::integral_constant<bool, false> none;
    std::integral_constant<bool, true> warm;
    std::integral_constant<bool, false> cold;

    // Tile fi complete for all waves, tile fi+1's copies (if any) still in
    // flight; then the copies of tile fi+2 into the stage of tile fi-2,
    // whose last reads (dV/dK of its block 1) ran in the first step of tile
    // fi-1.
    auto arrive = [&](int fi) {
        if (fi + 1 < nflat) {
            if (w < 2)
                wait_vmcnt<2 * LPM + 1>();
            else
                wait_vmcnt<2 * LPM>();
        } else {
            wait_vmcnt<0>();
        }
        __syncthreads();
        issue(fi + 2);
    };
    issue(0);
    issue(1);
    arrive(0);
    rebase_rows(0);
    rebase_trans(0);
    // Tile 0: block 0 has no predecessor.
    int qb = tile_row0(0);
    products(0, cold, nullptr);
    weights(none, 0, qb, pf0, dsf0, 0, pf1, dsf1, cold, nullptr);
    products(1, cold, thead(0));
    weights(prev, 1, qb + 32, pf1, dsf1, 0, pf0, dsf0, warm, nullptr);
    for (int fi = 1; fi < nflat; ++fi) {
        arrive(fi);
        rebase_rows(fi);
        qb = tile_row0(fi);
        // Within the tile each step's last MFMAs read the next step's first
        // fragments (the barrier of arrive() separates the tiles).
        products(0, cold, thead(1));
        weights(prev, 0, qb, pf0, dsf0, 1, pf1, dsf1, warm, rhead(1));   // dV/dK of block 1 of tile fi-1
        rebase_trans(fi);
        products(1, warm, thead(0));
        weights(prev, 1, qb + 32, pf1, dsf1, 0, pf0, dsf0, warm, nullptr);
    }
    finish(1, pf1, dsf1);

    // Lane (col, g) holds d = 32 mt + 8 (i / 4) + 4 g + i % 4 of key `key`.
    if (key >= N) return;
    float* dkr = a.dk + (head + key) * D;
    float* dvr = a.dv + (head + key) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d = mt * 32 + 8 * i4 + 4 * g;
            *reinterpret_cast<f32x4*>(dkr + d) =
                f32x4{dk_acc[mt][4 * i4], dk_acc[mt][4 * i4 + 1], dk_acc[mt][4 * i4 + 2],
                      dk_acc[mt][4 * i4 + 3]} * a.scale;
            *reinterpret_cast<f32x4*>(dvr + d) =
                f32x4{dv_acc[mt][4 * i4], dv_acc[mt][4 * i4 + 1], dv_acc[mt][4 * i4 + 2],
                      dv_acc[mt][4 * i4 + 3]};
        }
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch_bwd(BwdArgs a, hipStream_t stream) {
    void* params[] = {(void*)&a};
    const int64_t rows = (int64_t)a.BH * a.N;
    const unsigned pre_grid = (unsigned)((rows + (256 / (D / 8)) - 1) / (256 / (D / 8)));
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_pre_kernel<BF16, D>),
                                   dim3(pre_grid), dim3(256), params, 0, stream);
    if (e != hipSuccess) return e;
    constexpr int kv_rows = 32 * dkdv_waves<D>();
    const unsigned grid = (unsigned)(((a.N + kv_rows - 1) / kv_rows) * a.BHkv);
    const void* dkdv;
    if constexpr (D == 128)
        dkdv = reinterpret_cast<const void*>(&attn_bwd_dkdv_pipe_kernel<BF16, CAUSAL>);
    else
        dkdv = reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<BF16, D, CAUSAL>);
    e = hipLaunchKernel(dkdv, dim3(grid), dim3(64 * dkdv_waves<D>()), params, 0, stream);
    if (e != hipSuccess) return e;
    const unsigned dq_grid = (unsigned)(((a.N + kDqRows - 1) / kDqRows) * a.BH);
    return hipLaunchKernel(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<BF16, D, CAUSAL>),
                           dim3(dq_grid), dim3(64 * kDqWaves), params, 0, stream);
}

}  // namespace

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const float* o,
                           const float* lse, const void* dout, float* dq, float* dk, float* dv,
                           float* workspace, int B, int H, int Hkv, int N, int D, bool causal,
                           bool bf16, hipStream_t stream) {
    BwdArgs a{};
    a.q = static_cast<const u16*>(q);
    a.k = static_cast<const u16*>(k);
    a.v = static_cast<const u16*>(v);
    a.o = o;
    a.lse = lse;
    a.dout = static_cast<const u16*>(dout);
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.BH = B * H;
    a.H = H;
    a.Hkv = Hkv;
    a.BHkv = B * Hkv;
    a.N = N;
    a.dd = workspace;
    a.lse2 = workspace + (int64_t)B * H * N;
    a.scale_log2 = kLog2e / __builtin_sqrtf((float)D);
    a.scale = 1.0f / __builtin_sqrtf((float)D);
    if (D == 128) {
        if (bf16)
            return causal ? launch_bwd<true, 128, true>(a, stream) : launch_bwd<true, 128, false>(a, stream);
        return causal ? launch_bwd<false, 128, true>(a, stream) : launch_bwd<false, 128, false>(a, stream);
    }
    if (bf16)
        return causal ? launch_bwd<true, 64, true>(a, stream) : launch_bwd<true, 64, false>(a, stream);
    return causal ? launch_bwd<false, 64, true>(a, stream) : launch_bwd<false, 64, false>(a, stream);
}

}  // namespace osc
