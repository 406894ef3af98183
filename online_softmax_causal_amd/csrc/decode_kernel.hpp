// The paged decode kernel, compiled twice from this one source: by
// decode.hip as every other kernel is built, and by decode_short.hip with
// VGPR-form MFMAs (the form that is faster for short segments; see
// launch_paged_decode).  The kernel sits in an anonymous namespace, so each
// file links its own instantiation.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"
#include "mfma_tile.hpp"
#include "online_merge.hpp"

namespace osc {

struct DecodeArgs {
    const u16* q;            // [B, Hq, D]
    const u16* cache;        // [P, 2, T, Hkv, D]
    const int* block_table;  // [B, max_pages]
    const int* lengths;      // [B]
    float* o;                // [B, Hq, D]      (one segment)
    float* lse;              // [B, Hq]
    float* part_o;           // [nseg, B*Hq, D] (several segments)
    float2* part_ml;         // [nseg, B*Hq]: (m, l), base-2 units
    int B, Hq, Hkv, P, max_pages;
    int log2_page;           // T = 2^log2_page tokens per page
    int seg_tokens;          // tokens per segment, a multiple of kDecTile
    int nseg;
    float scale_log2;        // log2(e) / sqrt(D)
};

// paged_decode_kernel<bf16, D> over `grid` workgroups of one wave, as built in
// decode_short.hip (VGPR-form MFMAs).
hipError_t launch_decode_kernel_vgpr(const DecodeArgs& a, bool bf16, int D, unsigned grid,
                                     hipStream_t stream);

namespace {

constexpr int kDecStages = 4;  // LDS stages
constexpr int kDecDist = 3;    // tiles copied ahead of the one being computed


template <bool BF16, int D>
__global__ void __launch_bounds__(64)
paged_decode_kernel(DecodeArgs a) {
    using M = Mma<BF16>;
    constexpr int CPR = D / 8;            // 16-byte chunks per row
    constexpr int RPB = 1024 / (2 * D);   // rows per 1 KiB copy block
    constexpr int BPT = kDecTile / RPB;   // copy blocks per tile (K or V)
    constexpr int LPT = 2 * BPT;          // copies per tile
    constexpr int TILE = kDecTile * D;    // 16-bit elements per K (or V) tile
    constexpr int KS = D / 16, MT = D / 32;
    __shared__ __attribute__((aligned(1024))) u16 lds[kDecStages * 2 * TILE];
    __shared__ int page_ids[kDecMaxSegTokens + 1];

    const int lane = threadIdx.x;
    const int col = lane & 31, g = lane >> 5;
    const int group = a.Hq / a.Hkv;
    const int bid = blockIdx.x;
    const int kvh = bid % a.Hkv;
    const int b = (bid / a.Hkv) % a.B;
    const int seg = bid / (a.Hkv * a.B);
    const int lp = a.log2_page;
    const int T = 1 << lp;
    const int cap = a.max_pages << lp;
    const int len = a.lengths[b];
    bool bad = len < 1 || len > cap;
    const int t0 = seg * a.seg_tokens;
    const int t1 = bad ? t0 : min(t0 + a.seg_tokens, len);
    const int ntl = t1 > t0 ? (t1 - t0 + kDecTile - 1) / kDecTile : 0;

    // Page ids of the segment's pages, checked against the cache size.
    const int p0 = t0 >> lp;
    const int np = ntl > 0 ? ((t1 - 1) >> lp) - p0 + 1 : 0;
    bool pid_bad = false;
    for (int i = lane; i < np; i += 64) {
        int pid = a.block_table[(int64_t)b * a.max_pages + p0 + i];
        if (pid < 0 || pid >= a.P) {
            pid_bad = true;
            pid = 0;
        }
        page_ids[i] = pid;
    }
    bad = bad || __builtin_amdgcn_ballot_w64(pid_bad) != 0;
    const int ntiles = bad ? 0 : ntl;
    __syncthreads();

    // Query fragments (MFMA B operand): column col is query head
    // kvh * group + col of request b.
    const int head = kvh * group + col;
    const bool live_col = col < group;
    const int64_t qrow = (int64_t)b * a.Hq + head;
    u32x4 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = live_col ? *reinterpret_cast<const u32x4*>(a.q + qrow * D + ks * 16 + 8 * g)
                          : u32x4{0u, 0u, 0u, 0u};

    // LDS offsets of this lane's K fragment (one per 16-wide d step, key row
    // col) and V^T fragment halves (ds_read_b64_tr_b16: rows tr_key and
    // tr_key + 8 of each 16-key group).
    const int sw = chunk_swizzle<D>(col);
    int fk[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) fk[ks] = col * D + (((2 * ks + g) ^ sw) << 3);
    const int tr_key = 4 * g + ((lane >> 2) & 3);
    const int dh = (lane >> 4) & 1;
    int fv[MT][2];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = tr_key + 8 * r;
            const int c = 4 * mt + 2 * dh + ((lane & 3) >> 1);
            fv[mt][r] = row * D + ((c ^ chunk_swizzle<D>(row)) << 3) + 4 * (lane & 1);
        }

    const int64_t kv_stride = (int64_t)T * a.Hkv * D;  // K row -> V row of the same token
    auto issue = [&](int i) {
        if (i >= ntiles) return;
        const int tt0 = t0 + i * kDecTile;
        u16* kd = lds + (i % kDecStages) * 2 * TILE;
#pragma unroll
        for (int j = 0; j < BPT; ++j) {
            const int r = j * RPB + lane / CPR;
            const int c = (lane % CPR) ^ chunk_swizzle<D>(r);
            const int t = min(tt0 + r, t1 - 1);
            const int pid = page_ids[(t >> lp) - p0];
            const int64_t row = ((int64_t)pid * 2 * T + (t & (T - 1))) * a.Hkv + kvh;
            const u16* src = a.cache + row * D + c * 8;
            // Each cached row is read by one workgroup once per call: the
            // copies carry the non-temporal hint, so the stream does not
            // displace reusable lines from the caches.
            copy_to_lds16_at_nt(src, kd + j * 512);
            copy_to_lds16_at_nt(src + kv_stride, kd + TILE + j * 512);
        }
    };

    f32x16 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
    float m = -INFINITY, l = 0.0f;

    // Q (and the page ids) first, so that no later wait for them also waits
    // for the tile copies.
    wait_vmcnt<0>();
#pragma unroll
    for (int i = 0; i < kDecDist; ++i) issue(i);
    for (int i = 0; i < ntiles; ++i) {
        // Tile i complete: the copies of tiles i+1, i+2 may stay in flight.
        const int ahead = min(ntiles - 1 - i, kDecDist - 1);
        if (ahead >= 2)
            wait_vmcnt<2 * LPT>();
        else if (ahead == 1)
            wait_vmcnt<LPT>();
        else
            wait_vmcnt<0>();
        // Stage (i + 3) % 4 held tile i - 1, whose reads all completed in the
        // previous iteration.
        issue(i + kDecDist);
        const u16* kt = lds + (i % kDecStages) * 2 * TILE;
        const u16* vt = kt + TILE;

        f32x16 s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            s = M::run(*reinterpret_cast<const u32x4*>(kt + fk[ks]), qf[ks], s);
        // Lane (col, g) holds keys 8(e/4) + 4g + e%4 of the tile; keys at or
        // past t1 are masked.
        const int tt0 = t0 + i * kDecTile;
        if (tt0 + kDecTile > t1) {
            const int lim = t1 - 1 - tt0 - 4 * g;
#pragma unroll
            for (int e = 0; e < 16; ++e) s[e] = 8 * (e >> 2) + (e & 3) > lim ? -INFINITY : s[e];
        }
        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, s[e]);
        mx = fmaxf(mx, swap32_f32(mx));
        const float tile_m = mx * a.scale_log2;
        const bool grow = tile_m > m + rescale_slack<BF16>();
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float m_new = grow ? tile_m : m;
            const float alpha = grow ? online_rescale(m, m_new) : 1.0f;
            l *= alpha;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
            m = m_new;
        }
        const float pivot = online_pivot(m);
        u32x4 pf[2];
        float rs0 = 0.0f, rs1 = 0.0f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float p[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) p[jj] = fast_exp2(fmaf(s[8 * u + jj], a.scale_log2, -pivot));
            pf[u] = u32x4{M::pack(p[0], p[1]), M::pack(p[2], p[3]), M::pack(p[4], p[5]),
                          M::pack(p[6], p[7])};
            if constexpr (M::kSumRounded) {
                rs0 = M::sum2(pf[u][0], rs0);
                rs1 = M::sum2(pf[u][1], rs1);
                rs0 = M::sum2(pf[u][2], rs0);
                rs1 = M::sum2(pf[u][3], rs1);
            } else {
#pragma unroll
                for (int jj = 0; jj < 8; jj += 2) {
                    rs0 += p[jj];
                    rs1 += p[jj + 1];
                }
            }
        }
        l += rs0 + rs1;
        // O^T += V^T P^T, 16 keys per MFMA: B-operand slot 8g+j of group u
        // holds key 16u + 8(j/4) + 4g + j%4, the order of the S^T layout.
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const u16* base = vt + u * 16 * D;
                acc[mt] = M::run(tr16_b64x2(base + fv[mt][0], base + fv[mt][1]), pf[u], acc[mt]);
            }
    }

    // Epilogue: lanes col and col + 32 hold halves of head col's sum and the
    // d rows 8(e/4) + 4g + e%4 of each 32-row block of O^T.
    const float l_tot = l + swap32_f32(l);
    if (!live_col) return;
    const float nan = __builtin_nanf("");
    if (a.nseg > 1) {
        const int64_t part = (int64_t)seg * a.B * a.Hq + qrow;
        float* po = a.part_o + part * D;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f32x4 r = {acc[mt][4 * i4 + 0], acc[mt][4 * i4 + 1], acc[mt][4 * i4 + 2],
                           acc[mt][4 * i4 + 3]};
                if (bad) r = f32x4{nan, nan, nan, nan};
                *reinterpret_cast<f32x4*>(po + mt * 32 + 8 * i4 + 4 * g) = r;
            }
        if (g == 0) a.part_ml[part] = bad ? float2{nan, nan} : float2{m, l_tot};
        return;
    }
    const float inv = bad ? nan : 1.0f / l_tot;
    float* orow = a.o + qrow * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 r = {acc[mt][4 * i4 + 0] * inv, acc[mt][4 * i4 + 1] * inv,
                             acc[mt][4 * i4 + 2] * inv, acc[mt][4 * i4 + 3] * inv};
            *reinterpret_cast<f32x4*>(orow + mt * 32 + 8 * i4 + 4 * g) = r;
        }
    if (g == 0) a.lse[qrow] = bad ? nan : (m + log2f(l_tot)) * kLn2;
}

// paged_decode_kernel<bf16, D> as built in the including file.
inline hipError_t launch_decode_kernel_here(const DecodeArgs& a, bool bf16, int D, unsigned grid,
                                            hipStream_t stream) {
    const void* fn;
    if (D == 128)
        fn = bf16 ? reinterpret_cast<const void*>(&paged_decode_kernel<true, 128>)
                  : reinterpret_cast<const void*>(&paged_decode_kernel<false, 128>);
    else
        fn = bf16 ? reinterpret_cast<const void*>(&paged_decode_kernel<true, 64>)
                  : reinterpret_cast<const void*>(&paged_decode_kernel<false, 64>);
    DecodeArgs copy = a;
    void* params[] = {(void*)&copy};
    return hipLaunchKernel(fn, dim3(grid), dim3(64), params, 0, stream);
}

}  // namespace
}  // namespace osc
