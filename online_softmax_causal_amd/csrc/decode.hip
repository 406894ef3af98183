// Paged grouped-query decode on gfx950: one query token per request attends
// over that request's cached keys and values, which live in fixed-size pages
// of a shared cache and are found through a per-request page table.
//
// Method: "CUDA KV Cache: paged storage and long-context decode"
// (chengzipai.xyz).  Section 2: the cache is [P][2][T][Hkv][D] (page, K or V,
// token within the page, K/V head, dim) and logical token t of request b sits
// in physical page block_table[b][t / T] at offset t mod T.  Section 3: the
// address translation is done inside the attention kernel (no gathered copy)
// and the g = Hq / Hkv query heads of a group read the same K/V head
// floor(h / g) (no copied heads).  Section 5: per token, a score q.k/sqrt(D),
// then the online-softmax update of the running max, running sum and FP32
// output.  Section 6.3: one workgroup serves a whole query-head group, so the
// group's K/V are read once.  Section 6.4: the tokens are split into segments
// whose partial states (m, l, o) are merged afterwards.
//
// gfx950 mapping (one wave per workgroup, one workgroup per (segment,
// request, K/V head)):
//   * The group's g <= 32 query heads are the 32 columns of the MFMA B
//     operand (columns past g hold zeros and are never stored), exactly as 32
//     query rows are in the prefill kernel: S^T = K Q^T and O^T += V^T P^T on
//     v_mfma_f32_32x32x16, one lane per (head, half of the keys).
//   * Tiles of 32 tokens are gathered page by page straight into LDS with
//     global_load_lds_dwordx4 (each lane copies 16 bytes of one token row;
//     the row's page comes from the segment's page ids, staged in LDS once),
//     four stages deep, three tiles ahead.  Rows past the request's length
//     re-read its last token and are masked.
//   * The online-softmax state and its conditional rescale are those of the
//     prefill kernel (base-2 units, slack 2^8).
//
// HBM-bound: per (request, K/V head) the kernel reads len * D * 2 * 2 bytes of
// K and V once; the MFMA work (padded to 32 heads) is far below the matrix
// rate at that traffic.
//
// Invalid device data (a length outside [1, max_pages * T] or a page id
// outside [0, P) among the pages a request uses) cannot be reported through
// the C call, which returns before the kernel runs: such a request's outputs
// are set to NaN and no out-of-range address is read.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"
#include "mfma_tile.hpp"
#include "online_merge.hpp"

namespace osc {
namespace {

constexpr int kDecStages = 4;  // LDS stages
constexpr int kDecDist = 3;    // tiles copied ahead of the one being computed

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

}  // namespace

// Segments: the automatic plan aims at about 512 workgroups (B * Hkv *
// segments), one round of two resident workgroups per CU: more segments add
// merge traffic and per-workgroup start-up for no extra bandwidth (measured
// on the benchmark shapes, 1K to 32K tokens).  A caller's request > 0 is
// taken as is.  Segments are whole tiles
// and at most kDecMaxSegTokens tokens (the LDS page-id slots), so the count
// is then raised to what the capacity needs.  Sized by the capacity
// max_pages * T, since the lengths are device data the host does not read.
DecodePlan paged_decode_plan(int64_t B, int64_t Hkv, int64_t cap, int requested) {
    const int64_t tiles = (cap + kDecTile - 1) / kDecTile;
    int64_t want = requested > 0 ? requested : (512 + B * Hkv - 1) / (B * Hkv);
    if (want > tiles) want = tiles;
    if (want < 1) want = 1;
    int64_t seg_tiles = (tiles + want - 1) / want;
    const int64_t max_tiles = kDecMaxSegTokens / kDecTile;
    if (seg_tiles > max_tiles) seg_tiles = max_tiles;
    DecodePlan p;
    p.seg_tokens = (int)(seg_tiles * kDecTile);
    p.nseg = (int)((tiles + seg_tiles - 1) / seg_tiles);
    return p;
}

hipError_t launch_paged_decode(const void* q, const void* cache, const int* block_table,
                               const int* lengths, float* o, float* lse, int B, int Hq, int Hkv,
                               int D, int log2_page, int P, int max_pages, bool bf16,
                               const DecodePlan& plan, float* part_o, float2* part_ml,
                               hipStream_t stream) {
    DecodeArgs a{};
    a.q = static_cast<const u16*>(q);
    a.cache = static_cast<const u16*>(cache);
    a.block_table = block_table;
    a.lengths = lengths;
    a.o = o;
    a.lse = lse;
    a.part_o = part_o;
    a.part_ml = part_ml;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.P = P;
    a.max_pages = max_pages;
    a.log2_page = log2_page;
    a.seg_tokens = plan.seg_tokens;
    a.nseg = plan.nseg;
    a.scale_log2 = kLog2e / __builtin_sqrtf((float)D);
    const void* fn;
    if (D == 128)
        fn = bf16 ? reinterpret_cast<const void*>(&paged_decode_kernel<true, 128>)
                  : reinterpret_cast<const void*>(&paged_decode_kernel<false, 128>);
    else
        fn = bf16 ? reinterpret_cast<const void*>(&paged_decode_kernel<true, 64>)
                  : reinterpret_cast<const void*>(&paged_decode_kernel<false, 64>);
    void* params[] = {(void*)&a};
    const unsigned grid = (unsigned)((int64_t)B * Hkv * plan.nseg);
    hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(64), params, 0, stream);
    if (e != hipSuccess || plan.nseg == 1) return e;
    return launch_splitkv_merge(part_o, part_ml, o, lse, B * Hq, 1, D, plan.nseg, 1, false, stream);
}

}  // namespace osc
