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
#include "decode_kernel.hpp"

namespace osc {

namespace {
constexpr int kDecShortSegTokens = 512;  // see launch_paged_decode
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
    const unsigned grid = (unsigned)((int64_t)B * Hkv * plan.nseg);
    // Segments of at most kDecShortSegTokens tokens run the VGPR-form build of
    // the kernel (no accumulator copies between AGPRs and VGPRs), longer ones
    // this file's: in paired runs (B8 Hq32 Hkv8 D128, 16-token pages) the
    // VGPR form took 8-9% off 128- and 512-token segments, matched at 1024 and
    // was 3.6% slower at 2048.
    const hipError_t e = plan.seg_tokens <= kDecShortSegTokens
                             ? launch_decode_kernel_vgpr(a, bf16, D, grid, stream)
                             : launch_decode_kernel_here(a, bf16, D, grid, stream);
    if (e != hipSuccess || plan.nseg == 1) return e;
    return launch_splitkv_merge(part_o, part_ml, o, lse, B * Hq, 1, D, plan.nseg, 1, false, stream);
}

}  // namespace osc
