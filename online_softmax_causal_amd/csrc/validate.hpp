// Host-side argument checks for the C ABI.  Pure C++: no HIP call, so every
// rejection happens before anything touches the device (and can be exercised
// on a machine without a GPU).
#pragma once

#include <cstdint>

#include "osc_attn.h"

namespace osc {

// a*b for non-negative operands, false if it would reach 2^62.
inline bool mul_below_2_62(int64_t a, int64_t b, int64_t* out) {
    const int64_t lim = int64_t(1) << 62;
    if (a != 0 && b > (lim - 1) / a) return false;
    *out = a * b;
    return true;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + static_cast<uintptr_t>(bbytes) && b0 < a0 + static_cast<uintptr_t>(abytes);
}

// q, o, lse cover B*H heads; k, v cover B*Hkv heads (Hkv divides H).
inline attn_status_t validate_attn(const void* q, const void* k, const void* v, const float* o,
                                   const float* lse, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                                   int64_t D, attn_dtype_t dtype) {
    if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || Hkv < 1 || N < 1 || D < 1) return ATTN_ERR_SHAPE;
    if (Hkv > H || H % Hkv != 0) return ATTN_ERR_SHAPE;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return ATTN_ERR_UNSUPPORTED;
    int64_t bh = 0, bhn = 0, total = 0, nd = 0;
    if (!mul_below_2_62(B, H, &bh) || !mul_below_2_62(bh, N, &bhn) ||
        !mul_below_2_62(bhn, D, &total) || !mul_below_2_62(N, D, &nd))
        return ATTN_ERR_SHAPE;
    if (nd >= (int64_t(1) << 31) || bh >= (int64_t(1) << 31)) return ATTN_ERR_SHAPE;
    // One workgroup per 128-query tile at most: the grid must stay below 2^31.
    if (bh * ((N + 127) / 128) >= (int64_t(1) << 31)) return ATTN_ERR_SHAPE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lse, 4))
        return ATTN_ERR_ALIGN;
    const int64_t q_bytes = total * 2, kv_bytes = (total / H) * Hkv * 2;
    const int64_t o_bytes = total * 4, lse_bytes = bhn * 4;
    const void* ins[3] = {q, k, v};
    const int64_t in_bytes[3] = {q_bytes, kv_bytes, kv_bytes};
    for (int i = 0; i < 3; ++i)
        if (overlap(o, o_bytes, ins[i], in_bytes[i]) || overlap(lse, lse_bytes, ins[i], in_bytes[i]))
            return ATTN_ERR_ALIAS;
    if (overlap(o, o_bytes, lse, lse_bytes)) return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

// Workspace of a split-KV call that needs `need` bytes (0: none is used).
// The attention arguments have been validated already.
inline attn_status_t validate_workspace(const void* ws, int64_t ws_bytes, int64_t need,
                                        const void* q, const void* k, const void* v,
                                        const float* o, const float* lse, int64_t B, int64_t H,
                                        int64_t Hkv, int64_t N, int64_t D) {
    if (need == 0) return ATTN_OK;
    if (!ws) return ATTN_ERR_NULL;
    if (!aligned(ws, 16)) return ATTN_ERR_ALIGN;
    if (ws_bytes < need) return ATTN_ERR_WORKSPACE;
    const int64_t total = B * H * N * D;
    const int64_t kv = B * Hkv * N * D * 2;
    if (overlap(ws, need, q, total * 2) || overlap(ws, need, k, kv) || overlap(ws, need, v, kv) ||
        overlap(ws, need, o, total * 4) || overlap(ws, need, lse, B * H * N * 4))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

// Attention backward: q, k, v, dout [B,H,N,D] 16-bit; o, dq, dk, dv [B,H,N,D]
// and lse [B,H,N] FP32; workspace 8*B*H*N bytes.  The sizes and q, k, v, o,
// lse were checked by validate_attn (Hkv = H).
inline attn_status_t validate_bwd(const void* q, const void* k, const void* v, const float* o,
                                  const float* lse, const void* dout, const float* dq,
                                  const float* dk, const float* dv, const void* ws,
                                  int64_t ws_bytes, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                                  int64_t D) {
    if (!dout || !dq || !dk || !dv || !ws) return ATTN_ERR_NULL;
    if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(ws, 16))
        return ATTN_ERR_ALIGN;
    // Sizes were checked by validate_attn (below 2^62, Hkv divides H).
    const int64_t total = B * H * N * D, rows = B * H * N, kv = B * Hkv * N * D;
    if (ws_bytes < 8 * rows) return ATTN_ERR_WORKSPACE;
    const void* ins[6] = {q, k, v, o, lse, dout};
    const int64_t in_bytes[6] = {total * 2, kv * 2, kv * 2, total * 4, rows * 4, total * 2};
    const void* outs[4] = {dq, dk, dv, ws};
    const int64_t out_bytes[4] = {total * 4, kv * 4, kv * 4, rows * 8};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(outs[i], out_bytes[i], ins[j], in_bytes[j])) return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], out_bytes[i], outs[j], out_bytes[j])) return ATTN_ERR_ALIAS;
    }
    return ATTN_OK;
}

// Sizes of a paged decode call: false if they are invalid (a size < 1, Hkv
// not dividing Hq, or a product past the limits); *status then says which
// code to return.  Sets *log2_page for valid sizes.
inline bool paged_sizes_ok(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                           int64_t num_pages, int64_t max_pages, attn_status_t* status,
                           int* log2_page) {
    *status = ATTN_ERR_SHAPE;
    if (B < 1 || Hq < 1 || Hkv < 1 || D < 1 || page_size < 1 || num_pages < 1 || max_pages < 1)
        return false;
    if (Hq % Hkv != 0) return false;
    *status = ATTN_ERR_UNSUPPORTED;
    if (D != 64 && D != 128) return false;
    if (Hq / Hkv > 32) return false;
    if (page_size > 65536 || (page_size & (page_size - 1)) != 0) return false;
    int lp = 0;
    while ((int64_t(1) << lp) < page_size) ++lp;
    *log2_page = lp;
    *status = ATTN_ERR_SHAPE;
    int64_t rows = 0, elems = 0, cap = 0, bt = 0, bq = 0, bqd = 0;
    if (!mul_below_2_62(num_pages * 2, page_size, &rows) || !mul_below_2_62(rows, Hkv, &rows) ||
        !mul_below_2_62(rows, D, &elems))
        return false;
    if (!mul_below_2_62(max_pages, page_size, &cap) || cap >= (int64_t(1) << 31)) return false;
    if (!mul_below_2_62(B, max_pages, &bt) || bt >= (int64_t(1) << 31)) return false;
    if (!mul_below_2_62(B, Hq, &bq) || !mul_below_2_62(bq, D, &bqd) || bq >= (int64_t(1) << 31))
        return false;
    if (num_pages >= (int64_t(1) << 31)) return false;
    return true;
}

// Pointers of a paged decode call whose sizes passed paged_sizes_ok.
inline attn_status_t validate_paged(const void* q, const void* cache, const int32_t* block_table,
                                    const int32_t* lengths, const float* o, const float* lse,
                                    int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                    int64_t page_size, int64_t num_pages, int64_t max_pages,
                                    attn_dtype_t dtype) {
    if (!q || !cache || !block_table || !lengths || !o || !lse) return ATTN_ERR_NULL;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
    if (!aligned(q, 16) || !aligned(cache, 16) || !aligned(o, 16) || !aligned(block_table, 4) ||
        !aligned(lengths, 4) || !aligned(lse, 4))
        return ATTN_ERR_ALIGN;
    const int64_t q_bytes = B * Hq * D * 2;
    const int64_t cache_bytes = num_pages * 2 * page_size * Hkv * D * 2;
    const int64_t bt_bytes = B * max_pages * 4, len_bytes = B * 4;
    const int64_t o_bytes = B * Hq * D * 4, lse_bytes = B * Hq * 4;
    const void* ins[4] = {q, cache, block_table, lengths};
    const int64_t in_bytes[4] = {q_bytes, cache_bytes, bt_bytes, len_bytes};
    for (int i = 0; i < 4; ++i)
        if (overlap(o, o_bytes, ins[i], in_bytes[i]) || overlap(lse, lse_bytes, ins[i], in_bytes[i]))
            return ATTN_ERR_ALIAS;
    if (overlap(o, o_bytes, lse, lse_bytes)) return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

// Workspace of a paged decode call that needs `need` bytes (0: none is used).
inline attn_status_t validate_paged_workspace(const void* ws, int64_t ws_bytes, int64_t need,
                                              const void* q, const void* cache,
                                              const int32_t* block_table, const int32_t* lengths,
                                              const float* o, const float* lse, int64_t B,
                                              int64_t Hq, int64_t Hkv, int64_t D,
                                              int64_t page_size, int64_t num_pages,
                                              int64_t max_pages) {
    if (need == 0) return ATTN_OK;
    if (!ws) return ATTN_ERR_NULL;
    if (!aligned(ws, 16)) return ATTN_ERR_ALIGN;
    if (ws_bytes < need) return ATTN_ERR_WORKSPACE;
    if (overlap(ws, need, q, B * Hq * D * 2) ||
        overlap(ws, need, cache, num_pages * 2 * page_size * Hkv * D * 2) ||
        overlap(ws, need, block_table, B * max_pages * 4) || overlap(ws, need, lengths, B * 4) ||
        overlap(ws, need, o, B * Hq * D * 4) || overlap(ws, need, lse, B * Hq * 4))
        return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

inline attn_status_t validate_softmax(const float* x, const float* y, int64_t M, int64_t N) {
    if (!x || !y) return ATTN_ERR_NULL;
    if (M < 1 || N < 1) return ATTN_ERR_SHAPE;
    int64_t total = 0;
    if (!mul_below_2_62(M, N, &total)) return ATTN_ERR_SHAPE;
    if (M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31)) return ATTN_ERR_SHAPE;
    if (!aligned(x, 4) || !aligned(y, 4)) return ATTN_ERR_ALIGN;
    if (overlap(x, total * 4, y, total * 4)) return ATTN_ERR_ALIAS;
    return ATTN_OK;
}

}  // namespace osc
