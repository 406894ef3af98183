/*
 * osc_attn.h - C ABI of the MI355X (gfx950) attention library
 * (libosc_attn.so).
 *
 * Operations, all from the reference pages:
 *
 *   attn_fwd     exact scaled-dot-product attention forward,
 *                O = softmax(Q K^T / sqrt(D) + M) V, with M the causal mask
 *                (M_ij = 0 if j <= i, else -inf) or no mask.  Definition:
 *                "CUDA FlashAttention: from online softmax to long-sequence IO
 *                limits" (chengzipai.xyz), section 1; computed with the tiled
 *                online-softmax recurrence of its section 4 (running max m,
 *                running sum l, unnormalised FP32 output rescaled per K/V
 *                tile), which reaches the same result as the plain definition
 *                up to floating-point rounding.
 *   attn_fwd_gqa      the same with fewer K/V heads than query heads.
 *   attn_fwd_splitkv  the same with every head's keys split into segments
 *                whose partial states are merged afterwards.
 *   paged_decode one decode step over a paged K/V cache.
 *   attn_bwd     gradients of attn_fwd with respect to q, k and v.
 *   attn_bwd_gqa the same for attn_fwd_gqa (grouped K/V heads).
 *
 *   row_softmax  y = softmax(x) along each row of an FP32 matrix, computed
 *                with the online (m, d) recurrence and two-level merge of the
 *                softmax kernel study (lpnh.cn/news/2830604), sections 4.4
 *                and 4.6.  It shares its merge code with attn_fwd.
 *
 * Conventions (all entry points):
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates no memory (scratch space comes from a caller's workspace
 *     argument; paged_decode_noalloc uses a fixed array of the library
 *     instead, whose device address it keeps), keeps no other state between
 *     calls and never synchronises.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns at once.  Completion is observed with the caller's own stream or
 *     event synchronisation; a fault during execution surfaces there.
 *   - Arguments are validated before anything is enqueued.  On any error
 *     nothing is enqueued and the outputs are left untouched, with one
 *     exception: the calls that launch several kernels in order
 *     (attn_fwd_splitkv, paged_decode, paged_decode_noalloc, attn_bwd,
 *     attn_bwd_gqa) return ATTN_ERR_LAUNCH if the runtime refuses a later
 *     launch, and the kernels launched before it stay enqueued; the
 *     workspace and the outputs are then undefined.
 *   - Tensors are dense and row-major (contiguous); the library cannot check
 *     that the buffers are as large as the sizes say.
 *   - Unsupported shapes are rejected, never answered approximately (FA page,
 *     section 9: unsupported shapes must fall back explicitly rather than give
 *     silently wrong results).
 */
#ifndef OSC_ATTN_H
#define OSC_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same opaque type as HIP's hipStream_t. */
typedef struct ihipStream_t *hipStream_t;

/* Storage type of Q, K and V.  Arithmetic is FP32 in both cases: products on
 * the matrix cores accumulate in FP32, and the softmax state (m, l) and the
 * output accumulator are FP32 (FA page, section 2). */
typedef enum {
    ATTN_F16 = 0,  /* IEEE binary16 */
    ATTN_BF16 = 1  /* bfloat16 */
} attn_dtype_t;

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
    ATTN_ERR_SHAPE = 2,       /* a size < 1, or sizes whose product overflows the limits below */
    ATTN_ERR_UNSUPPORTED = 3, /* head dim not 64 or 128, or unknown dtype */
    ATTN_ERR_ALIGN = 4,       /* a pointer is not aligned as required below */
    ATTN_ERR_LAUNCH = 5,      /* the HIP runtime refused the kernel launch */
    ATTN_ERR_ALIAS = 6,       /* an output or workspace buffer overlaps another buffer */
    ATTN_ERR_WORKSPACE = 7    /* the workspace is smaller than the call needs */
} attn_status_t;

/* Largest segment count attn_fwd_splitkv accepts. */
#define ATTN_MAX_SPLITS 64

/*
 * attn_fwd - attention forward for B*H independent heads.
 *
 *   q, k, v  [B, H, N, D] of `dtype`, contiguous: element (b,h,n,d) at
 *            ((b*H + h)*N + n)*D + d.  16-byte aligned.
 *   o        [B, H, N, D] FP32 output, same indexing, 16-byte aligned.
 *            Row i of head (b,h) is sum_j p_ij v_j with p_ij the softmax
 *            weights of the scaled logits s_ij = q_i . k_j / sqrt(D).
 *   lse      [B, H, N] FP32 output, 4-byte aligned: the natural-log
 *            log-sum-exp of the scaled logits of each row,
 *            lse_i = ln sum_{j in J_i} exp(s_ij), kept for a backward pass
 *            (FA page, section 7).
 *   B, H, N  batch, heads, sequence length (Q and K/V have the same N).
 *   D        head dimension: 64 or 128 (FA page, section 7, gives these two
 *            dedicated layouts; other D return ATTN_ERR_UNSUPPORTED).
 *   causal   nonzero: key j is visible to query i iff j <= i (top-left
 *            aligned); zero: every key is visible.
 *   dtype    ATTN_F16 or ATTN_BF16, the storage type of q, k and v.
 *   stream   HIP stream to enqueue on.
 *
 * Limits: N*D < 2^31, B*H < 2^31, B*H*ceil(N/128) < 2^31 (the workgroup
 * count) and B*H*N*D < 2^62; other sizes ATTN_ERR_SHAPE.  o and lse must
 * not overlap q, k, v or each other.  The softmax scale is fixed at
 * 1/sqrt(D).
 */
attn_status_t attn_fwd(const void *q, const void *k, const void *v, float *o, float *lse,
                       int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                       attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_fwd_gqa - attention forward with grouped key/value heads
 * (grouped-query / multi-query attention).
 *
 * Query head h of batch b attends with K/V head floor(h / (H / Hkv)) of the
 * same batch, without the K/V heads being copied ("CUDA KV Cache: paged
 * storage and long-context decode" (chengzipai.xyz), section 3: the query
 * head maps to the shared KV head as h_kv = floor(h_q / g); FA page,
 * section 7).  Hkv = H is attn_fwd; Hkv = 1 is multi-query attention.
 *
 *   q        [B, H, N, D] of `dtype`, 16-byte aligned.
 *   k, v     [B, Hkv, N, D] of `dtype`, 16-byte aligned.
 *   o, lse   as for attn_fwd ([B, H, N, D] and [B, H, N], FP32).
 *   Hkv      number of key/value heads: 1 <= Hkv <= H and H % Hkv == 0,
 *            else ATTN_ERR_SHAPE.
 * Everything else (D, dtype, causal, limits, errors, stream) is as for attn_fwd.
 */
attn_status_t attn_fwd_gqa(const void *q, const void *k, const void *v, float *o, float *lse,
                           int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal,
                           attn_dtype_t dtype, hipStream_t stream);

/*
 * attn_fwd_splitkv - attention forward with the keys of every head split into
 * segments (split-KV).
 *
 * Each workgroup handles one query tile against one key segment and stores
 * that segment's partial state (m, l, unnormalised o) in the workspace; a
 * second kernel then merges the segments of each row with
 * m = max_s m_s, l = sum_s l_s e^(m_s - m), O = sum_s o_s e^(m_s - m) / l
 * ("CUDA KV Cache: paged storage and long-context decode" (chengzipai.xyz),
 * section 6.4; FA page, section 7: split along K for long sequences with few
 * heads).  The result is the attn_fwd_gqa result up to rounding.  Both
 * kernels are enqueued on `stream`.
 *
 *   q, k, v, o, lse, B, H, Hkv, N, D, causal, dtype  as for attn_fwd_gqa.
 *   num_splits  0: the library chooses (one segment when B*H and N already
 *               fill the GPU, else up to 16); 1..ATTN_MAX_SPLITS: that many
 *               segments at most.  Segments hold a multiple of 256 keys, so
 *               fewer may be used for short N.  Larger values: ATTN_ERR_SHAPE.
 *   workspace   device buffer owned by the caller, 16-byte aligned, of at
 *               least attn_fwd_splitkv_workspace(B, H, N, D, causal,
 *               num_splits) bytes; it must not overlap q, k, v, o or lse.
 *               Its contents on entry do not matter and are undefined after
 *               the call.  May be NULL when that size is 0 (one segment).
 *               Two calls that run at the same time need separate workspaces.
 *   workspace_bytes  size of `workspace`; too small: ATTN_ERR_WORKSPACE.
 */
attn_status_t attn_fwd_splitkv(const void *q, const void *k, const void *v, float *o, float *lse,
                               int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal,
                               attn_dtype_t dtype, int num_splits, void *workspace,
                               int64_t workspace_bytes, hipStream_t stream);

/*
 * attn_fwd_splitkv_workspace - bytes of workspace attn_fwd_splitkv needs for
 * these sizes (0 if it uses one segment), or -1 if the sizes or num_splits
 * are invalid.  Pure host computation; enqueues nothing.
 */
int64_t attn_fwd_splitkv_workspace(int64_t B, int64_t H, int64_t N, int64_t D, int causal,
                                   int num_splits);

/* Largest segment count paged_decode accepts. */
#define PAGED_MAX_SPLITS 4096

/*
 * paged_decode - one decode step of grouped-query attention over a paged
 * key/value cache: for each request b and query head h,
 *     o[b,h] = sum_{t < len_b} p_t v_t,  p = softmax over t of q[b,h] . k_t / sqrt(D),
 *     lse[b,h] = ln sum_{t < len_b} exp(q[b,h] . k_t / sqrt(D)),
 * where k_t, v_t are the cached key and value of logical token t of request b
 * for K/V head floor(h / (Hq / Hkv)).  Definition and layout: "CUDA KV Cache:
 * paged storage and long-context decode" (chengzipai.xyz), section 2 (cache
 * [P][2][T][Hkv][D]; logical token t lives in physical page
 * block_table[b][t / T] at offset t mod T), section 3 (the query head group
 * shares its K/V head; the translation happens inside the kernel, nothing is
 * gathered or copied) and section 5 (online softmax over the tokens).  The
 * query is the request's newest token, so every cached token is visible.
 *
 *   q            [B, Hq, D] of `dtype`, 16-byte aligned.
 *   cache        [P, 2, T, Hkv, D] of `dtype`, 16-byte aligned: page p, K (0)
 *                or V (1), token slot, K/V head, dim; element
 *                (((p*2 + kind)*T + slot)*Hkv + head)*D + d.
 *   block_table  [B, max_pages] int32 (device), 4-byte aligned: entry
 *                (b, i) is the physical page of request b's logical page i.
 *                Only the pages holding tokens < len_b are read; each must
 *                be in [0, P).
 *   lengths      [B] int32 (device), 4-byte aligned: tokens of request b,
 *                1 <= len_b <= max_pages * T.
 *   o            [B, Hq, D] FP32 output, 16-byte aligned.
 *   lse          [B, Hq] FP32 output (natural log), 4-byte aligned.
 *   B, Hq, Hkv   requests, query heads, K/V heads: Hq % Hkv == 0 (else
 *                ATTN_ERR_SHAPE) and Hq / Hkv <= 32 (else ATTN_ERR_UNSUPPORTED).
 *   D            64 or 128 (else ATTN_ERR_UNSUPPORTED).
 *   page_size    T, a power of two up to 65536 (else ATTN_ERR_UNSUPPORTED).
 *   num_pages    P, pages in the cache.   max_pages  columns of block_table.
 *   dtype        ATTN_F16 or ATTN_BF16 (q and cache).
 *   num_splits   0: the library chooses; 1..PAGED_MAX_SPLITS: split each
 *                request's token range [0, max_pages*T) into about that many
 *                segments (KV page, section 6.4), merged as in
 *                attn_fwd_splitkv.  A segment holds at most 2048 tokens, so
 *                long ranges may get more.  Other values: ATTN_ERR_SHAPE.
 *   workspace, workspace_bytes  as for attn_fwd_splitkv, sized by
 *                paged_decode_workspace(...); NULL allowed when that is 0.
 *   stream       HIP stream to enqueue on.
 *
 * lengths and block_table are device data, which the call does not read:
 * a request whose length is out of range, or which uses a page id out of
 * range, gets NaN in all of its o and lse entries (no out-of-range address is
 * read).  Limits: P*2*T*Hkv*D < 2^62, P < 2^31, max_pages*T < 2^31,
 * B*max_pages < 2^31, B*Hq < 2^31, and B*Hkv times the number of segments
 * below 2^31 (the workgroup count); other sizes ATTN_ERR_SHAPE.
 * o, lse and the workspace must not overlap the inputs or each other.
 */
attn_status_t paged_decode(const void *q, const void *cache, const int32_t *block_table,
                           const int32_t *lengths, float *o, float *lse, int64_t B, int64_t Hq,
                           int64_t Hkv, int64_t D, int64_t page_size, int64_t num_pages,
                           int64_t max_pages, attn_dtype_t dtype, int num_splits, void *workspace,
                           int64_t workspace_bytes, hipStream_t stream);

/*
 * paged_decode_workspace - bytes of workspace paged_decode needs for these
 * sizes (0 if it uses one segment), or -1 if they are invalid.  Pure host
 * computation; enqueues nothing.
 */
int64_t paged_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                               int64_t max_pages, int num_splits);

/* Bytes of the fixed segment-state array of paged_decode_noalloc (32 MiB). */
#define PAGED_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)

/*
 * paged_decode_noalloc - paged_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same call without a workspace argument.  The
 * segment states go to a fixed array of PAGED_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on every device it runs on until the process ends.
 * The call itself allocates nothing (no hipMalloc, no hipFree); its first
 * call on a device looks up that device's array address (hipGetSymbolAddress)
 * with the device current and keeps it.
 *
 *   Arguments, layouts, errors and results as for paged_decode, which it
 *   matches bit for bit.  The stream must belong to the current device.
 *   paged_decode_workspace(...) above PAGED_NOALLOC_SCRATCH_BYTES:
 *   ATTN_ERR_WORKSPACE (pass a smaller num_splits or use paged_decode).
 *   The address lookup failing: ATTN_ERR_LAUNCH.
 *
 * All calls on one device share its array, and each segment's state is
 * written before it is read, so nothing carries over from one call to the
 * next.  Calls whose kernels may overlap on one device (different streams
 * without ordering between them) race on the array: order them.
 */
attn_status_t paged_decode_noalloc(const void *q, const void *cache, const int32_t *block_table,
                                   const int32_t *lengths, float *o, float *lse, int64_t B,
                                   int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                                   int64_t num_pages, int64_t max_pages, attn_dtype_t dtype,
                                   int num_splits, hipStream_t stream);

/*
 * attn_bwd - gradients of the attention forward (attn_fwd) with respect to
 * q, k and v, for an upstream gradient dout = dL/dO.
 *
 * The pages define only the forward; the FA page (section 7) keeps the
 * log-sum-exp so that a backward pass can rebuild the softmax weights without
 * storing them.  This call does that: with s_ij = q_i . k_j / sqrt(D) over
 * the visible keys and p_ij = exp(s_ij - lse_i),
 *     dV_j = sum_i p_ij dO_i,
 *     dP_ij = dO_i . v_j,   Delta_i = dO_i . O_i,   dS_ij = p_ij (dP_ij - Delta_i),
 *     dQ_i = sum_j dS_ij k_j / sqrt(D),   dK_j = sum_i dS_ij q_i / sqrt(D),
 * which is the derivative of the section 1 definition (Delta_i equals
 * sum_j p_ij dP_ij because each softmax row sums to one).  Every output
 * element is written by one workgroup in a fixed order: no atomics, and the
 * result is bit-for-bit repeatable.
 *
 *   q, k, v  [B, H, N, D] of `dtype`, 16-byte aligned: the forward's inputs.
 *   o        [B, H, N, D] FP32, 16-byte aligned: attn_fwd's output for them.
 *   lse      [B, H, N] FP32, 4-byte aligned: attn_fwd's log-sum-exp.
 *   dout     [B, H, N, D] of `dtype`, 16-byte aligned: dL/dO.
 *   dq, dk, dv  [B, H, N, D] FP32 outputs, 16-byte aligned.
 *   B, H, N, D, causal, dtype  as for attn_fwd (D 64 or 128; K/V heads
 *            equal to query heads).
 *   workspace  device buffer owned by the caller, 16-byte aligned, of at
 *            least attn_bwd_workspace(B, H, N) bytes (8 per row): it receives
 *            Delta and lse in base 2 before the gradient kernels read them.
 *            Its contents on entry do not matter and are undefined after the
 *            call.  Two calls that run at the same time need separate ones.
 *   workspace_bytes  size of `workspace`; too small: ATTN_ERR_WORKSPACE.
 *   stream   HIP stream to enqueue on (three kernels, in order).
 *
 * Errors: NULL pointer ATTN_ERR_NULL, sizes and limits as for attn_fwd,
 * alignment ATTN_ERR_ALIGN; dq, dk, dv and the workspace must not overlap
 * any input or each other (ATTN_ERR_ALIAS).  o and lse are used as given: a
 * pair that does not come from attn_fwd on the same q, k, v gives gradients
 * of nothing in particular, without an error.
 */
attn_status_t attn_bwd(const void *q, const void *k, const void *v, const float *o,
                       const float *lse, const void *dout, float *dq, float *dk, float *dv,
                       int64_t B, int64_t H, int64_t N, int64_t D, int causal, attn_dtype_t dtype,
                       void *workspace, int64_t workspace_bytes, hipStream_t stream);

/*
 * attn_bwd_gqa - attn_bwd for attn_fwd_gqa: Hkv key/value heads shared by
 * groups of g = H / Hkv query heads.
 *
 * Query head h of batch b reads K/V head floor(h / g) of the same batch
 * ("CUDA KV Cache: paged storage and long-context decode" (chengzipai.xyz),
 * section 3), so by the chain rule dQ of head h is the attn_bwd formula
 * against that K/V head, and dK, dV of a K/V head are the sums over its
 * group of the formula's per-head dK, dV.  The sum is accumulated inside one
 * workgroup per key tile (no atomics; bit-for-bit repeatable).
 *
 *   q, o, dout, dq  [B, H, N, D];  lse [B, H, N]  (as for attn_bwd).
 *   k, v     [B, Hkv, N, D] of `dtype`, 16-byte aligned: attn_fwd_gqa's K, V.
 *   dk, dv   [B, Hkv, N, D] FP32 outputs, 16-byte aligned.
 *   Hkv      1 <= Hkv <= H and H % Hkv == 0, else ATTN_ERR_SHAPE.
 *   workspace  at least attn_bwd_workspace(B, H, N) bytes (per query row).
 * Everything else (D, dtype, causal, limits, errors, stream) is as for
 * attn_bwd; attn_bwd is this call with Hkv = H.
 */
attn_status_t attn_bwd_gqa(const void *q, const void *k, const void *v, const float *o,
                           const float *lse, const void *dout, float *dq, float *dk, float *dv,
                           int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal,
                           attn_dtype_t dtype, void *workspace, int64_t workspace_bytes,
                           hipStream_t stream);

/*
 * attn_bwd_workspace - bytes of workspace attn_bwd and attn_bwd_gqa need
 * (8 * B*H*N, H the query heads), or -1 if the sizes are invalid.  Pure host
 * computation; enqueues nothing.
 */
int64_t attn_bwd_workspace(int64_t B, int64_t H, int64_t N);

/*
 * row_softmax - y[r, :] = softmax(x[r, :]) for r < M.
 *
 *   x   [M, N] FP32 input, row-major, 4-byte aligned (rows need not be
 *       16-byte aligned; misaligned row starts are handled inside).
 *   y   [M, N] FP32 output, same layout; must not overlap x.
 *   M   number of rows, 1 <= M < 2^31;  N  row length, 1 <= N < 2^31;
 *       M*N < 2^62.
 *   stream  HIP stream to enqueue on.
 *
 * Errors: x or y NULL ATTN_ERR_NULL; a size outside the limits above
 * ATTN_ERR_SHAPE; x or y not 4-byte aligned ATTN_ERR_ALIGN; x and y
 * overlapping ATTN_ERR_ALIAS.  Nothing is enqueued on an error.
 */
attn_status_t row_softmax(const float *x, float *y, int64_t M, int64_t N, hipStream_t stream);

/* Static English text for a status code (never NULL). */
const char *attn_status_str(attn_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* OSC_ATTN_H */
