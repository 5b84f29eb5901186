/*
 * attn.h -- C ABI of the fused attention forward for AMD MI355X (gfx950).
 *
 * One pass computes, per query row and query head,
 *
 *     s_j   = scale * <q, k_j>            over the visible keys j
 *     lse   = log(sum_j exp(s_j))          (natural log, fp32)
 *     out   = sum_j exp(s_j - lse) * v_j
 *
 * without writing the score matrix to memory: scores live in registers and an
 * online softmax (running maximum and running sum, rescaled whenever the
 * maximum grows) folds each block of keys into the output.  This is the
 * fused scheme of "FlashAttention-3 内核在最新大模型推理中的集成实践"
 * (section 一: tiles in on-chip memory, online softmax accumulated in place;
 * section 四: the rescaling must never be dropped) and of "FlashInfer
 * Attention Kernel技术解析" (section 1.3: QK^T, softmax with wave-level
 * reductions, and PV as one pipeline).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensors are dense, row-major, and live in device memory unless the
 *    argument says "host".  q, k, v (or the page pools), out and the
 *    workspaces start at 16-byte aligned addresses (ATTN_E_UNSUPPORTED
 *    otherwise; every device allocation is).  Element types: ATTN_F32
 *    (float), ATTN_BF16 (bfloat16 bits) or ATTN_F16 (IEEE half bits).  `out`
 *    has the input element type; `lse` is float.
 *  - Grouped heads: query head h reads KV head h / (Hq / Hkv); Hq must be a
 *    multiple of Hkv ("FlashAttention-3 ..." section 二: queries carry
 *    num_heads, keys/values num_kv_heads).
 *  - Causal masking is aligned to the bottom right: query i of a sequence with
 *    Lq queries and Lk keys sees key j iff j <= i + (Lk - Lq).  A query row
 *    that sees no key gets out = 0 and lse = -inf.
 *  - Paged KV pools use the NHD layout [num_pages, page_size, Hkv, D]
 *    ("FlashInfer内核库深度解析", KV-cache layout: NHD suits multi-head
 *    parallelism); logical token t of request b is at
 *    pool[page_table[b * max_pages_per_req + t / page_size]][t % page_size].
 *    Table entries past ceil(kv_len / page_size) are never read.
 *  - Ownership: the caller owns every buffer.  These entry points allocate no
 *    device memory, keep no state between calls (apart from the optional
 *    timing facility below), enqueue all work asynchronously on `stream`
 *    (a hipStream_t; NULL means the default stream) and never synchronise
 *    the device.  Host arrays are read only during the call.  `out`, `lse`
 *    and `workspace` must not alias any input.
 *  - Errors: every argument check runs before anything is enqueued; a
 *    failing call returns a status, writes nothing and launches nothing.
 *    attn_last_error() then describes the failure (thread-local text).
 *    Device-resident index data (page tables, lengths, cu_seqlens) cannot be
 *    checked on the host without a sync, so the kernels clamp it instead:
 *    every memory access stays inside the sizes passed here, and output
 *    computed from inconsistent device data is NaN.  Decode: a request with
 *    a page id outside [0, num_pages) or a kv_len above max_kv_len or
 *    max_pages_per_req * page_size gets NaN in all its out and lse rows.
 *    Prefill: rows whose visible keys reach an out-of-range page id, and the
 *    rows of a sequence longer than max_seqlen_q, with more keys than
 *    max_seqlen_k (paged: a kv_len above max_kv_len or max_pages_per_req *
 *    page_size), are NaN; of such a sequence only its first
 *    ceil(max_seqlen_q / 128) * 128 rows are written, and a key count above
 *    its bound makes the kernel read none of its keys.
 *  - Empty caches: when nothing can be read (prefill total_k 0; decode and
 *    paged prefill max_kv_len 0) the key/value tensors and the page table
 *    may be NULL.
 *  - Size limits: every token count and length argument (total_q, total_k,
 *    max_seqlen_q, max_seqlen_k, max_kv_len) is at most ATTN_MAX_TOKENS
 *    (2^30), and a 16-bit decode batch keeps B * (ceil(max_kv_len / 16) + 1)
 *    * ceil(Hkv / 8) at most ATTN_MAX_TOKENS; larger values return
 *    ATTN_E_UNSUPPORTED.  Within these limits every index sum on the host and
 *    in the kernels fits a 32-bit int.  A workspace size that does not fit a
 *    size_t is returned as SIZE_MAX by the size queries and rejected with
 *    ATTN_E_SHAPE by the calls.
 */
#ifndef ATTN_H
#define ATTN_H

#include <limits.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_E_NULL = 1,        /* a required pointer is NULL                          */
  ATTN_E_SHAPE = 2,       /* a size is negative or sizes are inconsistent         */
  ATTN_E_DTYPE = 3,       /* unknown element type                                 */
  ATTN_E_UNSUPPORTED = 4, /* valid request that this build has no kernel for     */
  ATTN_E_VALUE = 5,       /* a non-finite scale                                   */
  ATTN_E_WORKSPACE = 6,   /* workspace missing or smaller than the size query     */
  ATTN_E_HIP = 7,         /* the HIP runtime rejected a launch                    */
  /* range markers, never returned: any int passed to attn_status_string is
   * a value of the type */
  ATTN_STATUS_RANGE_MIN_ = INT_MIN,
  ATTN_STATUS_RANGE_MAX_ = INT_MAX
} attn_status;

/* The two range markers are not element types: they make every int a value
 * of the enumeration, so that an out-of-range dtype from a caller is a
 * defined value that the entry points reject with ATTN_E_DTYPE. */
typedef enum {
  ATTN_F32 = 0,
  ATTN_BF16 = 1,
  ATTN_F16 = 2,
  ATTN_DTYPE_RANGE_MIN_ = INT_MIN,
  ATTN_DTYPE_RANGE_MAX_ = INT_MAX
} attn_dtype;

#define ATTN_MAX_TOKENS (1 << 30)

/* ------------------------------------------------------------------------ */
/* Batched decode over a paged KV cache.
 *
 * One query token per request attends to that request's kv_len cached tokens
 * (no mask).  The G = Hq/Hkv query heads that share a KV head are processed
 * together, so every K/V byte is read from HBM once.  Pages, page tables and
 * per-request lengths follow "FlashInfer内核库深度解析" (PageAttention:
 * fixed-size pages addressed through a table) and "FlashAttention-3 ..."
 * section 二 (physical block addressing in continuous batching).
 *
 * bf16 / f16: the (request, KV head, page) units of the batch are cut into equal
 * runs, one per wave, computed on the device from kv_lens (balanced over
 * ragged lengths); Q.K^T and P.V run on the matrix cores.  Runs that cover
 * only part of a (request, KV head) pair leave partial (o, lse) states in the
 * workspace, merged by their log-sum-exp in a second kernel.  split_pages,
 * when > 0, fixes the run length (in pages); 0 lets the library choose.
 * fp32: each request is cut into splits of split_pages pages (0: default);
 * one work item per (request, KV head, split), merged the same way.
 *
 *  q           [B, Hq, D]                   dtype
 *  k_pages     [num_pages, page_size, Hkv, D] dtype
 *  v_pages     [num_pages, page_size, Hkv, D] dtype
 *  page_table  [B, max_pages_per_req]       int32
 *  kv_lens     [B]                          int32, 0 <= kv_len <= max_kv_len
 *  max_kv_len  host int: an upper bound of every kv_len (sizes the plan)
 *  split_pages host int: run / split length in pages (BF16/F16: in 16-token
 *              blocks); 0 picks a default
 *  scale       finite float (the caller's softmax scale, usually 1/sqrt(D))
 *  out         [B, Hq, D]                   dtype
 *  lse         [B, Hq]                      float
 *  workspace   device scratch of at least attn_decode_paged_workspace_size()
 *              bytes, 16-byte aligned (else ATTN_E_UNSUPPORTED; may be NULL
 *              when that size is 0); contents on entry do not matter and are
 *              clobbered.
 *
 * Supported: dtype BF16 or F16 with D in {64, 128, 256}, or F32 with D in {64, 128};
 * Hq/Hkv in {1, 2, 4, 8}; page_size 16, 32, 64, 128 or 256 (BF16/F16; the
 * kernel walks 16-token blocks, so a cache gives the same result bit for bit
 * whatever its page size) or 16 (F32).  Anything else returns
 * ATTN_E_UNSUPPORTED.  The workspace size depends on dtype, the sizes and
 * split_pages only (not on the device or on kv_lens).
 */
size_t attn_decode_paged_workspace_size(attn_dtype dtype, int B, int Hq, int Hkv, int D,
                                        int page_size, int max_kv_len, int split_pages);

attn_status attn_decode_paged(attn_dtype dtype, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* page_table,
                              const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                              int page_size, int num_pages, int max_pages_per_req,
                              int max_kv_len, int split_pages, float scale, void* out,
                              float* lse, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ------------------------------------------------------------------------ */
/* attn_decode_paged for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, results, supported shapes and NaN rules are those of
 * attn_decode_paged (NHD pages) without the workspace: the partial states go
 * to a static device array of ATTN_DECODE_NOALLOC_SCRATCH_BYTES owned by the
 * library, one per GPU, held until the process ends.  The call allocates
 * nothing (no hipMalloc / hipFree, no allocating library routine).
 *
 *  - A call whose attn_decode_paged_workspace_size(dtype, ...) exceeds
 *    ATTN_DECODE_NOALLOC_SCRATCH_BYTES returns ATTN_E_WORKSPACE and launches
 *    nothing (use attn_decode_paged with a workspace then).  The bf16 decode
 *    of 64 requests of up to 4096 tokens, Hq 32, Hkv 8, D 128 needs ~35 MB.
 *  - Every call on one GPU uses that GPU's array: calls that overlap on one
 *    GPU (other streams, other threads, concurrent graph replays) race and
 *    give undefined results.  Calls ordered on one stream do not.
 *  - The array's contents on entry do not matter; they keep the last call's
 *    partial states.
 *  - The first call on a device looks up the array's device address
 *    (hipGetSymbolAddress); a failure there returns ATTN_E_HIP.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)
attn_status attn_decode_paged_noalloc(attn_dtype dtype, const void* q, const void* k_pages,
                                      const void* v_pages, const int32_t* page_table,
                                      const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                      int page_size, int num_pages, int max_pages_per_req,
                                      int max_kv_len, int split_pages, float scale, void* out,
                                      float* lse, void* stream);

/* ------------------------------------------------------------------------ */
/* Batched decode over a paged KV cache stored as 8-bit floats E4M3 (FP8 of
 * "FlashInfer内核库深度解析", precision support), one scale per tensor:
 * token t's key is k_scale * E4M3(k byte), its value v_scale * E4M3(v byte).
 * The key scale is folded into the softmax exponent's scale and the value
 * scale into the output normalisation ("FlashAttention-3 ..." section 一), so
 * the result equals attn_decode_paged on the dequantised cache up to
 * rounding, while half the K/V bytes are read.
 *
 *  dtype       type of q and out: ATTN_BF16 or ATTN_F16 (ATTN_F32 ->
 *              ATTN_E_UNSUPPORTED); the E4M3 bytes are converted to it
 *              exactly before the matrix-core products
 *  k_pages, v_pages  [num_pages, page_size, Hkv, D] uint8 (E4M3 bytes;
 *              0x7F / 0xFF are NaN)
 *  k_scale, v_scale  finite floats (else ATTN_E_VALUE)
 *  workspace   attn_decode_paged_workspace_size(dtype, ...) bytes, as for
 *              attn_decode_paged with the same dtype
 * Everything else, the supported shapes and the NaN rules are those of
 * attn_decode_paged with a 16-bit dtype.
 */
attn_status attn_decode_paged_fp8(attn_dtype dtype, const void* q, const void* k_pages,
                                  const void* v_pages, const int32_t* page_table,
                                  const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                  int page_size, int num_pages, int max_pages_per_req,
                                  int max_kv_len, int split_pages, float scale, float k_scale,
                                  float v_scale, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Ragged prefill addressed by cu_seqlens ("FlashAttention-3 ..." section 二:
 * packed [total_tokens, heads, head_dim] tensors, prefix offsets of length
 * batch+1, max_seqlen_q / max_seqlen_k, softmax_scale and causal).
 *
 *  q            [total_q, Hq, D]   bf16 or f16
 *  k, v         [total_k, Hkv, D]  same type
 *  cu_seqlens_q [B+1] int32, nondecreasing, cu[0] = 0, cu[B] <= total_q
 *  cu_seqlens_k [B+1] int32, same rules against total_k
 *  max_seqlen_q, max_seqlen_k  host ints bounding every per-sequence length
 *  causal       0 or 1 (bottom-right aligned)
 *  out          [total_q, Hq, D] same type;  lse [total_q, Hq] float
 *
 * Query tiles of 128 rows run on bf16 / f16 MFMA with fp32 accumulation; K/V
 * tiles are staged through LDS; tiles wholly above the causal diagonal are
 * never loaded.  Supported: dtype BF16 or F16; D in {128, 256}; any Hq
 * multiple of Hkv;
 * Hq * B * ceil(max_seqlen_q / 128) below 2^31 - 8 (else ATTN_E_SHAPE).
 * Rows of out/lse outside every [cu_seqlens_q[b], cu_seqlens_q[b+1]) are
 * not written.
 */
attn_status attn_prefill_varlen(attn_dtype dtype, const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int B, int Hq, int Hkv, int D, int total_q, int total_k,
                                int max_seqlen_q, int max_seqlen_k, int causal, float scale,
                                void* out, float* lse, void* stream);

/* ------------------------------------------------------------------------ */
/* Chunked prefill over a paged KV cache ("FlashAttention-3 ..." section 二:
 * chunked prefill and PagedAttention block addressing).  Request b's
 * queries are the last Lq_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] of its
 * kv_lens[b] cached tokens (their own K/V already written to the cache), so
 * the causal mask is bottom-right aligned.  Pages may be shared between
 * requests (a common prefix).
 *
 *  q            [total_q, Hq, D] bf16 or f16;   cu_seqlens_q [B+1] int32
 *  k_pages, v_pages [num_pages, page_size, Hkv, D] same type
 *  page_table   [B, max_pages_per_req] int32;  kv_lens [B] int32
 *  max_seqlen_q, max_kv_len  host bounds
 *  out [total_q, Hq, D] same type;  lse [total_q, Hq] float
 *
 * Supported: dtype BF16 or F16; D in {128, 256}; page_size 16, 32, 64, 128 or
 * 256 (the same cache gives the same result bit for bit whatever its page
 * size); the same work-item bound as attn_prefill_varlen.
 */
attn_status attn_prefill_paged(attn_dtype dtype, const void* q, const int32_t* cu_seqlens_q,
                               const void* k_pages, const void* v_pages,
                               const int32_t* page_table, const int32_t* kv_lens, int B, int Hq,
                               int Hkv, int D, int total_q, int page_size, int num_pages,
                               int max_pages_per_req, int max_seqlen_q, int max_kv_len,
                               int causal, float scale, void* out, float* lse, void* stream);

/* ------------------------------------------------------------------------ */
/* Chunked prefill over a paged KV cache whose first shared_prefix_len tokens
 * are the same pages for every request (shared-prefix reuse of the batch
 * processing layer in "FlashInfer内核库深度解析"), computed as a cascade:
 *   1. every query row of every request attends, without a mask, to the
 *      shared prefix, read through the first shared_prefix_len / 16 entries
 *      of page_table row 0 -- one pass over the prefix K/V for the whole
 *      batch instead of one per request;
 *   2. each request's rows attend to its own keys after the prefix (causal
 *      or not, as in attn_prefill_paged) and, before being stored, are
 *      merged with the result of pass 1 by the log-sum-exp rule of the
 *      online softmax ("FlashAttention-3 ..." section 一).
 * The result is that of attn_prefill_paged with the same arguments, up to
 * rounding, provided that:
 *   - every row of page_table starts with the same shared_prefix_len / 16
 *     page ids (row 0's are the ones read);
 *   - shared_prefix_len is a multiple of page_size and at most max_kv_len;
 *   - kv_lens[b] >= shared_prefix_len, and with causal also
 *     kv_lens[b] - shared_prefix_len >= Lq_b, i.e. every query of request b
 *     sees the whole prefix.  Rows of a request that breaks this are NaN.
 * shared_prefix_len = 0 is exactly attn_prefill_paged (no workspace used).
 *
 *  workspace  device memory of at least
 *             attn_prefill_paged_cascade_workspace_size(dtype, total_q, Hq, D)
 *             bytes, 256-byte aligned, owned by the caller; it holds the
 *             pass-1 state (a [total_q, Hq, D] array of the input type and a
 *             [total_q, Hq] float array); contents on entry do not matter.
 *             Two calls sharing a workspace must not overlap.
 * Other arguments, supported shapes and NaN rules as attn_prefill_paged;
 * pass 1 also needs Hq * ceil(total_q / 128) below 2^31 - 8 (ATTN_E_SHAPE).
 */
size_t attn_prefill_paged_cascade_workspace_size(attn_dtype dtype, int total_q, int Hq, int D);
attn_status attn_prefill_paged_cascade(attn_dtype dtype, const void* q,
                                       const int32_t* cu_seqlens_q, const void* k_pages,
                                       const void* v_pages, const int32_t* page_table,
                                       const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                       int total_q, int page_size, int num_pages,
                                       int max_pages_per_req, int max_seqlen_q, int max_kv_len,
                                       int shared_prefix_len, int causal, float scale, void* out,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* ------------------------------------------------------------------------ */
/* Merge of two attention states over disjoint key sets of the same query
 * rows: the aggregation step of the online softmax ("FlashAttention-3 ..."
 * section 一) applied to finished partial results.  A state is (o, lse): o
 * normalised over its keys, lse the natural log of its normaliser.  With
 * mx = max(lse_a, lse_b) and w = exp(lse - mx) per side,
 *   out = (w_a o_a + w_b o_b) / (w_a + w_b),  lse_out = mx + log(w_a + w_b).
 * An empty side (lse = -inf) has weight 0 and its o is not read; both empty
 * gives out = 0, lse_out = -inf; a NaN lse on either side gives NaN.
 *
 *  o_a, o_b, out       [rows, D] of dtype (F32, BF16 or F16), 16-byte aligned
 *  lse_a, lse_b, lse_out  [rows] float
 *  rows  number of (token, head) pairs;  D in {64, 128, 256}
 * out may be o_a or o_b and lse_out may be lse_a or lse_b (in place); other
 * overlaps are not allowed.  fp32 arithmetic, one rounding to dtype.
 */
attn_status attn_merge_states(attn_dtype dtype, const void* o_a, const float* lse_a,
                              const void* o_b, const float* lse_b, int rows, int D, void* out,
                              float* lse_out, void* stream);

/* ------------------------------------------------------------------------ */
/* Batched decode with a sliding window: the query (the request's last token)
 * sees only keys kv_len-1-window_left .. kv_len-1 (window_left = -1: all,
 * i.e. attn_decode_paged; other negative values return ATTN_E_VALUE).  With
 * a 16-bit dtype the pages before the window are never read; with F32 their
 * keys are masked.  kv_layout: 0 NHD, 1 HND pages.  Everything else, the
 * workspace included, as attn_decode_paged.
 */
attn_status attn_decode_paged_window(attn_dtype dtype, int kv_layout, int window_left,
                                     const void* q, const void* k_pages, const void* v_pages,
                                     const int32_t* page_table, const int32_t* kv_lens, int B,
                                     int Hq, int Hkv, int D, int page_size, int num_pages,
                                     int max_pages_per_req, int max_kv_len, int split_pages,
                                     float scale, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Batched decode with the rotary position embedding applied in the kernel
 * (the dynamic RoPE of FlashInfer's single-request decode, "FlashInfer内核库
 * 深度解析", decode kernels), for caches that hold keys before rotation.
 * The query is at position kv_len - 1, key t at position t.  Each pair
 * (x_d, x_{d+D/2}), d < D/2, of q and of every key is turned by the angle
 *   position / rope_scale * rope_theta^(-2 d / D)
 * (x_d cos - x_{d+D/2} sin, x_{d+D/2} cos + x_d sin) -- the rotate-half
 * convention -- and rounded to the input type before the products.
 * rope_theta, rope_scale: finite and positive (else ATTN_E_VALUE).
 * Supported: BF16 / F16, D 64 or 128 (else ATTN_E_UNSUPPORTED); kv_layout,
 * window_left and everything else as attn_decode_paged_window.
 */
attn_status attn_decode_paged_rope(attn_dtype dtype, int kv_layout, int window_left,
                                   float rope_theta, float rope_scale, const void* q,
                                   const void* k_pages, const void* v_pages,
                                   const int32_t* page_table, const int32_t* kv_lens, int B, int Hq,
                                   int Hkv, int D, int page_size, int num_pages,
                                   int max_pages_per_req, int max_kv_len, int split_pages,
                                   float scale, void* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Decode over an E4M3 (fp8) cache with a sliding window: the window of
 * attn_decode_paged_window (the query sees keys kv_len-1-window_left ..
 * kv_len-1; window_left = -1: all, other negative values ATTN_E_VALUE; pages
 * before the window are never read) on the cache, scales and dtypes of
 * attn_decode_paged_fp8.  kv_layout: 0 NHD, 1 HND pages.
 */
attn_status attn_decode_paged_fp8_window(attn_dtype dtype, int kv_layout, int window_left,
                                         const void* q, const void* k_pages, const void* v_pages,
                                         const int32_t* page_table, const int32_t* kv_lens, int B,
                                         int Hq, int Hkv, int D, int page_size, int num_pages,
                                         int max_pages_per_req, int max_kv_len, int split_pages,
                                         float scale, float k_scale, float v_scale, void* out,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         void* stream);

/* ------------------------------------------------------------------------ */
/* Ragged and paged prefill with a sliding window (the window_size argument
 * of varlen_fwd in "FlashAttention-3 ..." section 二, a (left, right) pair):
 * query i of a sequence with Lq queries and Lk keys sees key j only if
 * j >= i + (Lk - Lq) - window_left and j <= i + (Lk - Lq) + window_right
 * (both aligned bottom-right like the causal mask).  -1 leaves that side
 * open (window_left = window_right = -1 are the calls above); other negative
 * values return ATTN_E_VALUE.  causal = 1 is the right window 0 and takes
 * precedence over window_right.  A window at least max_seqlen_q +
 * max_seqlen_k (paged: max_kv_len) wide bounds nothing.  Rows left with no
 * visible key get out = 0 and lse = -inf.  Whole key tiles outside a query
 * tile's windows are never loaded.  kv_layout: 0 NHD, 1 HND pages.
 * Everything else as attn_prefill_varlen / attn_prefill_paged.
 */
attn_status attn_prefill_varlen_window(attn_dtype dtype, const void* q, const void* k,
                                       const void* v, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_k, int B, int Hq, int Hkv, int D,
                                       int total_q, int total_k, int max_seqlen_q,
                                       int max_seqlen_k, int causal, int window_left,
                                       int window_right, float scale, void* out, float* lse,
                                       void* stream);
attn_status attn_prefill_paged_window(attn_dtype dtype, int kv_layout, const void* q,
                                      const int32_t* cu_seqlens_q, const void* k_pages,
                                      const void* v_pages, const int32_t* page_table,
                                      const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                      int total_q, int page_size, int num_pages,
                                      int max_pages_per_req, int max_seqlen_q, int max_kv_len,
                                      int causal, int window_left, int window_right,
                                      float scale, void* out, float* lse, void* stream);

/* ------------------------------------------------------------------------ */
/* The paged entry points above read NHD pages: [num_pages, page_size, Hkv, D],
 * the heads of one token adjacent.  Each has a twin for HND pages,
 * [num_pages, Hkv, page_size, D], where one head's page_size rows are
 * contiguous (the two layouts of "FlashInfer内核库深度解析", KV-cache
 * layout choice: NHD for many heads in parallel, HND for long,
 * bandwidth-bound sequences).  Arguments, results, workspace and errors are
 * those of the NHD call; only the order of the pool's middle dimensions
 * differs, so the same cache permuted gives the same result bit for bit.
 */
attn_status attn_decode_paged_hnd(attn_dtype dtype, const void* q, const void* k_pages,
                                  const void* v_pages, const int32_t* page_table,
                                  const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                  int page_size, int num_pages, int max_pages_per_req,
                                  int max_kv_len, int split_pages, float scale, void* out,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream);
attn_status attn_decode_paged_fp8_hnd(attn_dtype dtype, const void* q, const void* k_pages,
                                      const void* v_pages, const int32_t* page_table,
                                      const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                      int page_size, int num_pages, int max_pages_per_req,
                                      int max_kv_len, int split_pages, float scale,
                                      float k_scale, float v_scale, void* out, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream);
attn_status attn_prefill_paged_hnd(attn_dtype dtype, const void* q, const int32_t* cu_seqlens_q,
                                   const void* k_pages, const void* v_pages,
                                   const int32_t* page_table, const int32_t* kv_lens, int B,
                                   int Hq, int Hkv, int D, int total_q, int page_size,
                                   int num_pages, int max_pages_per_req, int max_seqlen_q,
                                   int max_kv_len, int causal, float scale, void* out,
                                   float* lse, void* stream);
attn_status attn_prefill_paged_cascade_hnd(attn_dtype dtype, const void* q,
                                           const int32_t* cu_seqlens_q, const void* k_pages,
                                           const void* v_pages, const int32_t* page_table,
                                           const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                           int total_q, int page_size, int num_pages,
                                           int max_pages_per_req, int max_seqlen_q,
                                           int max_kv_len, int shared_prefix_len, int causal,
                                           float scale, void* out, float* lse, void* workspace,
                                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Status text (static strings) and the detail of the calling thread's last
 * failing call (valid until that thread's next call into the library), after
 * the error table of "FlashInfer Attention Kernel技术解析" section 3.1 (each
 * failure named with its cause).  attn_last_hip_error() is the HIP runtime's
 * own text (hipGetErrorString and hipGetErrorName) for the error behind the
 * calling thread's last call when it returned ATTN_E_HIP, and "" when that
 * call returned anything else; attn_last_error() adds which launch failed. */
const char* attn_status_string(attn_status s);
const char* attn_last_error(void);
const char* attn_last_hip_error(void);

/* ------------------------------------------------------------------------ */
/* Optional kernel timing for benchmarks.  Between attn_timing_begin() and
 * attn_timing_end(), every kernel the library launches is bracketed by a
 * pair of hipEvents recorded on its launch stream.  attn_timing_end() waits
 * for those events and returns, per kernel kind, the summed milliseconds and
 * the number of launches.  Process-wide, not thread-safe; it creates HIP
 * events (no device memory).  At most `capacity` launches are recorded;
 * capacity must be 1 .. ATTN_TIMING_MAX_LAUNCHES (else ATTN_E_SHAPE). */
#define ATTN_TIMING_MAX_LAUNCHES (1 << 20)
typedef enum {
  ATTN_KERNEL_DECODE_SPLIT = 0,
  ATTN_KERNEL_DECODE_COMBINE = 1,
  ATTN_KERNEL_PREFILL = 2,
  ATTN_KERNEL_PREFILL_PAGED = 3,
  ATTN_KERNEL_MERGE = 4,
  ATTN_KERNEL_CASCADE_PREFIX = 5,
  ATTN_KERNEL_CASCADE_SUFFIX = 6,
  ATTN_KERNEL_KINDS = 7,
  /* range markers (not kinds), as for attn_dtype */
  ATTN_KERNEL_RANGE_MIN_ = INT_MIN,
  ATTN_KERNEL_RANGE_MAX_ = INT_MAX
} attn_kernel_kind;

attn_status attn_timing_begin(int capacity);
attn_status attn_timing_end(double* ms_per_kind, int* launches_per_kind);
const char* attn_kernel_name(attn_kernel_kind kind);

#ifdef __cplusplus
}
#endif
#endif /* ATTN_H */
