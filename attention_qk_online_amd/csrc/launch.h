// Internal host-side interface between the C ABI (api.cpp) and the kernel
// translation units.  Each launcher enqueues exactly one kernel on `stream`
// and returns the launch status; argument checks happen before, in api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct DecodeParams {
  const void* q;           // [B, Hq, D]
  const void* k_pages;     // [num_pages, P, Hkv, D]
  const void* v_pages;
  const int32_t* page_table;  // [B, max_pages]
  const int32_t* kv_lens;     // [B]
  void* out;               // [B, Hq, D]
  float* lse;              // [B, Hq]
  float* part_o;           // workspace: partial outputs (layout per kernel below)
  float* part_lse;         // workspace: partial log-sum-exp
  // workspace (bf16 balanced schedule): [B + 1] first unit of each request
  // in the batch's unit order, then the total; written by workgroup 0 of the
  // main kernel, read by the merge kernel.
  int32_t* unit_start;
  int B, Hq, Hkv, num_pages, max_pages, max_kv_len, split_pages;
  // Pages hold 16 << page_shift tokens (16-bit path; the fp32 path takes 16
  // only).  The kernels work in 16-token blocks: block k of a request is
  // block k & ((1 << page_shift) - 1) of page table[k >> page_shift].
  int page_shift;
  int max_tokens;          // max_pages * page size, capped at INT_MAX (table capacity)
  // fp32 split grid: n_splits splits of split_pages pages per request,
  //   part_o [B, n_splits, Hq, D], part_lse [B, n_splits, Hq].
  int n_splits;
  // bf16 balanced schedule: KV heads form nhg groups of hw heads (one wave
  //   each); the (request, head group, page) units are cut into equal runs,
  //   one per workgroup (n_groups in the grid, looping when runs outnumber
  //   them); a run has split_pages units when split_pages > 0, else
  //   max(min_run, ceil(units / n_groups)).  A (request, head group) pair
  //   spans at most max_segs runs;
  //   part_o [B, Hkv, max_segs, G, D], part_lse [B, Hkv, max_segs, G].
  int hw, nhg, n_groups, min_run, max_segs;
  float scale_log2;        // softmax scale * log2(e) (E4M3 cache: times the key scale)
  float v_scale;           // E4M3 cache only: scale of the values
  // Page layout: 0 = NHD [page, slot, kv head, d], 1 = HND [page, kv head, slot, d].
  int kv_hnd;
  // Sliding window: the query (the last token) sees keys kv_len-1-window_left
  // .. kv_len-1; -1 = every key.
  int window_left;
  // Rotary position embedding applied in the kernel to q (position kv_len-1)
  // and to each key (its token index): pairs (d, d + D/2) turned by the angle
  // position * rope_inv_scale * 2^(-2 d / D * log2(theta)).
  float rope_log2_theta, rope_inv_scale;
};

struct PrefillParams {
  const void* q;           // [total_q, Hq, D]
  const void* k;           // contiguous: [total_k, Hkv, D]; paged: pool [num_pages, P, Hkv, D]
  const void* v;
  const int32_t* cu_q;     // [B+1]
  const int32_t* cu_k;     // [B+1] (contiguous only)
  const int32_t* page_table;  // [B, max_pages] (paged only)
  const int32_t* kv_lens;     // [B]            (paged only)
  void* out;               // [total_q, Hq, D]
  float* lse;              // [total_q, Hq]
  int B, Hq, Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k;
  int num_pages, max_pages;
  int causal;
  int q_tiles;             // ceil(max_seqlen_q / BM)
  // Paged only.  Request b's keys start at column kv_offset / 16 of row b
  // (row stride table_stride) and number kv_lens[b] - kv_offset; with
  // kv_offset > 0 and causal, a request with fewer keys than queries is
  // invalid (its rows become NaN).  When kv_len_fixed >= 0 the launch is
  // instead one sequence of all total_q query rows attending to the first
  // kv_len_fixed keys of page-table row 0 (cu_q, kv_lens unused).
  int table_stride, kv_offset, kv_len_fixed;
  // When merge_lse is set, the state (merge_o, merge_lse) -- laid out like
  // out / lse -- is merged into each written row before it is stored.
  const void* merge_o;
  const float* merge_lse;
  // Paged only: page layout, 0 = NHD, 1 = HND (as DecodeParams::kv_hnd).
  int kv_hnd;
  // Sliding window: query i sees only keys >= i + (Lk - Lq) - window_left
  // (bottom-right aligned like the causal mask); -1 = no window.
  int window_left;
  // Right side of the window: query i sees only keys <= i + (Lk - Lq) +
  // window_right; -1 = no bound.  causal is the right window 0 and takes
  // precedence.
  int window_right;
  // Paged only: pages hold 16 << page_shift tokens; max_tokens = max_pages *
  // page size (capped at INT_MAX), the capacity of a page-table row.
  int page_shift, max_tokens;
  float scale_log2;
};

// dtype: 0 = f32, 1 = bf16, 2 = f16 (values of attn_dtype).
bool decode_supported(int dtype, int D, int G, int page_size);
// fp8_kv: K/V pages are E4M3 bytes (16-bit dtype only); rope: rotary
// embedding of q and k in the kernel (16-bit dtype, D 64 or 128, not fp8_kv).
hipError_t launch_decode_split(const DecodeParams& p, int dtype, int D, int G, bool fp8_kv,
                               bool rope, hipStream_t s);
hipError_t launch_decode_combine(const DecodeParams& p, int dtype, int D, int G, hipStream_t s);
// Device address of the file-scope decode scratch array (partial states of
// the allocation-free decode entry point) on the current device, taken once
// per device with hipGetSymbolAddress; *bytes receives its size.
hipError_t decode_scratch(void** ptr, size_t* bytes);
// Workgroups (of up to 8 waves, one per KV head) per CU in the balanced bf16 grid.
#ifndef ATTN_DECODE_GROUPS_PER_CU
#define ATTN_DECODE_GROUPS_PER_CU 1
#endif
constexpr int kDecodeGroupsPerCU = ATTN_DECODE_GROUPS_PER_CU;

// Log-sum-exp merge of two states over `rows` (token, head) rows of D elements;
// out / lse may alias the b side (each element is read before it is written
// by the same thread).
bool merge_supported(int dtype, int D);
hipError_t launch_merge_states(const void* oa, const float* la, const void* ob, const float* lb,
                               void* out, float* lse, long rows, int dtype, int D, hipStream_t s);

// Query rows per workgroup of the prefill kernels (grid sizing on the host).
constexpr int kPrefillBM = 128;
bool prefill_supported(int dtype, int D);
// head_dim 256 on four pairs of waves, 32 rows a pair (prefill256.hip).
hipError_t launch_prefill_d256(const PrefillParams& p, int dtype, bool paged, hipStream_t s);
hipError_t launch_prefill(const PrefillParams& p, int dtype, int D, bool paged, hipStream_t s);

}  // namespace attn
