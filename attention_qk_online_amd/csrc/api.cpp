// C ABI entry points: argument checks, the split plan for decode, launches
// and the optional kernel-timing facility.  Declarations and the contract of
// every entry point are in include/attn.h.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <initializer_list>
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "launch.h"

namespace {

thread_local char g_last_error[512] = "";
// The HIP runtime's text for the error behind the calling thread's last
// ATTN_E_HIP (empty when its last call returned something else).
thread_local char g_last_hip_error[256] = "";

attn_status fail(attn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

attn_status fail_hip(hipError_t e, const char* what) {
  snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s (%s)", hipGetErrorString(e),
           hipGetErrorName(e));
  return fail(ATTN_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- timing ---
struct TimingRecord {
  hipEvent_t start, stop;
  int kind;
};
struct Timing {
  bool on = false;
  int capacity = 0;
  int used = 0;
  std::vector<TimingRecord> recs;
} g_timing;

// Launch `fn` (returns hipError_t) bracketed by timing events when enabled.
template <typename F>
hipError_t timed(int kind, hipStream_t s, F&& fn) {
  TimingRecord* rec = nullptr;
  if (g_timing.on && g_timing.used < g_timing.capacity) {
    rec = &g_timing.recs[g_timing.used++];
    rec->kind = kind;
    (void)hipEventRecord(rec->start, s);
  }
  hipError_t e = fn();
  if (rec) (void)hipEventRecord(rec->stop, s);
  return e;
}

// ------------------------------------------------------------ decode plan ---
// fp32 path.  Pages per split when the caller passes 0: aim for about
// kUnitsTarget work items over the whole batch (B * Hkv * splits of the
// longest request), with splits of at least kMinSplitPages pages -- two per
// wave of the split kernel's eight, one batch of loads -- so a short request
// is one work item (no combine) and partial states stay a small fraction of
// the KV bytes.
constexpr int kUnitsTarget = 2048;
constexpr int kMinSplitPages = 16;
// The decode kernel keeps one wave's page ids in a single VGPR: 64 per wave,
// 8 waves per workgroup.
constexpr int kMaxSplitPages = 512;

int auto_split_pages(int B, int Hkv, int max_pages) {
  if (max_pages <= 0) return kMinSplitPages;
  long pairs = (long)B * Hkv;
  long want = (kUnitsTarget + pairs - 1) / (pairs > 0 ? pairs : 1);
  if (want < 1) want = 1;
  long sp = (max_pages + want - 1) / want;
  if (sp < kMinSplitPages) sp = kMinSplitPages;
  return (int)sp;
}

struct DecodePlan {
  int split_pages, n_splits;   // fp32 split grid
  int min_run, max_segs;       // bf16 balanced runs
  size_t part_o_elems, part_lse_elems;
  size_t bytes;                // workspace bytes (0: none needed)
};

// Smallest run of the balanced bf16 schedule when the caller leaves the run
// length to the library: partial states stay well below the KV bytes.
constexpr int kMinRun = 8;

// Size arithmetic that saturates at SIZE_MAX instead of wrapping (a size
// query then reports SIZE_MAX and the call ATTN_E_SHAPE).
size_t mul_sat(size_t a, std::initializer_list<long long> xs) {
  size_t r = a;
  for (long long x : xs)
    if (r == SIZE_MAX || x < 0 || __builtin_mul_overflow(r, (size_t)x, &r)) return SIZE_MAX;
  return r;
}
size_t add_sat(size_t a, size_t b) {
  size_t r;
  return __builtin_add_overflow(a, b, &r) ? SIZE_MAX : r;
}
size_t round256(size_t bytes) { return bytes > SIZE_MAX - 255 ? SIZE_MAX : (bytes + 255) & ~(size_t)255; }
size_t aligned_bytes(size_t floats) {
  return floats > SIZE_MAX / sizeof(float) ? SIZE_MAX : round256(floats * sizeof(float));
}

// True when the product of the non-negative factors is at most `limit`.
bool product_at_most(std::initializer_list<long long> xs, long long limit) {
  long long r = 1;
  for (long long x : xs)
    if (x < 0 || __builtin_mul_overflow(r, x, &r) || r > limit) return false;
  return true;
}

DecodePlan plan_decode(int dtype, int B, int Hq, int Hkv, int D, int page_size, int max_kv_len,
                       int split_pages) {
  DecodePlan pl{};
  // Page and block counts of an int length fit an int.
  const int max_pages = page_size > 0 ? (int)(((long long)max_kv_len + page_size - 1) / page_size) : 0;
  if (dtype == ATTN_BF16 || dtype == ATTN_F16) {
    // The balanced schedule counts 16-token blocks, whatever the page size.
    const long long max_blocks = ((long long)max_kv_len + 15) / 16;
    // A (request, KV head) pair of at most max_blocks units spans at most
    // ceil(max_blocks / run) + 1 runs, and every run has >= min_run units.
    pl.split_pages = split_pages;
    pl.min_run = split_pages > 0 ? split_pages : kMinRun;
    pl.max_segs = (int)((max_blocks + pl.min_run - 1) / pl.min_run + 1);
    const size_t slots = mul_sat(1, {B, Hkv, pl.max_segs, Hq / (Hkv > 0 ? Hkv : 1)});
    pl.part_o_elems = mul_sat(slots, {D});
    pl.part_lse_elems = slots;
    // + the first unit of each request and the total (B + 1 int32)
    pl.bytes = add_sat(add_sat(aligned_bytes(pl.part_o_elems), aligned_bytes(pl.part_lse_elems)),
                       aligned_bytes((size_t)B + 1));
    return pl;
  }
  pl.split_pages = split_pages > 0 ? split_pages : auto_split_pages(B, Hkv, max_pages);
  if (pl.split_pages > kMaxSplitPages) pl.split_pages = kMaxSplitPages;
  pl.n_splits = max_pages > 0 ? (int)(((long long)max_pages + pl.split_pages - 1) / pl.split_pages) : 1;
  if (pl.n_splits < 1) pl.n_splits = 1;
  if (pl.n_splits == 1) return pl;
  pl.part_lse_elems = mul_sat(1, {B, pl.n_splits, Hq});
  pl.part_o_elems = mul_sat(pl.part_lse_elems, {D});
  pl.bytes = add_sat(aligned_bytes(pl.part_o_elems), aligned_bytes(pl.part_lse_elems));
  return pl;
}

// Compute units of the current device (cached per device id; threads that
// race on a first query store the same value).
int device_cus() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool dtype_ok(attn_dtype d) { return d == ATTN_F32 || d == ATTN_BF16 || d == ATTN_F16; }

}  // namespace

extern "C" {

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "null pointer argument";
    case ATTN_E_SHAPE: return "invalid or inconsistent sizes";
    case ATTN_E_DTYPE: return "unknown element type";
    case ATTN_E_UNSUPPORTED: return "configuration not supported by this build";
    case ATTN_E_VALUE: return "invalid value (non-finite scale)";
    case ATTN_E_WORKSPACE: return "workspace missing or too small";
    case ATTN_E_HIP: return "HIP runtime error";
    default: break;
  }
  return "unknown status";
}

const char* attn_last_error(void) { return g_last_error; }

const char* attn_last_hip_error(void) { return g_last_hip_error; }

const char* attn_kernel_name(attn_kernel_kind kind) {
  switch (kind) {
    case ATTN_KERNEL_DECODE_SPLIT: return "decode_split";
    case ATTN_KERNEL_DECODE_COMBINE: return "decode_combine";
    case ATTN_KERNEL_PREFILL: return "prefill";
    case ATTN_KERNEL_PREFILL_PAGED: return "prefill_paged";
    case ATTN_KERNEL_MERGE: return "merge";
    case ATTN_KERNEL_CASCADE_PREFIX: return "cascade_prefix";
    case ATTN_KERNEL_CASCADE_SUFFIX: return "cascade_suffix";
    default: return "unknown";
  }
}

size_t attn_decode_paged_workspace_size(attn_dtype dtype, int B, int Hq, int Hkv, int D,
                                        int page_size, int max_kv_len, int split_pages) {
  if (!dtype_ok(dtype) || B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || page_size <= 0 ||
      max_kv_len < 0 || split_pages < 0 || Hq % Hkv != 0)
    return 0;
  return plan_decode((int)dtype, B, Hq, Hkv, D, page_size, max_kv_len, split_pages).bytes;
}

// Both decode entry points; fp8_kv: the pages hold E4M3 bytes with scales
// k_scale / v_scale.
static attn_status decode_impl(attn_dtype dtype, bool fp8_kv, int kv_hnd, int window_left,
                               bool rope, float rope_theta, float rope_scale, const void* q,
                               const void* k_pages,
                               const void* v_pages, const int32_t* page_table,
                               const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                               int page_size, int num_pages, int max_pages_per_req,
                               int max_kv_len, int split_pages, float scale, float k_scale,
                               float v_scale, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, void* stream, bool noalloc = false) {
  g_last_error[0] = 0;
  g_last_hip_error[0] = 0;
  if (!dtype_ok(dtype)) return fail(ATTN_E_DTYPE, "dtype %d is not ATTN_F32/ATTN_BF16/ATTN_F16", dtype);
  if (fp8_kv && dtype == ATTN_F32)
    return fail(ATTN_E_UNSUPPORTED, "decode_paged_fp8: queries must be ATTN_BF16 or ATTN_F16");
  if (fp8_kv && (!std::isfinite(k_scale) || !std::isfinite(v_scale)))
    return fail(ATTN_E_VALUE, "k_scale / v_scale not finite");
  if (window_left < -1) return fail(ATTN_E_VALUE, "window_left=%d (-1 = no window)", window_left);
  if (rope && !(std::isfinite(rope_theta) && rope_theta > 0.f && std::isfinite(rope_scale) &&
                rope_scale > 0.f))
    return fail(ATTN_E_VALUE, "rope_theta / rope_scale must be finite and positive");
  if (rope && (dtype == ATTN_F32 || (D != 64 && D != 128)))
    return fail(ATTN_E_UNSUPPORTED, "rotary decode: dtype=%d D=%d not built (bf16/f16, D 64 or 128)",
                dtype, D);
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || page_size <= 0 || num_pages < 0 ||
      max_pages_per_req < 0 || max_kv_len < 0 || split_pages < 0)
    return fail(ATTN_E_SHAPE,
                "negative or zero size (B=%d Hq=%d Hkv=%d D=%d page_size=%d num_pages=%d "
                "max_pages_per_req=%d max_kv_len=%d split_pages=%d)",
                B, Hq, Hkv, D, page_size, num_pages, max_pages_per_req, max_kv_len, split_pages);
  if (Hq % Hkv != 0) return fail(ATTN_E_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if ((long)max_kv_len > (long)max_pages_per_req * page_size)
    return fail(ATTN_E_SHAPE, "max_kv_len=%d exceeds max_pages_per_req*page_size=%ld", max_kv_len,
                (long)max_pages_per_req * page_size);
  if (max_kv_len > ATTN_MAX_TOKENS)
    return fail(ATTN_E_UNSUPPORTED, "max_kv_len=%d exceeds ATTN_MAX_TOKENS=%d", max_kv_len,
                ATTN_MAX_TOKENS);
  // The balanced schedule counts (request, head group, 16-token block) units
  // of the whole batch in an int.
  if (dtype != ATTN_F32 &&
      !product_at_most({B, ((long long)max_kv_len + 15) / 16 + 1, ((long long)Hkv + 7) / 8},
                       ATTN_MAX_TOKENS))
    return fail(ATTN_E_UNSUPPORTED, "decode: B=%d x (ceil(max_kv_len/16)+1) x ceil(Hkv/8) "
                "exceeds ATTN_MAX_TOKENS=%d", B, ATTN_MAX_TOKENS);
  if (!std::isfinite(scale)) return fail(ATTN_E_VALUE, "scale is not finite");
  const int G = Hq / Hkv;
  if (!attn::decode_supported((int)dtype, D, G, page_size))
    return fail(ATTN_E_UNSUPPORTED, "decode: dtype=%d D=%d G=%d page_size=%d not built "
                "(bf16/f16: D in {64,128,256}, page_size 16, 32, ..., 256; f32: D in {64,128}, page_size 16; G in {1,2,4,8})", dtype, D, G, page_size);
  if (dtype != ATTN_F32 &&
      (long)num_pages * (kv_hnd ? Hkv : 1) * (page_size / 16) > (long)INT_MAX)
    return fail(ATTN_E_UNSUPPORTED, "decode: num_pages=%d too large for 16-token block ids "
                "(num_pages * %s page_size/16 must stay below 2^31)", num_pages,
                kv_hnd ? "Hkv *" : "");
  if (B == 0) return ATTN_OK;
  // With max_kv_len 0 no page is read (a longer kv_len is inconsistent and
  // only poisons its request), so the cache and its table may be empty.
  if (!q || !kv_lens || !out || !lse || (max_kv_len > 0 && (!k_pages || !v_pages || !page_table)))
    return fail(ATTN_E_NULL, "a required pointer is NULL");
  if (num_pages == 0 && max_kv_len > 0)
    return fail(ATTN_E_SHAPE, "num_pages is 0 but max_kv_len=%d", max_kv_len);
  const DecodePlan pl = plan_decode((int)dtype, B, Hq, Hkv, D, page_size, max_kv_len, split_pages);
  if (pl.bytes == SIZE_MAX)
    return fail(ATTN_E_SHAPE, "decode: the workspace size does not fit in size_t");
  if (noalloc && pl.bytes > 0) {
    // Partial states in the static per-device array instead of a workspace.
    if (pl.bytes > (size_t)ATTN_DECODE_NOALLOC_SCRATCH_BYTES)
      return fail(ATTN_E_WORKSPACE,
                  "decode_paged_noalloc: this call needs %zu bytes of partial state, more than the "
                  "%zu-byte static scratch array (use attn_decode_paged with a workspace)",
                  pl.bytes, (size_t)ATTN_DECODE_NOALLOC_SCRATCH_BYTES);
    const hipError_t e = attn::decode_scratch(&workspace, &workspace_bytes);
    if (e != hipSuccess)
      return fail_hip(e, "decode_paged_noalloc: scratch address");
  }
  if (pl.bytes > 0 && (!workspace || workspace_bytes < pl.bytes))
    return fail(ATTN_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", pl.bytes,
                workspace ? workspace_bytes : (size_t)0);
  if (((uintptr_t)q | (uintptr_t)k_pages | (uintptr_t)v_pages | (uintptr_t)out) % 16 != 0)
    return fail(ATTN_E_UNSUPPORTED, "q, k_pages, v_pages and out must be 16-byte aligned");
  if (pl.bytes > 0 && (uintptr_t)workspace % 16 != 0)
    return fail(ATTN_E_UNSUPPORTED, "workspace must be 16-byte aligned");

  attn::DecodeParams p{};
  p.q = q; p.k_pages = k_pages; p.v_pages = v_pages;
  p.page_table = page_table; p.kv_lens = kv_lens;
  p.out = out; p.lse = lse;
  if (pl.bytes > 0) {
    p.part_o = reinterpret_cast<float*>(workspace);
    const size_t o_bytes = aligned_bytes(pl.part_o_elems);
    p.part_lse = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + o_bytes);
    if (dtype != ATTN_F32)
      p.unit_start = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(workspace) + o_bytes +
                                                aligned_bytes(pl.part_lse_elems));
  }
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.num_pages = num_pages; p.max_pages = max_pages_per_req;
  p.max_kv_len = max_kv_len; p.split_pages = pl.split_pages; p.n_splits = pl.n_splits;
  p.min_run = pl.min_run; p.max_segs = pl.max_segs;
  p.page_shift = 0;
  while ((16 << p.page_shift) < page_size) ++p.page_shift;   // page_size = 16 << shift (checked)
  p.max_tokens = (int)std::min<long>((long)max_pages_per_req * page_size, (long)INT_MAX);
  // Balanced bf16 grid: one wave per KV head of a group of up to 8 heads,
  // kDecodeGroupsPerCU workgroups per compute unit.
  p.hw = Hkv < 8 ? Hkv : 8;
  p.nhg = (int)(((long long)Hkv + p.hw - 1) / p.hw);
  p.n_groups = attn::kDecodeGroupsPerCU * device_cus();
  p.scale_log2 = fp8_kv ? scale * k_scale * kLog2e : scale * kLog2e;
  p.v_scale = fp8_kv ? v_scale : 1.f;
  p.kv_hnd = kv_hnd;
  p.window_left = window_left;
  p.rope_log2_theta = rope ? std::log2(rope_theta) : 0.f;
  p.rope_inv_scale = rope ? 1.f / rope_scale : 1.f;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = timed(ATTN_KERNEL_DECODE_SPLIT, s,
                       [&] { return attn::launch_decode_split(p, (int)dtype, D, G, fp8_kv, rope, s); });
  if (e != hipSuccess)
    return fail_hip(e, "decode_split launch");
  if (dtype != ATTN_F32 || pl.n_splits > 1) {
    e = timed(ATTN_KERNEL_DECODE_COMBINE, s,
              [&] { return attn::launch_decode_combine(p, (int)dtype, D, G, s); });
    if (e != hipSuccess)
      return fail_hip(e, "decode_combine launch");
  }
  return ATTN_OK;
}

attn_status attn_decode_paged(attn_dtype dtype, const void* q, const void* k_pages,
                              const void* v_pages, const int32_t* page_table,
                              const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                              int page_size, int num_pages, int max_pages_per_req,
                              int max_kv_len, int split_pages, float scale, void* out,
                              float* lse, void* workspace, size_t workspace_bytes,
                              void* stream) {
  return decode_impl(dtype, false, 0, -1, false, 0.f, 0.f, q, k_pages, v_pages, page_table,
                     kv_lens, B, Hq, Hkv, D,
                     page_size, num_pages, max_pages_per_req, max_kv_len, split_pages, scale, 1.f,
                     1.f, out, lse, workspace, workspace_bytes, stream);
}

attn_status attn_decode_paged_noalloc(attn_dtype dtype, const void* q, const void* k_pages,
                                      const void* v_pages, const int32_t* page_table,
                                      const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                      int page_size, int num_pages, int max_pages_per_req,
                                      int max_kv_len, int split_pages, float scale, void* out,
                                      float* lse, void* stream) {
  return decode_impl(dtype, false, 0, -1, false, 0.f, 0.f, q, k_pages, v_pages, page_table,
                     kv_lens, B, Hq, Hkv, D, page_size, num_pages, max_pages_per_req, max_kv_len,
                     split_pages, scale, 1.f, 1.f, out, lse, nullptr, 0, stream,
                     /*noalloc=*/true);
}

attn_status attn_decode_paged_hnd(attn_dtype dtype, const void* q, const void* k_pages,
                                  const void* v_pages, const int32_t* page_table,
                                  const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                  int page_size, int num_pages, int max_pages_per_req,
                                  int max_kv_len, int split_pages, float scale, void* out,
                                  float* lse, void* workspace, size_t workspace_bytes,
                                  void* stream) {
  return decode_impl(dtype, false, 1, -1, false, 0.f, 0.f, q, k_pages, v_pages, page_table,
                     kv_lens, B, Hq, Hkv, D,
                     page_size, num_pages, max_pages_per_req, max_kv_len, split_pages, scale, 1.f,
                     1.f, out, lse, workspace, workspace_bytes, stream);
}

attn_status attn_decode_paged_fp8(attn_dtype dtype, const void* q, const void* k_pages,
                                  const void* v_pages, const int32_t* page_table,
                                  const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                  int page_size, int num_pages, int max_pages_per_req,
                                  int max_kv_len, int split_pages, float scale, float k_scale,
                                  float v_scale, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_impl(dtype, true, 0, -1, false, 0.f, 0.f, q, k_pages, v_pages, page_table,
                     kv_lens, B, Hq, Hkv, D,
                     page_size, num_pages, max_pages_per_req, max_kv_len, split_pages, scale,
                     k_scale, v_scale, out, lse, workspace, workspace_bytes, stream);
}

attn_status attn_decode_paged_fp8_window(attn_dtype dtype, int kv_layout, int window_left,
                                         const void* q, const void* k_pages, const void* v_pages,
                                         const int32_t* page_table, const int32_t* kv_lens, int B,
                                         int Hq, int Hkv, int D, int page_size, int num_pages,
                                         int max_pages_per_req, int max_kv_len, int split_pages,
                                         float scale, float k_scale, float v_scale, void* out,
                                         float* lse, void* workspace, size_t workspace_bytes,
                                         void* stream) {
  g_last_error[0] = 0;
  g_last_hip_error[0] = 0;
  if (kv_layout != 0 && kv_layout != 1)
    return fail(ATTN_E_VALUE, "kv_layout=%d (0 = NHD, 1 = HND)", kv_layout);
  return decode_impl(dtype, true, kv_layout, window_left, false, 0.f, 0.f, q, k_pages, v_pages,
                     page_table, kv_lens, B, Hq, Hkv, D, page_size, num_pages, max_pages_per_req,
                     max_kv_len, split_pages, scale, k_scale, v_scale, out, lse, workspace,
                     workspace_bytes, stream);
}

attn_status attn_decode_paged_window(attn_dtype dtype, int kv_layout, int window_left,
                                     const void* q, const void* k_pages, const void* v_pages,
                                     const int32_t* page_table, const int32_t* kv_lens, int B,
                                     int Hq, int Hkv, int D, int page_size, int num_pages,
                                     int max_pages_per_req, int max_kv_len, int split_pages,
                                     float scale, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  g_last_hip_error[0] = 0;
  if (kv_layout != 0 && kv_layout != 1)
    return fail(ATTN_E_VALUE, "kv_layout=%d (0 = NHD, 1 = HND)", kv_layout);
  return decode_impl(dtype, false, kv_layout, window_left, false, 0.f, 0.f, q, k_pages, v_pages,
                     page_table,
                     kv_lens, B, Hq, Hkv, D, page_size, num_pages, max_pages_per_req, max_kv_len,
                     split_pages, scale, 1.f, 1.f, out, lse, workspace, workspace_bytes, stream);
}

attn_status attn_decode_paged_rope(attn_dtype dtype, int kv_layout, int window_left,
                                   float rope_theta, float rope_scale, const void* q,
                                   const void* k_pages, const void* v_pages,
                                   const int32_t* page_table, const int32_t* kv_lens, int B, int Hq,
                                   int Hkv, int D, int page_size, int num_pages,
                                   int max_pages_per_req, int max_kv_len, int split_pages,
                                   float scale, void* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  g_last_error[0] = 0;
  g_last_hip_error[0] = 0;
  if (kv_layout != 0 && kv_layout != 1)
    return fail(ATTN_E_VALUE, "kv_layout=%d (0 = NHD, 1 = HND)", kv_layout);
  return decode_impl(dtype, false, kv_layout, window_left, true, rope_theta, rope_scale, q,
                     k_pages, v_pages, page_table, kv_lens, B, Hq, Hkv, D, page_size, num_pages,
                     max_pages_per_req, max_kv_len, split_pages, scale, 1.f, 1.f, out, lse,
                     workspace, workspace_bytes, stream);
}

attn_status attn_decode_paged_fp8_hnd(attn_dtype dtype, const void* q, const void* k_pages,
                                      const void* v_pages, const int32_t* page_table,
                                      const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                      int page_size, int num_pages, int max_pages_per_req,
                                      int max_kv_len, int split_pages, float scale,
                                      float k_scale, float v_scale, void* out, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(dtype, true, 1, -1, false, 0.f, 0.f, q, k_pages, v_pages, page_table,
                     kv_lens, B, Hq, Hkv, D,
                     page_size, num_pages, max_pages_per_req, max_kv_len, split_pages, scale,
                     k_scale, v_scale, out, lse, workspace, workspace_bytes, stream);
}

static attn_status check_prefill_common(attn_dtype dtype, int B, int Hq, int Hkv, int D,
                                        int total_q, int max_seqlen_q, int causal, float scale) {
  if (!dtype_ok(dtype)) return fail(ATTN_E_DTYPE, "dtype %d is not ATTN_F32/ATTN_BF16/ATTN_F16", dtype);
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || total_q < 0 || max_seqlen_q < 0)
    return fail(ATTN_E_SHAPE, "negative or zero size (B=%d Hq=%d Hkv=%d D=%d total_q=%d "
                "max_seqlen_q=%d)", B, Hq, Hkv, D, total_q, max_seqlen_q);
  if (Hq % Hkv != 0) return fail(ATTN_E_SHAPE, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (total_q > ATTN_MAX_TOKENS || max_seqlen_q > ATTN_MAX_TOKENS)
    return fail(ATTN_E_UNSUPPORTED, "total_q=%d or max_seqlen_q=%d exceeds ATTN_MAX_TOKENS=%d",
                total_q, max_seqlen_q, ATTN_MAX_TOKENS);
  if (causal != 0 && causal != 1) return fail(ATTN_E_VALUE, "causal must be 0 or 1");
  if (!std::isfinite(scale)) return fail(ATTN_E_VALUE, "scale is not finite");
  if (!attn::prefill_supported((int)dtype, D))
    return fail(ATTN_E_UNSUPPORTED, "prefill: dtype=%d D=%d not built (bf16/f16, D in {128,256})",
                dtype, D);
  // One workgroup per (query head, sequence, query tile), indexed by an int.
  const long long tiles = ((long long)max_seqlen_q + attn::kPrefillBM - 1) / attn::kPrefillBM;
  if (!product_at_most({Hq, B, tiles}, INT_MAX - 8))
    return fail(ATTN_E_SHAPE, "Hq=%d x B=%d x ceil(max_seqlen_q / %d)=%lld work items exceeds %d",
                Hq, B, attn::kPrefillBM, tiles, INT_MAX - 8);
  return ATTN_OK;
}

// Query i of a sequence (Lq <= max_q queries, Lk <= max_k keys) sees keys
// i + (Lk - Lq) - left .. i + (Lk - Lq) + right.  Since i + (Lk - Lq) lies in
// [Lk - Lq, Lk - 1], a left side of at least max_k and a right side of at
// least max_q bound nothing: they become -1, which also keeps the kernels'
// index sums (at most a length plus a window, each below 2^30) inside an int.
static void window_clamp(int left, int right, int max_q, int max_k, attn::PrefillParams& p) {
  p.window_left = left >= max_k ? -1 : left;
  p.window_right = right >= max_q ? -1 : right;
}

static attn_status prefill_varlen_impl(attn_dtype dtype, const void* q, const void* k,
                                       const void* v, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_k, int B, int Hq, int Hkv, int D,
                                       int total_q, int total_k, int max_seqlen_q,
                                       int max_seqlen_k, int causal, int window_left,
                                       int window_right, float scale, void* out, float* lse,
                                       void* stream) {
  g_last_error[0] = 0;
  g_last_hip_error[0] = 0;
  attn_status st = check_prefill_common(dtype, B, Hq, Hkv, D, total_q, max_seqlen_q, causal, scale);
  if (st != ATTN_OK) return st;
  if (window_left < -1) return fail(ATTN_E_VALUE, "window_left=%d (-1 = no window)", window_left);
  if (window_right < -1)
    return fail(ATTN_E_VALUE, "window_right=%d (-1 = no bound)", window_right);
  if (total_k < 0 || max_seqlen_k < 0)
    return fail(ATTN_E_SHAPE, "negative total_k=%d or max_seqlen_k=%d", total_k, max_seqlen_k);
  if (total_k > ATTN_MAX_TOKENS || max_seqlen_k > ATTN_MAX_TOKENS)
    return fail(ATTN_E_UNSUPPORTED, "total_k=%d or max_seqlen_k=%d exceeds ATTN_MAX_TOKENS=%d",
                total_k, max_seqlen_k, ATTN_MAX_TOKENS);
  if (B == 0 || max_seqlen_q == 0 || total_q == 0) return ATTN_OK;
  // With total_k 0 every sequence has no keys: k and v are never read.
  if (!q || !cu_seqlens_q || !cu_seqlens_k || !out || !lse || (total_k > 0 && (!k || !v)))
    return fail(ATTN_E_NULL, "a required pointer is NULL");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) % 16 != 0)
    return fail(ATTN_E_UNSUPPORTED, "q, k, v and out must be 16-byte aligned");
  attn::PrefillParams p{};
  p.q = q; p.k = k; p.v = v; p.cu_q = cu_seqlens_q; p.cu_k = cu_seqlens_k;
  p.out = out; p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.total_q = total_q; p.total_k = total_k;
  p.max_seqlen_q = max_seqlen_q; p.max_seqlen_k = max_seqlen_k; p.causal = causal;
  p.q_tiles = (max_seqlen_q + attn::kPrefillBM - 1) / attn::kPrefillBM;
  p.scale_log2 = scale * kLog2e;
  window_clamp(window_left, window_right, max_seqlen_q, max_seqlen_k, p);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = timed(ATTN_KERNEL_PREFILL, s, [&] { return attn::launch_prefill(p, (int)dtype, D, false, s); });
  if (e != hipSuccess) return fail_hip(e, "prefill launch");
  return ATTN_OK;
}

attn_status attn_prefill_varlen(attn_dtype dtype, const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int B, int Hq, int Hkv, int D, int total_q, int total_k,
                                int max_seqlen_q, int max_seqlen_k, int causal, float scale,
                                void* out, float* lse, void* stream) {
  return prefill_varlen_impl(dtype, q, k, v, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, D, total_q,
                             total_k, max_seqlen_q, max_seqlen_k, causal, -1, -1, scale, out, lse,
                             stream);
}

attn_status attn_prefill_varlen_window(attn_dtype dtype, const void* q, const void* k,
                                       const void* v, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_k, int B, int Hq, int Hkv, int D,
                                       int total_q, int total_k, int max_seqlen_q,
                                       int max_seqlen_k, int causal, int window_left,
                                       int window_right, float scale, void* out, float* lse,
                                       void* stream) {
  return prefill_varlen_impl(dtype, q, k, v, cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, D, total_q,
                             total_k, max_seqlen_q, max_seqlen_k, causal, window_left,
                             window_right, scale, out, lse, stream);
}

// Checks shared by the paged prefill entry points; on ATTN_OK, `p` holds the
// launch parameters of the plain paged call and `empty` says there is no work.
static attn_status paged_prefill_params(attn_dtype dtype, const void* q,
                                        const int32_t* cu_seqlens_q, const void* k_pages,
                                        const void* v_pages, const int32_t* page_table,
                                        const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                        int total_q, int page_size, int num_pages,
                                        int max_pages_per_req, int max_seqlen_q, int max_kv_len,
                                        int causal, float scale, void* out, float* lse,
                                        int kv_hnd, attn::PrefillParams& p, bool& empty) {
  attn_status st = check_prefill_common(dtype, B, Hq, Hkv, D, total_q, max_seqlen_q, causal, scale);
  if (st != ATTN_OK) return st;
  if (page_size <= 0 || num_pages < 0 || max_pages_per_req < 0 || max_kv_len < 0)
    return fail(ATTN_E_SHAPE, "negative or zero size (page_size=%d num_pages=%d "
                "max_pages_per_req=%d max_kv_len=%d)", page_size, num_pages, max_pages_per_req,
                max_kv_len);
  if (page_size < 16 || page_size > 256 || (page_size & (page_size - 1)) != 0)
    return fail(ATTN_E_UNSUPPORTED, "prefill_paged: page_size=%d not built (16, 32, ..., 256)",
                page_size);
  if (max_kv_len > ATTN_MAX_TOKENS)
    return fail(ATTN_E_UNSUPPORTED, "max_kv_len=%d exceeds ATTN_MAX_TOKENS=%d", max_kv_len,
                ATTN_MAX_TOKENS);
  if ((long)num_pages * (kv_hnd ? Hkv : 1) * (page_size / 16) > (long)INT_MAX)
    return fail(ATTN_E_UNSUPPORTED, "prefill_paged: num_pages=%d too large for 16-token block ids",
                num_pages);
  if ((long)max_kv_len > (long)max_pages_per_req * page_size)
    return fail(ATTN_E_SHAPE, "max_kv_len=%d exceeds max_pages_per_req*page_size=%ld", max_kv_len,
                (long)max_pages_per_req * page_size);
  empty = B == 0 || max_seqlen_q == 0 || total_q == 0;
  if (empty) return ATTN_OK;
  // With max_kv_len 0 no page is read (see the decode check).
  if (!q || !cu_seqlens_q || !kv_lens || !out || !lse ||
      (max_kv_len > 0 && (!k_pages || !v_pages || !page_table)))
    return fail(ATTN_E_NULL, "a required pointer is NULL");
  if (num_pages == 0 && max_kv_len > 0)
    return fail(ATTN_E_SHAPE, "num_pages is 0 but max_kv_len=%d", max_kv_len);
  if (((uintptr_t)q | (uintptr_t)k_pages | (uintptr_t)v_pages | (uintptr_t)out) % 16 != 0)
    return fail(ATTN_E_UNSUPPORTED, "q, k_pages, v_pages and out must be 16-byte aligned");
  p = attn::PrefillParams{};
  p.q = q; p.k = k_pages; p.v = v_pages; p.cu_q = cu_seqlens_q;
  p.page_table = page_table; p.kv_lens = kv_lens;
  p.out = out; p.lse = lse;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.total_q = total_q; p.total_k = 0;
  p.max_seqlen_q = max_seqlen_q; p.max_seqlen_k = max_kv_len;
  p.num_pages = num_pages; p.max_pages = max_pages_per_req; p.causal = causal;
  p.table_stride = max_pages_per_req; p.kv_offset = 0; p.kv_len_fixed = -1;
  p.kv_hnd = kv_hnd;
  p.window_left = -1;
  p.window_right = -1;
  p.page_shift = 0;
  while ((16 << p.page_shift) < page_size) ++p.page_shift;
  p.max_tokens = (int)std::min<long>((long)max_pages_per_req * page_size, (long)INT_MAX);
  p.q_tiles = (max_seqlen_q + attn::kPrefillBM - 1) / attn::kPrefillBM;
  p.scale_log2 = scale * kLog2e;
  return ATTN_OK;
}

static attn_status prefill_paged_impl(attn_dtype dtype, int kv_hnd, int window_left,
                                      int window_right, const void* q,
                                      const int32_t* cu_seqlens_q, const void* k_pages,
                                      const void* v_pages, const int32_t* page_table,
                                      const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                      int total_q, int page_size, int num_pages,
                                      int max_pages_per_req, int max_seqlen_q, int max_kv_len,
                                      int causal, float scale, void* out, float* lse,
                                      void* stream) {
  g_last_error[0] = 0;
  g_last_hip_error[0] = 0;
  attn::PrefillParams p;
  bool empty = false;
  attn_status st = paged_prefill_params(dtype, q, cu_seqlens_q, k_pages, v_pages, page_table,
                                        kv_lens, B, Hq, Hkv, D, total_q, page_size, num_pages,
                                        max_pages_per_req, max_seqlen_q, max_kv_len, causal, scale,
                                        out, lse, kv_hnd, p, empty);
  if (st != ATTN_OK) return st;
  if (window_left < -1) return fail(ATTN_E_VALUE, "window_left=%d (-1 = no window)", window_left);
  if (window_right < -1)
    return fail(ATTN_E_VALUE, "window_right=%d (-1 = no bound)", window_right);
  if (empty) return ATTN_OK;
  window_clamp(window_left, window_right, max_seqlen_q, max_kv_len, p);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e =
      timed(ATTN_KERNEL_PREFILL_PAGED, s, [&] { return attn::launch_prefill(p, (int)dtype, D, true, s); });
  if (e != hipSuccess) return fail_hip(e, "prefill_paged launch");
  return ATTN_OK;
}

attn_status attn_prefill_paged(attn_dtype dtype, const void* q, const int32_t* cu_seqlens_q,
                               const void* k_pages, const void* v_pages,
                               const int32_t* page_table, const int32_t* kv_lens, int B, int Hq,
                               int Hkv, int D, int total_q, int page_size, int num_pages,
                               int max_pages_per_req, int max_seqlen_q, int max_kv_len,
                               int causal, float scale, void* out, float* lse, void* stream) {
  return prefill_paged_impl(dtype, 0, -1, -1, q, cu_seqlens_q, k_pages, v_pages, page_table, kv_lens, B,
                            Hq, Hkv, D, total_q, page_size, num_pages, max_pages_per_req,
                            max_seqlen_q, max_kv_len, causal, scale, out, lse, stream);
}

attn_status attn_prefill_paged_hnd(attn_dtype dtype, const void* q, const int32_t* cu_seqlens_q,
                                   const void* k_pages, const void* v_pages,
                                   const int32_t* page_table, const int32_t* kv_lens, int B,
                                   int Hq, int Hkv, int D, int total_q, int page_size,
                                   int num_pages, int max_pages_per_req, int max_seqlen_q,
                                   int max_kv_len, int causal, float scale, void* out,
                                   float* lse, void* stream) {
  return prefill_paged_impl(dtype, 1, -1, -1, q, cu_seqlens_q, k_pages, v_pages, page_table, kv_lens, B,
                            Hq, Hkv, D, total_q, page_size, num_pages, max_pages_per_req,
                            max_seqlen_q, max_kv_len, causal, scale, out, lse, stream);
}

attn_status attn_prefill_paged_window(attn_dtype dtype, int kv_layout, const void* q,
                                      const int32_t* cu_seqlens_q, const void* k_pages,
                                      const void* v_pages, const int32_t* page_table,
                                      const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                      int total_q, int page_size, int num_pages,
                                      int max_pages_per_req, int max_seqlen_q, int max_kv_len,
                                      int causal, int window_left, int window_right,
                                      float scale, void* out, float* lse, void* stream) {
  g_last_error[0] = 0;
  g_last_hip_error[0] = 0;
  if (kv_layout != 0 && kv_layout != 1)
    return fail(ATTN_E_VALUE, "kv_layout=%d (0 = NHD, 1 = HND)", kv_layout);
  return prefill_paged_impl(dtype, kv_layout, window_left, window_right, q, cu_seqlens_q, k_pages, v_pages,
                            page_table, kv_lens, B, Hq, Hkv, D, total_q, page_size, num_pages,
                            max_pages_per_req, max_seqlen_q, max_kv_len, causal, scale, out, lse,
                            stream);
}

static size_t elem_bytes(attn_dtype dtype) { return dtype == ATTN_F32 ? 4 : 2; }

size_t attn_prefill_paged_cascade_workspace_size(attn_dtype dtype, int total_q, int Hq, int D) {
  if (!dtype_ok(dtype) || total_q < 0 || Hq <= 0 || D <= 0) return 0;
  const size_t rows = mul_sat(1, {total_q, Hq});
  return add_sat(round256(mul_sat(rows, {D, (long long)elem_bytes(dtype)})), aligned_bytes(rows));
}

static attn_status cascade_impl(attn_dtype dtype, int kv_hnd, const void* q,
                                       const int32_t* cu_seqlens_q, const void* k_pages,
                                       const void* v_pages, const int32_t* page_table,
                                       const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                       int total_q, int page_size, int num_pages,
                                       int max_pages_per_req, int max_seqlen_q, int max_kv_len,
                                       int shared_prefix_len, int causal, float scale, void* out,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  g_last_error[0] = 0;
  g_last_hip_error[0] = 0;
  attn::PrefillParams p;
  bool empty = false;
  attn_status st = paged_prefill_params(dtype, q, cu_seqlens_q, k_pages, v_pages, page_table,
                                        kv_lens, B, Hq, Hkv, D, total_q, page_size, num_pages,
                                        max_pages_per_req, max_seqlen_q, max_kv_len, causal, scale,
                                        out, lse, kv_hnd, p, empty);
  if (st != ATTN_OK) return st;
  if (shared_prefix_len < 0 || shared_prefix_len % page_size != 0)
    return fail(ATTN_E_SHAPE, "shared_prefix_len=%d is not a non-negative multiple of "
                "page_size=%d", shared_prefix_len, page_size);
  if (shared_prefix_len > max_kv_len)
    return fail(ATTN_E_SHAPE, "shared_prefix_len=%d exceeds max_kv_len=%d", shared_prefix_len,
                max_kv_len);
  if (empty) return ATTN_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (shared_prefix_len == 0) {
    hipError_t e = timed(ATTN_KERNEL_PREFILL_PAGED, s,
                         [&] { return attn::launch_prefill(p, (int)dtype, D, true, s); });
    if (e != hipSuccess) return fail_hip(e, "prefill_paged launch");
    return ATTN_OK;
  }
  // The shared-prefix pass runs every query row as one sequence.
  const long long tiles = ((long long)total_q + attn::kPrefillBM - 1) / attn::kPrefillBM;
  if (!product_at_most({Hq, tiles}, INT_MAX - 8))
    return fail(ATTN_E_SHAPE, "Hq=%d x ceil(total_q / %d)=%lld work items exceeds %d", Hq,
                attn::kPrefillBM, tiles, INT_MAX - 8);
  const size_t need = attn_prefill_paged_cascade_workspace_size(dtype, total_q, Hq, D);
  if (!workspace || workspace_bytes < need)
    return fail(ATTN_E_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace_bytes);
  if ((uintptr_t)workspace % 256 != 0)
    return fail(ATTN_E_UNSUPPORTED, "workspace must be 256-byte aligned");
  void* pre_o = workspace;
  float* pre_lse = reinterpret_cast<float*>(
      reinterpret_cast<char*>(workspace) +
      round256(mul_sat(1, {total_q, Hq, D, (long long)elem_bytes(dtype)})));

  attn::PrefillParams pre = p;
  pre.B = 1;
  pre.causal = 0;
  pre.kv_len_fixed = shared_prefix_len;
  pre.max_seqlen_q = total_q;
  pre.q_tiles = (total_q + attn::kPrefillBM - 1) / attn::kPrefillBM;
  pre.out = pre_o;
  pre.lse = pre_lse;
  hipError_t e = timed(ATTN_KERNEL_CASCADE_PREFIX, s,
                       [&] { return attn::launch_prefill(pre, (int)dtype, D, true, s); });
  if (e != hipSuccess) return fail_hip(e, "cascade prefix launch");

  attn::PrefillParams suf = p;
  suf.kv_offset = shared_prefix_len;
  suf.merge_o = pre_o;
  suf.merge_lse = pre_lse;
  e = timed(ATTN_KERNEL_CASCADE_SUFFIX, s,
            [&] { return attn::launch_prefill(suf, (int)dtype, D, true, s); });
  if (e != hipSuccess) return fail_hip(e, "cascade suffix launch");
  return ATTN_OK;
}

attn_status attn_prefill_paged_cascade(attn_dtype dtype, const void* q,
                                       const int32_t* cu_seqlens_q, const void* k_pages,
                                       const void* v_pages, const int32_t* page_table,
                                       const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                       int total_q, int page_size, int num_pages,
                                       int max_pages_per_req, int max_seqlen_q, int max_kv_len,
                                       int shared_prefix_len, int causal, float scale, void* out,
                                       float* lse, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  return cascade_impl(dtype, 0, q, cu_seqlens_q, k_pages, v_pages, page_table, kv_lens, B, Hq,
                      Hkv, D, total_q, page_size, num_pages, max_pages_per_req, max_seqlen_q,
                      max_kv_len, shared_prefix_len, causal, scale, out, lse, workspace,
                      workspace_bytes, stream);
}

attn_status attn_prefill_paged_cascade_hnd(attn_dtype dtype, const void* q,
                                           const int32_t* cu_seqlens_q, const void* k_pages,
                                           const void* v_pages, const int32_t* page_table,
                                           const int32_t* kv_lens, int B, int Hq, int Hkv, int D,
                                           int total_q, int page_size, int num_pages,
                                           int max_pages_per_req, int max_seqlen_q,
                                           int max_kv_len, int shared_prefix_len, int causal,
                                           float scale, void* out, float* lse, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  return cascade_impl(dtype, 1, q, cu_seqlens_q, k_pages, v_pages, page_table, kv_lens, B, Hq,
                      Hkv, D, total_q, page_size, num_pages, max_pages_per_req, max_seqlen_q,
                      max_kv_len, shared_prefix_len, causal, scale, out, lse, workspace,
                      workspace_bytes, stream);
}

attn_status attn_merge_states(attn_dtype dtype, const void* o_a, const float* lse_a,
                              const void* o_b, const float* lse_b, int rows, int D, void* out,
                              float* lse_out, void* stream) {
  g_last_error[0] = 0;
  g_last_hip_error[0] = 0;
  if (!dtype_ok(dtype)) return fail(ATTN_E_DTYPE, "dtype %d is not ATTN_F32/ATTN_BF16/ATTN_F16", dtype);
  if (rows < 0 || D <= 0) return fail(ATTN_E_SHAPE, "rows=%d D=%d", rows, D);
  if (!attn::merge_supported((int)dtype, D))
    return fail(ATTN_E_UNSUPPORTED, "merge_states: D=%d not built (64, 128, 256)", D);
  if (rows == 0) return ATTN_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !out || !lse_out)
    return fail(ATTN_E_NULL, "a required pointer is NULL");
  if (((uintptr_t)o_a | (uintptr_t)o_b | (uintptr_t)out) % 16 != 0)
    return fail(ATTN_E_UNSUPPORTED, "o_a, o_b and out must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = timed(ATTN_KERNEL_MERGE, s, [&] {
    return attn::launch_merge_states(o_a, lse_a, o_b, lse_b, out, lse_out, rows, (int)dtype, D, s);
  });
  if (e != hipSuccess) return fail_hip(e, "merge_states launch");
  return ATTN_OK;
}

attn_status attn_timing_begin(int capacity) {
  g_last_error[0] = 0;
  g_last_hip_error[0] = 0;
  if (capacity <= 0 || capacity > ATTN_TIMING_MAX_LAUNCHES)
    return fail(ATTN_E_SHAPE, "capacity=%d outside 1 .. ATTN_TIMING_MAX_LAUNCHES=%d", capacity,
                ATTN_TIMING_MAX_LAUNCHES);
  while ((int)g_timing.recs.size() < capacity) {
    TimingRecord r{};
    hipError_t e = hipEventCreate(&r.start);
    if (e != hipSuccess) return fail_hip(e, "hipEventCreate");
    e = hipEventCreate(&r.stop);
    if (e != hipSuccess) {
      (void)hipEventDestroy(r.start);
      return fail_hip(e, "hipEventCreate");
    }
    g_timing.recs.push_back(r);
  }
  g_timing.capacity = capacity;
  g_timing.used = 0;
  g_timing.on = true;
  return ATTN_OK;
}

attn_status attn_timing_end(double* ms_per_kind, int* launches_per_kind) {
  g_last_error[0] = 0;
  g_last_hip_error[0] = 0;
  g_timing.on = false;
  for (int k = 0; k < ATTN_KERNEL_KINDS; ++k) {
    if (ms_per_kind) ms_per_kind[k] = 0.0;
    if (launches_per_kind) launches_per_kind[k] = 0;
  }
  for (int i = 0; i < g_timing.used; ++i) {
    TimingRecord& r = g_timing.recs[i];
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, r.start, r.stop);
    if (e != hipSuccess) return fail_hip(e, "hipEventElapsedTime");
    if (ms_per_kind) ms_per_kind[r.kind] += ms;
    if (launches_per_kind) launches_per_kind[r.kind] += 1;
  }
  g_timing.used = 0;
  return ATTN_OK;
}

}  // extern "C"
