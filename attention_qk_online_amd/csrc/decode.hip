// Paged batched decode for gfx950: split-KV partitions streamed with 128-bit
// loads, wave64 DPP reductions and an online softmax; partial states merged
// by their log-sum-exp in a second kernel.
//
// Work item = (request b, KV head, split of `split_pages` pages).  A
// workgroup of NW waves owns one work item; wave w takes pages w, w+NW, ...
// of the split.  Inside a wave the 64 lanes form 4 groups of 16: group g
// reads tokens 4g..4g+3 of the current 16-token page, each lane holding a
// D/16-element slice of a K or V row, so a group reads whole rows with
// contiguous 16-byte loads ("FlashInfer Attention Kernel技术解析" section 1.2:
// each thread loads one 128-bit vector; "FlashInfer内核库深度解析": batched
// decode with coalesced memory access).  The G = Hq/Hkv query heads that
// share the KV head are held in registers, so K/V bytes are read once for
// the whole group (GQA).
//
// Per 4-token block and head: dot products -> sum over the 16 lanes with
// DPP -> running max m, running sum l and output o rescaled by
// 2^(m_old - m_new) ("FlashAttention-3 ..." section 一: online softmax,
// section 四: keep the rescaling).  Scores are kept in log2 units (scale is
// premultiplied by log2 e) so the exponentials are single v_exp_f32.
#include <atomic>
#include <type_traits>

#include "attn.h"

#include "common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kPage = 16;   // tokens per page handled by this kernel
constexpr int kNW = 8;      // waves per workgroup (fp32 split kernel)
constexpr int kMaxGroupWaves = 8;  // KV heads per workgroup (bf16 balanced kernel)
#ifndef ATTN_DECODE_BATCH
#define ATTN_DECODE_BATCH 2
#endif
constexpr int kBatch = ATTN_DECODE_BATCH;  // pages whose loads are issued together
#ifndef ATTN_DECODE_MFMA_BATCH
#define ATTN_DECODE_MFMA_BATCH 1
#endif
constexpr int kMfmaBatch = ATTN_DECODE_MFMA_BATCH;
#ifndef ATTN_DECODE_FP8_BATCH
#define ATTN_DECODE_FP8_BATCH 1
#endif
constexpr int kFp8Batch = ATTN_DECODE_FP8_BATCH;  // pages per batch with an E4M3 cache

template <typename T, int D>
struct Slice {
  static constexpr int VPL = D / 16;                     // elements per lane
  static constexpr int WORDS = VPL * (int)sizeof(T) / 4; // 32-bit words per lane
  uint32_t w[WORDS];

  // K/V rows are streamed once: non-temporal loads.
  __device__ __forceinline__ void load(const T* row) {
    const char* p = reinterpret_cast<const char*>(row);
    if constexpr (WORDS % 4 == 0) {
#pragma unroll
      for (int i = 0; i < WORDS / 4; ++i) {
        u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 16 * i));
        w[4 * i + 0] = x[0]; w[4 * i + 1] = x[1]; w[4 * i + 2] = x[2]; w[4 * i + 3] = x[3];
      }
    } else {
      static_assert(WORDS == 2, "slice of 8 bytes");
      u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
      w[0] = x[0]; w[1] = x[1];
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < WORDS; ++i) w[i] = 0u;
  }
  __device__ __forceinline__ float elem(int e) const {
    if constexpr (sizeof(T) == 4) {
      return __builtin_bit_cast(float, w[e]);
    } else {
      return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
    }
  }
  // Partial dot product of this lane's slice with the query slice `q`.
  __device__ __forceinline__ float dot(const Slice& q) const {
    float acc = 0.f;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int i = 0; i < WORDS; ++i)
        acc = __builtin_fmaf(__builtin_bit_cast(float, q.w[i]), __builtin_bit_cast(float, w[i]), acc);
    } else {
#pragma unroll
      for (int i = 0; i < WORDS; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, q.w[i]),
                                              __builtin_bit_cast(bf16x2, w[i]), acc, false);
    }
    return acc;
  }
};

template <typename T>
__device__ __forceinline__ void store_out(T* dst, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* dst, float x) { *dst = x; }
template <>
__device__ __forceinline__ void store_out<bf16_t>(bf16_t* dst, float x) {
  dst->bits = (uint16_t)f32_to_bf16_bits(x);
}
template <>
__device__ __forceinline__ void store_out<f16_t>(f16_t* dst, float x) {
  dst->bits = __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Number of valid tokens of request b after clamping inconsistent device data
// (negative, above max_kv_len or above the page table's capacity -> bad).
__device__ __forceinline__ int request_len(const DecodeParams& p, int b, bool& bad) {
  int kv = p.kv_lens[b];
  bad = kv < 0 || kv > p.max_kv_len || kv > p.max_tokens;
  return bad ? 0 : kv;
}

__device__ __forceinline__ int splits_of(int len, int split_pages) {
  int pages = (len + kPage - 1) / kPage;
  int ns = (pages + split_pages - 1) / split_pages;
  return ns < 1 ? 1 : ns;
}

template <typename T, int D, int G, int NB>
__global__ __launch_bounds__(kNW * 64) void decode_split_kernel(DecodeParams p) {
  using S = Slice<T, D>;
  constexpr int VPL = S::VPL;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = lane >> 4, gl = lane & 15;

  bool bad;
  const int len = request_len(p, b, bad);
  const int ns = splits_of(len, p.split_pages);
  if (split >= ns) return;
  const int pg_begin = split * p.split_pages;
  const int pg_end = min((len + kPage - 1) / kPage, pg_begin + p.split_pages);

  const T* qb = reinterpret_cast<const T*>(p.q) + ((size_t)b * p.Hq + (size_t)kvh * G) * D;
  S qs[G];
#pragma unroll
  for (int g = 0; g < G; ++g) qs[g].load(qb + (size_t)g * D + gl * VPL);

  float m[G], l[G], o[G][VPL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kNegInf;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < VPL; ++e) o[g][e] = 0.f;
  }

  const T* kbase = reinterpret_cast<const T*>(p.k_pages);
  const T* vbase = reinterpret_cast<const T*>(p.v_pages);
  // Elements between consecutive tokens of one head and from a page's start
  // to this head's first row: NHD interleaves the heads of a token, HND keeps
  // each head's 16 rows together.
  const size_t row_stride = p.kv_hnd ? (size_t)D : (size_t)p.Hkv * D;
  const size_t page_stride = (size_t)kPage * p.Hkv * D;
  const size_t lane_off = (size_t)kvh * (p.kv_hnd ? kPage * D : D) + gl * VPL;
  const int32_t* table = p.page_table + (size_t)b * p.max_pages;
  // First key inside the sliding window (pages before it are still visited,
  // their keys masked: the fp32 path serves short requests).
  const int win_lo = p.window_left >= 0 ? len - 1 - p.window_left : 0;

  // Pages of this wave: first, first + NW, first + 2 NW, ...  A split holds
  // at most 64 * NW pages, so all of this wave's page ids fit in one VGPR
  // (lane j holds the j-th id) and are read before the loop; each page then
  // takes its id with readlane, with no scalar load in front of its K/V loads.
  const int first = pg_begin + wave;
  const int n_w = first < pg_end ? (pg_end - first + kNW - 1) / kNW : 0;
  const int ids = lane < n_w ? table[first + kNW * lane] : 0;

  struct Buf {
    S k[4], v[4];
    bool ok;
  };
  // Loads are issued unconditionally (an id outside the pool is replaced by
  // page 0 and the page is flagged) so that no branch separates a load from
  // its use and the load counters stay exact across the rotation below.
  auto fetch = [&](int i, Buf& bf) {
    int pid = __builtin_amdgcn_readlane(ids, i);
    bf.ok = (unsigned)pid < (unsigned)p.num_pages;
    pid = bf.ok ? pid : 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const size_t off = (size_t)pid * page_stride + (size_t)(grp * 4 + t) * row_stride + lane_off;
      bf.k[t].load(kbase + off);
      bf.v[t].load(vbase + off);
    }
  };
  auto compute = [&](int i, Buf& bf) {
    if (!bf.ok) {
      bad = true;
      return;
    }
    const int tok0 = (first + kNW * i) * kPage + grp * 4;
    float s[4][G];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool valid = tok0 + t < len && tok0 + t >= win_lo;
      if (!valid) bf.v[t].zero();   // poisoned tail slots must not reach o (0 * NaN)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float d = row16_sum(bf.k[t].dot(qs[g])) * p.scale_log2;
        s[t][g] = valid ? d : kNegInf;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mb = fmaxf(fmaxf(s[0][g], s[1][g]), fmaxf(s[2][g], s[3][g]));
      const float mn = fmaxf(m[g], mb);
      const float mu = mn == kNegInf ? 0.f : mn;
      const float alpha = exp2_fast(m[g] - mu);
      float pr[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) pr[t] = exp2_fast(s[t][g] - mu);
      l[g] = l[g] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
#pragma unroll
      for (int e = 0; e < VPL; ++e) {
        float acc = o[g][e] * alpha;
#pragma unroll
        for (int t = 0; t < 4; ++t) acc = __builtin_fmaf(pr[t], bf.v[t].elem(e), acc);
        o[g][e] = acc;
      }
      m[g] = mn;
    }
  };

  // Pages go in batches of NB: all loads of a batch are issued first, then its
  // pages are folded in order, so the next page's loads stay in flight while
  // one page is computed.  Inside a batch the fetch index is clamped to the
  // wave's last page (duplicate loads hit in cache and are never used).
  Buf bufs[NB];
  const int last = n_w - 1;
  for (int i = 0; i < n_w; i += NB) {
#pragma unroll
    for (int j = 0; j < NB; ++j) fetch(min(i + j, last), bufs[j]);
#pragma unroll
    for (int j = 0; j < NB; ++j)
      if (j == 0 || i + j < n_w) compute(i + j, bufs[j]);
  }

  // Merge the four 16-lane groups of the wave (lane ^ 16, then lane ^ 32,
  // by lane-swap instructions rather than LDS permutes).
  auto partner = [](float x, int mask) { return mask == 16 ? swap_rows16(x) : swap_halves(x); };
#pragma unroll
  for (int mask = 16; mask <= 32; mask <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mo = partner(m[g], mask);
      float lo = partner(l[g], mask);
      float mn = fmaxf(m[g], mo);
      float mu = mn == kNegInf ? 0.f : mn;
      float a = exp2_fast(m[g] - mu), ao = exp2_fast(mo - mu);
      l[g] = l[g] * a + lo * ao;
#pragma unroll
      for (int e = 0; e < VPL; ++e) o[g][e] = o[g][e] * a + partner(o[g][e], mask) * ao;
      m[g] = mn;
    }
  }

  // Merge the waves through LDS; each thread then finishes some (head, d) pairs.
  __shared__ float sm_o[kNW][G][D];
  __shared__ float sm_m[kNW][G], sm_l[kNW][G];
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < VPL; ++e) sm_o[wave][g][gl * VPL + e] = o[g][e];
      if (lane == 0) { sm_m[wave][g] = m[g]; sm_l[wave][g] = l[g]; }
    }
  }
  const bool any_bad = __syncthreads_or(bad);

  const bool final_write = ns == 1;
  const float qnan = __builtin_nanf("");
  for (int idx = threadIdx.x; idx < G * D; idx += kNW * 64) {
    const int g = idx / D, d = idx % D;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kNW; ++w) mx = fmaxf(mx, sm_m[w][g]);
    const float mu = mx == kNegInf ? 0.f : mx;
    float lsum = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float a = exp2_fast(sm_m[w][g] - mu);
      lsum += sm_l[w][g] * a;
      acc += sm_o[w][g][d] * a;
    }
    float val = lsum > 0.f ? acc / lsum : 0.f;
    float lse_nat = lsum > 0.f ? (mu + log2_fast(lsum)) * kLn2 : kNegInf;
    if (any_bad) { val = qnan; lse_nat = qnan; }
    const int h = kvh * G + g;
    if (final_write) {
      store_out(reinterpret_cast<T*>(p.out) + ((size_t)b * p.Hq + h) * D + d, val);
      if (d == 0) p.lse[(size_t)b * p.Hq + h] = lse_nat;
    } else {
      const size_t unit = ((size_t)b * p.n_splits + split) * p.Hq + h;
      p.part_o[unit * D + d] = val;
      if (d == 0) p.part_lse[unit] = lse_nat;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 / fp16 decode on the matrix cores with a balanced schedule.
//
// Schedule: the (request, KV head, page) units of the whole batch are laid
// out request by request, KV head by KV head, and cut into equal runs, one
// per wave of the grid, so every wave streams the same number of KV bytes
// whatever the spread of request lengths ("FlashInfer内核库深度解析": batched
// kernels balance load by sequence length; "FlashInfer Attention Kernel技术
// 解析" section 2.2: schedule by length).  The cut is computed on the device
// from kv_lens, so the host needs no copy of the lengths.  A run that covers a
// whole (request, KV head) pair writes the final output; otherwise each run
// writes a partial (o, lse) and decode_merge_kernel combines them.
//
// Per 16-token page, on the matrix cores:
//   S^T[16 tokens x 16 head slots] = K_page . Q^T  (v_mfma_f32_16x16x32_bf16;
//        A operand read straight from HBM, 16 bytes per lane; the G query
//        heads of the KV head fill the first G of the 16 columns)
//   online softmax per column (each lane owns one head and four tokens)
//   O^T[16 d x 16 heads] += V^T . P^T            (v_mfma_f32_16x16x16_bf16;
//        V rows go through a per-wave LDS buffer and come back as V^T
//        fragments via ds_read_b64_tr_b16; P^T is the S^T accumulator as is)
// so per page only a few dozen vector instructions remain and the kernel is
// bound by HBM.  Pages are loaded in batches of NB per wave.
//
// With an 8-bit E4M3 cache (F8) the same schedule streams half the bytes:
// each lane loads 16-byte chunks of K (two k-steps' worth; the head
// dimension is permuted identically in Q and K so that a chunk is
// contiguous in memory) and of V, and converts them exactly to the 16-bit
// type in registers (v_cvt_scalef32_pk_{bf16,f16}_fp8) before the MFMAs and
// the LDS transpose.  The key scale is folded into the softmax exponent's
// scale on the host and the value scale into the final normalisation
// ("FlashAttention-3 ..." section 一: with FP8 the quantisation scale joins
// the exponent scaling instead of costing a separate pass).
template <int D>
struct MfmaDecodeCfg {
  static constexpr int KS = D / 32;          // 16x16x32 k-steps for Q.K
  static constexpr int CHV = D / 8;          // 16-byte chunks per V row
  static constexpr int LV = 16 * CHV / 64;   // V chunks per lane per page
  static constexpr int DB = D / 16;          // 16-row blocks of O^T
  static constexpr int ROWB = D * 2;         // bytes per V row in LDS
  static constexpr int UMASK = (D / 16 < 8 ? D / 16 : 8) - 1;  // swizzle of 32-byte units
  static constexpr int PAGEB = 16 * ROWB;    // LDS bytes of one page of V
};

// Byte offset in a page's V buffer of d-element `d` (multiple of 4) of row t:
// 32-byte units XOR (t mod 8) so the 16 rows of a transposing read spread over banks.
template <int D>
__device__ __forceinline__ int vpage_off(int t, int d) {
  using C = MfmaDecodeCfg<D>;
  return t * C::ROWB + ((((d >> 4) ^ (t & C::UMASK)) << 5) | ((d & 15) << 1));
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

// First page holding a key inside the sliding window (0 without one).
__device__ __forceinline__ int window_page0(const DecodeParams& p, int len) {
  const int lo = p.window_left >= 0 ? len - 1 - p.window_left : 0;
  return lo > 0 ? lo / kPage : 0;
}

// Pages of a request of `len` tokens that hold keys the query sees (the
// schedule's units), and the same for request b.
__device__ __forceinline__ int pages_from_len(const DecodeParams& p, int len) {
  return (len + kPage - 1) / kPage - window_page0(p, len);
}
__device__ __forceinline__ int pages_of(const DecodeParams& p, int b) {
  bool bad;
  return pages_from_len(p, request_len(p, b, bad));
}

__device__ __forceinline__ int wave_incl_scan(int x) {
  // Within each row of 16 lanes: DPP row_shr 1, 2, 4, 8 (a lane whose source
  // falls outside the row adds 0); then the totals of the rows before.
  // Called with all 64 lanes active (DPP reads inactive lanes' stale values).
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);
  const int lane = __lane_id();
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  return x + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// Units (pages x KV-head groups) of the whole batch.  For the first 64
// requests the lane's length (-1 for an inconsistent one) and the inclusive
// scan of units stay in len0 / incl0, so the run that follows finds its
// request without reading the lengths again.  With `publish` (one wave of
// the grid) the first unit of every request and the total go to
// p.unit_start for the merge kernel.
__device__ __forceinline__ int total_units(const DecodeParams& p, int& len0, int& incl0,
                                           bool publish) {
  int tot = 0;
  len0 = 0;
  incl0 = 0;
  for (int c = 0; c < p.B; c += 64) {
    const int b = c + __lane_id();
    bool bd = false;
    const int ln = b < p.B ? request_len(p, b, bd) : 0;
    const int u = b < p.B ? pages_from_len(p, ln) * p.nhg : 0;
    const int incl = wave_incl_scan(u);
    if (c == 0) {
      len0 = bd ? -1 : ln;
      incl0 = incl;
    }
    if (publish && b < p.B) p.unit_start[b] = tot + incl - u;
    tot += __builtin_amdgcn_readlane(incl, 63);
  }
  if (publish && __lane_id() == 0) p.unit_start[p.B] = tot;
  return tot;
}

__device__ __forceinline__ int run_length(const DecodeParams& p, int units) {
  if (p.split_pages > 0) return p.split_pages;
  const int w = (units + p.n_groups - 1) / p.n_groups;
  return w > p.min_run ? w : p.min_run;
}

// Per-wave LDS buffer for one page of V rows.
template <int D>
__device__ __forceinline__ char* decode_vbuf(int wave) {
  __shared__ __attribute__((aligned(16))) char vbuf[kMaxGroupWaves][MfmaDecodeCfg<D>::PAGEB];
  return vbuf[wave];
}

// Per-wave LDS buffer for one page of K rows as stored in the cache (ROWB
// bytes a row).
template <int D, int ROWB>
__device__ __forceinline__ char* decode_kbuf(int wave) {
  __shared__ __attribute__((aligned(16))) char kbuf[kMaxGroupWaves][kPage * ROWB];
  return kbuf[wave];
}

// Eight E4M3 bytes (two words) -> eight 16-bit elements, exactly.
template <typename H>
__device__ __forceinline__ typename H::v8 fp8x8(uint32_t w0, uint32_t w1) {
  const typename H::v2 a = H::template from_fp8x2<false>(w0), b = H::template from_fp8x2<true>(w0);
  const typename H::v2 c = H::template from_fp8x2<false>(w1), d = H::template from_fp8x2<true>(w1);
  return typename H::v8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// One run [u0, u1) of the balanced schedule.  A unit is one page of one
// group of hw KV heads; wave w of the workgroup folds KV head hg * hw + w of
// every unit, so a workgroup reads whole pages (all heads of a token are
// adjacent in the NHD layout).
template <typename E, int D, int G, int NB, bool F8, bool RP, bool LP>
__device__ __forceinline__ void decode_run(const DecodeParams& p, int u0, int u1, int W, int lane,
                                           int wave, int len0, int incl0) {
  static_assert(!(RP && F8), "rotary embedding on the 16-bit cache only");
  using C = MfmaDecodeCfg<D>;
  constexpr int GROWB = F8 ? D : 2 * D;                  // bytes of one K/V row in the cache
  constexpr int NK = F8 ? C::KS / 2 : C::KS;             // 16-byte K loads per lane per page
  constexpr int NV = F8 ? C::LV / 2 : C::LV;             // 16-byte V loads per lane per page
  constexpr int CHG = GROWB / 16;                        // 16-byte chunks per cache row
  using H = Half16<E>;
  using elem = typename H::elem;
  const int l16 = lane & 15, gq = lane >> 4;
  // Request holding unit u0 (scan of units per request, 64 requests at a
  // time; the first 64 come from total_units).  The lengths of the 64
  // requests from c_base on stay one per lane (lenv, -1 for an inconsistent
  // one), so later pieces read them without a memory round trip.
  int b = 0, start_b = 0, c_base = 0, lenv = 0;
  for (int c = 0, cum = 0; c < p.B; c += 64) {
    const int bb = c + lane;
    bool bd = false;
    int ln;
    if (c == 0) {
      bd = len0 < 0;
      ln = bd ? 0 : len0;
    } else {
      ln = bb < p.B ? request_len(p, bb, bd) : 0;
    }
    const int u = bb < p.B ? pages_from_len(p, ln) * p.nhg : 0;
    const int incl = c == 0 ? incl0 : wave_incl_scan(u);
    const int tot = __builtin_amdgcn_readlane(incl, 63);
    if (cum + tot > u0) {
      const uint64_t hit = __builtin_amdgcn_ballot_w64(cum + incl > u0);
      const int j = __builtin_ctzll(hit);
      b = c + j;
      start_b = cum + __builtin_amdgcn_readlane(incl, j) - __builtin_amdgcn_readlane(u, j);
      c_base = c;
      lenv = bd ? -1 : ln;
      break;
    }
    cum += tot;
  }
  auto len_of = [&](int bq) {
    const int i = bq - c_base;
    if (i >= 0 && i < 64) {
      const int v = __builtin_amdgcn_readlane(lenv, i);
      return v < 0 ? 0 : v;
    }
    bool bd;
    return request_len(p, bq, bd);
  };
  int np = pages_from_len(p, len_of(b));

  char* myv = decode_vbuf<D>(wave);
  // K rows also pass through LDS (except with the rotary embedding, which
  // rotates the fragments as loaded): each load instruction then covers
  // whole 128-byte lines of the cache (4 or more rows x the head's row
  // bytes) instead of half lines of 16 rows, which HBM serves faster
  // (main kernel 97.1 -> 94.9 us on the 576 MB batch).  The 16-byte chunks
  // of a row are XOR-swizzled by the row's 256-byte bank row so the 16 rows
  // read by one MFMA operand load hit distinct banks.
  constexpr bool KL = !RP;
  constexpr int RPB = 256 / GROWB > 0 ? 256 / GROWB : 1;  // K rows per 256 LDS bytes
  constexpr int SWM = (CHG < 16 ? CHG : 16) - 1;         // swizzle mask (chunks of a row)
  char* myk = KL ? decode_kbuf<D, GROWB>(wave) : nullptr;
  auto k_off = [&](int row, int chunk) { return row * GROWB + ((chunk ^ ((row / RPB) & SWM)) << 4); };
  const char* kbase = reinterpret_cast<const char*>(p.k_pages);
  const char* vbase = reinterpret_cast<const char*>(p.v_pages);
  // Bytes between consecutive tokens of one head, and per page (NHD
  // interleaves the heads of a token, HND keeps each head's 16 rows together).
  const size_t tok_b = p.kv_hnd ? (size_t)GROWB : (size_t)p.Hkv * GROWB;
  // 16-token blocks: block k of a request is block k mod m of page
  // table[k / m] (m = 1 << page_shift).  Lanes hold block ids: the index of
  // that block in the pool counted in strides of blk_b (NHD: page * m + sub;
  // HND: page * Hkv * m + sub, the head adding head_b), or -1 for an
  // out-of-range page id, so a page step costs what it does with 16-token pages.
  // With 16-token pages (!LP) a block id is the page id for both layouts.
  const size_t blk_b = (LP && p.kv_hnd) ? (size_t)kPage * GROWB : (size_t)kPage * p.Hkv * GROWB;
  const int shift = LP ? p.page_shift : 0;               // LP: pages of more than 16 tokens
  const size_t head_b = p.kv_hnd ? ((size_t)kPage << shift) * GROWB : (size_t)GROWB;
  const int blk_mask = (1 << shift) - 1;
  const int blk_per_page = LP ? (p.kv_hnd ? p.Hkv << shift : 1 << shift) : 1;
  // Lane value for block k of a table row: with 16-token pages the raw page
  // id (checked when the page is fetched), else the block id or -1.
  auto block_id = [&](const int32_t* row, int k) {
    if constexpr (!LP) return row[k];
    const int pid = row[k >> shift];
    return (unsigned)pid < (unsigned)p.num_pages ? pid * blk_per_page + (k & blk_mask) : -1;
  };
  const float c = p.scale_log2;
  const float qnan = __builtin_nanf("");

  struct Page {
    u32x4 k[NK], v[NV];
    bool ok;
  };

  // Q^T fragments: lane (head l16, k-group gq) holds q[head][32 ks + 8 gq .. +8]
  // (F8: q[head][64 (ks/2) + 16 gq + 8 (ks%2) .. +8], the order of its K chunks).
  auto load_q = [&](int bq, int kvq, typename H::v8 (&dst)[C::KS]) {
    const elem* qh = reinterpret_cast<const elem*>(p.q) +
                     ((size_t)bq * p.Hq + (size_t)kvq * G + (l16 < G ? l16 : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int d0 = F8 ? 64 * (ks / 2) + 16 * gq + 8 * (ks % 2) : 32 * ks + 8 * gq;
      const typename H::v8 v = *reinterpret_cast<const typename H::v8*>(qh + d0);
      dst[ks] = l16 < G ? v : typename H::v8{};
    }
  };
  typename H::v8 q_next[C::KS];
  int ids_next = 0, b_next = -1, hg_next = -1;

  int u = u0;
  while (u < u1) {
    while (u >= start_b + p.nhg * np) {       // next request with units
      start_b += p.nhg * np;
      ++b;
      np = pages_from_len(p, len_of(b));
    }
    const int r = u - start_b;
    const int hg = r / np, pg0 = r % np;
    const int start_pair = start_b + hg * np;
    const int n = min(u1, start_pair + np) - u;        // pages of this piece
    const int kvh = hg * p.hw + wave;
    if (kvh >= p.Hkv) {                                // idle wave of a partial head group
      u += n;
      continue;
    }
    const bool whole = start_pair / W == (start_pair + np - 1) / W;
    // Valid tokens (clamped) and the window: the piece's pages are counted
    // from page p0, the first one the window reaches; keys before win_lo
    // (relative to p0's first token) are masked.
    const int len_b = len_of(b);
    const int p0 = window_page0(p, len_b);
    const int len = len_b - p0 * kPage;
    const int win_lo = p.window_left >= 0 ? len_b - 1 - p.window_left - p0 * kPage : 0;

    typename H::v8 qf[C::KS];
    // Page-table row of request b; this piece starts at block blk0.
    // (16-token pages: the row pointer starts at the piece's first page.)
    const int blk0 = p0 + pg0;
    const int32_t* table = p.page_table + (size_t)b * p.max_pages + (LP ? 0 : blk0);
    const int kb = LP ? blk0 : 0;
    int ids0;
    if (b == b_next && hg == hg_next) {        // prefetched during the previous piece
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) qf[ks] = q_next[ks];
      ids0 = ids_next;
    } else {
      load_q(b, kvh, qf);
      ids0 = lane < min(64, n) ? block_id(table, kb + lane) : 0;
    }
    // The next piece of the run starts at page 0 of the next (request, head
    // group) pair with units: fetch its query and first page ids now, so
    // they are in registers when this piece ends (head_dim 256 has no
    // registers to spare for it).
    if (D <= 128 && u + n < u1) {
      int bq = b, hq = hg + 1;
      if (hq >= p.nhg) {
        hq = 0;
        for (++bq; bq < p.B && pages_from_len(p, len_of(bq)) == 0; ++bq) {}
      }
      const int kvq = hq * p.hw + wave;
      if (bq < p.B && kvq < p.Hkv) {
        const int lq = len_of(bq);
        const int npq = pages_from_len(p, lq);
        load_q(bq, kvq, q_next);
        const int w0 = window_page0(p, lq);
        const int32_t* tq = p.page_table + (size_t)bq * p.max_pages + (LP ? 0 : w0);
        ids_next = lane < min(64, npq) ? block_id(tq, (LP ? w0 : 0) + lane) : 0;
        b_next = bq;
        hg_next = hq;
      }
    }
    // Rotary embedding: lane pair j = (k-step j / 8 < KS/2, element j % 8)
    // holds d = 32 (j / 8) + 8 gq + j % 8 in qf[j / 8] and d + D/2 in
    // qf[j / 8 + KS/2] (likewise for K), so each lane turns its own pairs.
    constexpr int NR = RP ? C::KS / 2 * 8 : 1;
    float rf[NR], rc[NR], rs[NR], tc[NR], ts[NR];
    if constexpr (RP) {
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const int d = 32 * (j / 8) + 8 * gq + j % 8;
        rf[j] = exp2f(-(float)(2 * d) / D * p.rope_log2_theta) * p.rope_inv_scale;
        float sq, cq;
        sincosf((float)(len_b - 1) * rf[j], &sq, &cq);
        const int ks = j / 8, e = j % 8;
        const float x = (float)qf[ks][e], y = (float)qf[ks + C::KS / 2][e];
        qf[ks][e] = (elem)(x * cq - y * sq);
        qf[ks + C::KS / 2][e] = (elem)(y * cq + x * sq);
        sincosf(16.f * rf[j], &ts[j], &tc[j]);      // one page further on
      }
    }
    f32x4 o[C::DB];
#pragma unroll
    for (int i = 0; i < C::DB; ++i) o[i] = f32x4{};
    float m = kNegInf, lsum = 0.f;
    bool bad = false;
    const char* kh = kbase + (size_t)kvh * head_b;
    const char* vh = vbase + (size_t)kvh * head_b;

    for (int c0 = 0; c0 < n; c0 += 64) {
      const int nc = min(64, n - c0);
      const int ids = c0 == 0 ? ids0 : lane < nc ? block_id(table, kb + c0 + lane) : 0;
      if constexpr (RP) {
        // Angle of this lane's key (token l16 of the page) at the first page of
        // the chunk, exact; later pages advance it by a 16-token rotation.
        const float pos = (float)((p0 + pg0 + c0) * kPage + l16);
#pragma unroll
        for (int j = 0; j < NR; ++j) sincosf(pos * rf[j], &rs[j], &rc[j]);
      }
      // Every K/V byte is read once: the loads carry the non-temporal hint so
      // the streamed pages do not displace cached lines as regular reads do
      // (main kernel 106-107 -> 97-98 us on the 576 MB batch).
      auto fetch = [&](int i, Page& pg) {
        int bid = __builtin_amdgcn_readlane(ids, i);
        pg.ok = LP ? bid >= 0 : (unsigned)bid < (unsigned)p.num_pages;
        bid = pg.ok ? bid : 0;
        const char* kp = kh + (size_t)bid * blk_b;
        const char* vp = vh + (size_t)bid * blk_b;
#pragma unroll
        for (int j = 0; j < NK; ++j) {
          if constexpr (KL) {
            const int ci = lane + 64 * j;                // row ci / CHG, chunk ci % CHG
            pg.k[j] = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(kp + (ci / CHG) * tok_b + (ci % CHG) * 16));
          } else {                                       // lane (l16, gq): its operand chunks
            const int off = F8 ? 64 * j + 16 * gq : (32 * j + 8 * gq) * 2;
            pg.k[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + l16 * tok_b + off));
          }
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int ci = lane + 64 * j;
          pg.v[j] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(vp + (ci / CHG) * tok_b + (ci % CHG) * 16));
        }
      };
      auto fold = [&](int i, Page& pg) {
        if (!pg.ok) {
          bad = true;
          return;
        }
        const int nval = len - (pg0 + c0 + i) * kPage;   // valid tokens in this page
        const int nlo = win_lo - (pg0 + c0 + i) * kPage;  // first one inside the window
        // V rows to LDS (rows past the end zeroed: poisoned slots must not reach O)
#pragma unroll
        for (int j = 0; j < NV; ++j) {
          const int ci = lane + 64 * j;
          const int t = ci / CHG, ch = ci % CHG;
          const u32x4 v = (t < nval && t >= nlo) ? pg.v[j] : u32x4{0u, 0u, 0u, 0u};
          if constexpr (F8) {
            // 16 bytes -> 16 elements, one 32-byte unit of the LDS row
            char* dst = myv + vpage_off<D>(t, ch * 16);
            *reinterpret_cast<typename H::v8*>(dst) = fp8x8<H>(v[0], v[1]);
            *reinterpret_cast<typename H::v8*>(dst + 16) = fp8x8<H>(v[2], v[3]);
          } else {
            *reinterpret_cast<u32x4*>(myv + vpage_off<D>(t, ch * 8)) = v;
          }
        }
        // K chunks in the MFMA operand order: lane (l16, gq) takes chunk
        // 4 j + gq of row l16 (bytes 64 j + 16 gq .. +16).
        u32x4 kc[NK];
        if constexpr (KL) {
#pragma unroll
          for (int j = 0; j < NK; ++j) {
            const int ci = lane + 64 * j;
            *reinterpret_cast<u32x4*>(myk + k_off(ci / CHG, ci % CHG)) = pg.k[j];
          }
#pragma unroll
          for (int j = 0; j < NK; ++j) kc[j] = *reinterpret_cast<const u32x4*>(myk + k_off(l16, 4 * j + gq));
        } else {
#pragma unroll
          for (int j = 0; j < NK; ++j) kc[j] = pg.k[j];
        }
        typename H::v8 kfr[C::KS];
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
          if constexpr (F8)
            kfr[ks] = ks % 2 == 0 ? fp8x8<H>(kc[ks / 2][0], kc[ks / 2][1])
                                  : fp8x8<H>(kc[ks / 2][2], kc[ks / 2][3]);
          else
            kfr[ks] = __builtin_bit_cast(typename H::v8, kc[ks]);
        }
        if constexpr (RP) {
#pragma unroll
          for (int j = 0; j < NR; ++j) {
            const int ks = j / 8, e = j % 8;
            const float x = (float)kfr[ks][e], y = (float)kfr[ks + C::KS / 2][e];
            kfr[ks][e] = (elem)(x * rc[j] - y * rs[j]);
            kfr[ks + C::KS / 2][e] = (elem)(y * rc[j] + x * rs[j]);
            const float c2 = rc[j] * tc[j] - rs[j] * ts[j];
            rs[j] = rs[j] * tc[j] + rc[j] * ts[j];
            rc[j] = c2;
          }
        }
        f32x4 s = {};
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) s = H::mfma16x16x32(kfr[ks], qf[ks], s);
        float mx = kNegInf;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float v = (4 * gq + rr < nval && 4 * gq + rr >= nlo) ? s[rr] * c : kNegInf;
          s[rr] = v;
          mx = fmaxf(mx, v);
        }
        mx = max_halves(max_rows16(mx));
        const float mn = fmaxf(m, mx);
        const float mu = mn == kNegInf ? 0.f : mn;
        const float alpha = exp2_fast(m - mu);
        m = mn;
        typename H::v4 pb;
        float ps = 0.f;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float e = exp2_fast(s[rr] - mu);
          ps += e;
          pb[rr] = (elem)e;
        }
        lsum = lsum * alpha + ps;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
          for (int db = 0; db < C::DB; ++db)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) o[db][rr] *= alpha;
        }
        const int t_rd = 4 * gq + (l16 >> 2);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)((lds_char*)myv + vpage_off<D>(t_rd, db * 16 + 4 * (l16 & 3))));
          o[db] = H::mfma16x16x16(__builtin_bit_cast(typename H::v4, a), pb, o[db]);
        }
      };
      const int last = nc - 1;
      if constexpr (F8) {
        // Software pipeline (an E4M3 page is half the bytes, so one page in
        // flight per wave leaves HBM idle): the loads of the next NB pages
        // are in flight while a page is folded.  Past the last page the
        // fetch repeats it (an L2 hit), so the count of loads in flight is
        // the same on every path.
        constexpr int DEP = NB + 1;
        Page ring[DEP];
#pragma unroll
        for (int j = 0; j < DEP - 1; ++j) fetch(min(j, last), ring[j]);
        for (int i = 0; i < nc; i += DEP) {
#pragma unroll
          for (int j = 0; j < DEP; ++j) {
            if (j == 0 || i + j < nc) {
              fetch(min(i + j + DEP - 1, last), ring[(j + DEP - 1) % DEP]);
              fold(i + j, ring[j]);
            }
          }
        }
      } else {
        Page bufs[NB];
        for (int i = 0; i < nc; i += NB) {
#pragma unroll
          for (int j = 0; j < NB; ++j) fetch(min(i + j, last), bufs[j]);
#pragma unroll
          for (int j = 0; j < NB; ++j)
            if (j == 0 || i + j < nc) fold(i + j, bufs[j]);
        }
      }
    }

    // Finish the piece: lane (head l16, group gq) holds d = 16 db + 4 gq + rr.
    const float ltot = sum_halves(sum_rows16(lsum));
    float inv = ltot > 0.f ? (F8 ? p.v_scale : 1.f) / ltot : 0.f;
    float lse_nat = ltot > 0.f ? (m + log2_fast(ltot)) * kLn2 : kNegInf;
    if (bad) { inv = qnan; lse_nat = qnan; }
    if (l16 < G) {
      const int h = kvh * G + l16;
      if (whole) {
        elem* og = reinterpret_cast<elem*>(p.out) + ((size_t)b * p.Hq + h) * D + 4 * gq;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          typename H::v4 v;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) v[rr] = (elem)(o[db][rr] * inv);
          *reinterpret_cast<typename H::v4*>(og + 16 * db) = v;
        }
        if (gq == 0) p.lse[(size_t)b * p.Hq + h] = lse_nat;
      } else {
        const size_t slot = ((size_t)b * p.Hkv + kvh) * p.max_segs + (u / W - start_pair / W);
        float* po = p.part_o + (slot * G + l16) * D + 4 * gq;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          f32x4 v;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) v[rr] = o[db][rr] * inv;
          *reinterpret_cast<f32x4*>(po + 16 * db) = v;
        }
        if (gq == 0) p.part_lse[slot * G + l16] = lse_nat;
      }
    }
    u += n;
  }
}

template <typename E, int D, int G, int NB, bool F8, bool RP, bool LP>
__global__ __launch_bounds__(kMaxGroupWaves * 64, D == 256 ? 1 : 2) void decode_mfma_kernel(DecodeParams p) {
  static_assert(G >= 1 && G <= 16, "one 16-column MFMA tile holds the query heads");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  int len0, incl0;
  const int U = total_units(p, len0, incl0, blockIdx.x == 0 && wave == 0);
  const int W = run_length(p, U);
  for (int run = blockIdx.x; (long)run * W < U; run += gridDim.x) {
    decode_run<E, D, G, NB, F8, RP, LP>(p, run * W, min(run * W + W, U), W, lane, wave, len0, incl0);
  }
}

// Merge of the balanced runs: one workgroup per (KV head, request) with S
// waves per query head of the group, wave sl folding the pair's segments
// sl, sl + S, ...; with S > 1 (a batch of a few long requests, each split
// over hundreds of runs) the S partial states of a head are combined
// through LDS.  The request's first unit and the batch's unit count come
// from unit_start, written by the main kernel.
// Lanes own d.  Pairs held by a single run were written by that run; empty
// requests get out 0 and lse -inf and inconsistent ones NaN.
// HPW query heads per workgroup: G (S waves each), or 1, the head then
// taken from blockIdx.z / DS; DS slices of d, the slice blockIdx.z % DS.
template <typename E, int D, int G, int S, int DS, int HPW>
__global__ __launch_bounds__(HPW * S * 64) void decode_merge_kernel(DecodeParams p) {
  static_assert(HPW == G || HPW == 1, "all heads of the group, or one");
  constexpr int DW = D / DS;                        // d of this workgroup
  constexpr int DL = DW / 64 > 0 ? DW / 64 : 1;
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int d0 = (blockIdx.z % DS) * DW;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = HPW == G ? wv / S : (int)blockIdx.z / DS, sl = wv % S;
  const bool lse_writer = blockIdx.z % DS == 0;
  const int h = kvh * G + g;
  const size_t slot0 = ((size_t)b * p.Hkv + kvh) * p.max_segs;
  const float* pl = p.part_lse + slot0 * G + g;           // stride G between segments
  const float* po = p.part_o + (slot0 * G + g) * D + d0;  // stride G*D between segments
  // This wave takes segments sl, sl + S, sl + 2S, ... (local segment js is
  // segment sl + S js).  Chunks of 64 local segments: lane j holds local
  // segment j0 + j's lse and weight, and the partial outputs are read MB
  // local segments at a time.  With S waves per head (a pair spanning many
  // runs) the first chunk's lse values and first batch of partial outputs
  // are requested before the segment count is known: every slot below
  // max_segs exists in the workspace, and values past the count are never
  // used (selected away, not multiplied by 0), so the lengths and the
  // partial states arrive in the same memory round trip (single request of
  // 32768 keys: merge 6.1 -> 5.5 us).  With one wave per head the pairs
  // span a few runs and most slots past the count were never written: the
  // same early loads made the merge slower there (5.3 -> 5.9 us, 64
  // requests), so that path loads after the count.
  constexpr int MB = D > 128 ? 16 : 32;
  constexpr int SPEC = S > 1 ? MB : 0;
  const int n_slot = p.max_segs > sl ? (p.max_segs - sl + S - 1) / S : 0;
  float v[MB][DL];
  auto load_o = [&](int js, int lim) {
#pragma unroll
    for (int t = 0; t < MB; ++t)
#pragma unroll
      for (int i = 0; i < DL; ++i)
        v[t][i] = (js + t < lim && lane + 64 * i < DW) ? po[(size_t)(sl + S * (js + t)) * G * D + lane + 64 * i] : 0.f;
  };
  float ls_first = kNegInf;
  if constexpr (SPEC > 0) {
    ls_first = lane < n_slot ? pl[(size_t)(sl + S * lane) * G] : kNegInf;
    load_o(0, min(SPEC, n_slot));
  }

  // The batch's unit count and request b's first unit, as the main kernel
  // counted them (no scan of the lengths here).
  const int U = p.unit_start[p.B], pre = p.unit_start[b];
  const int W = run_length(p, U);
  bool bad;
  request_len(p, b, bad);
  const int np = pages_of(p, b);
  const int start_pair = pre + (kvh / p.hw) * np;
  const int nseg = np > 0 ? (start_pair + np - 1) / W - start_pair / W + 1 : 0;
  if (nseg == 1) return;                 // the same for every wave of the workgroup
  E* og = reinterpret_cast<E*>(p.out) + ((size_t)b * p.Hq + h) * D + d0;
  if (bad || nseg == 0) {
    if (sl == 0) {
      const float val = bad ? __builtin_nanf("") : 0.f;
      for (int d = lane; d < DW; d += 64) store_out(og + d, val);
      if (lane == 0 && lse_writer) p.lse[(size_t)b * p.Hq + h] = bad ? val : kNegInf;
    }
    return;
  }
  const int n_loc = nseg > sl ? (nseg - sl + S - 1) / S : 0;   // local segments of this wave
  float acc[DL] = {};
  float mx = kNegInf, ws = 0.f;
  bool nan_seen = false;
  for (int j0 = 0; j0 < n_loc; j0 += 64) {
    const int nj = min(64, n_loc - j0);
    const bool early = SPEC > 0 && j0 == 0;       // lse and first batch requested above
    float ls = ls_first;
    if (!early) ls = lane < nj ? pl[(size_t)(sl + S * (j0 + lane)) * G] : kNegInf;
    ls = lane < nj ? ls : kNegInf;
    nan_seen |= __builtin_amdgcn_ballot_w64(ls != ls) != 0;
    const float mnew = fmaxf(mx, wave_max(ls));
    const float mu = mnew == kNegInf ? 0.f : mnew;
    const float resc = exp2_fast((mx - mu) * kLog2e);
    const float w = lane < nj ? exp2_fast((ls - mu) * kLog2e) : 0.f;
    ws = ws * resc + wave_sum(w);
#pragma unroll
    for (int i = 0; i < DL; ++i) acc[i] *= resc;
    mx = mnew;
    for (int j = 0; j < nj; j += MB) {
      if (!early || j > 0) load_o(j0 + j, n_loc);
#pragma unroll
      for (int t = 0; t < MB; ++t) {
        const float wt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), min(j + t, 63)));
#pragma unroll
        for (int i = 0; i < DL; ++i) acc[i] += j + t < nj ? wt * v[t][i] : 0.f;
      }
    }
  }
  const int gs = HPW == G ? g : 0;        // this head's first wave slot in the workgroup
  if constexpr (S == 1) {
    const float mu = mx == kNegInf ? 0.f : mx;
    const float inv = ws > 0.f ? 1.f / ws : 0.f;
    float lse_nat = ws > 0.f ? mu + log2_fast(ws) * kLn2 : kNegInf;
    if (nan_seen) lse_nat = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < DL; ++i)
      if (lane + 64 * i < DW) store_out(og + lane + 64 * i, nan_seen ? lse_nat : acc[i] * inv);
    if (lane == 0 && lse_writer) p.lse[(size_t)b * p.Hq + h] = lse_nat;
    return;
  }
  // Combine the S slices of each head: weights e^(mx_s - M) over the slices'
  // maxima M; an empty slice (mx -inf, ws 0, acc 0) adds nothing.
  __shared__ float sh_acc[16][DW];
  __shared__ float sh_mx[16], sh_ws[16];
  __shared__ int sh_nan[16];
#pragma unroll
  for (int i = 0; i < DL; ++i)
    if (lane + 64 * i < DW) sh_acc[wv][lane + 64 * i] = acc[i];
  if (lane == 0) {
    sh_mx[wv] = mx;
    sh_ws[wv] = ws;
    sh_nan[wv] = nan_seen ? 1 : 0;
  }
  __syncthreads();
  if (sl != 0) return;
  float M = kNegInf;
  bool any_nan = false;
#pragma unroll
  for (int k = 0; k < S; ++k) {
    M = fmaxf(M, sh_mx[gs * S + k]);
    any_nan |= sh_nan[gs * S + k] != 0;
  }
  const float mu = M == kNegInf ? 0.f : M;
  float wtot = 0.f, tot[DL] = {};
#pragma unroll
  for (int k = 0; k < S; ++k) {
    const float f = exp2_fast((sh_mx[gs * S + k] - mu) * kLog2e);
    wtot += f * sh_ws[gs * S + k];
#pragma unroll
    for (int i = 0; i < DL; ++i)
      if (lane + 64 * i < DW) tot[i] += f * sh_acc[gs * S + k][lane + 64 * i];
  }
  const float inv = wtot > 0.f ? 1.f / wtot : 0.f;
  float lse_nat = wtot > 0.f ? mu + log2_fast(wtot) * kLn2 : kNegInf;
  if (any_nan) lse_nat = __builtin_nanf("");
#pragma unroll
  for (int i = 0; i < DL; ++i)
    if (lane + 64 * i < DW) store_out(og + lane + 64 * i, any_nan ? lse_nat : tot[i] * inv);
  if (lane == 0 && lse_writer) p.lse[(size_t)b * p.Hq + h] = lse_nat;
}

// One thread per (head, d); requests with a single split were finished above.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeParams p) {
  constexpr int HPB = 256 / D;   // heads per block
  const int b = blockIdx.y;
  const int h = blockIdx.x * HPB + threadIdx.x / D;
  const int d = threadIdx.x % D;
  if (h >= p.Hq) return;
  bool bad;
  const int len = request_len(p, b, bad);
  const int ns = splits_of(len, p.split_pages);
  if (ns <= 1) return;
  const size_t base = (size_t)b * p.n_splits * p.Hq + h;
  float mx = kNegInf;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, p.part_lse[base + (size_t)s * p.Hq]);
  const float mu = mx == kNegInf ? 0.f : mx;
  float wsum = 0.f, acc = 0.f;
  bool nan_seen = false;
  for (int s = 0; s < ns; ++s) {
    const float ls = p.part_lse[base + (size_t)s * p.Hq];
    nan_seen |= ls != ls;
    const float w = exp2_fast((ls - mu) * kLog2e);
    wsum += w;
    acc += w * p.part_o[(base + (size_t)s * p.Hq) * D + d];
  }
  float val = wsum > 0.f ? acc / wsum : 0.f;
  float lse_nat = wsum > 0.f ? mu + log2_fast(wsum) * kLn2 : kNegInf;
  if (nan_seen) { val = __builtin_nanf(""); lse_nat = val; }
  store_out(reinterpret_cast<T*>(p.out) + ((size_t)b * p.Hq + h) * D + d, val);
  if (d == 0) p.lse[(size_t)b * p.Hq + h] = lse_nat;
}

template <typename T, int D, int G>
hipError_t launch_split_t(const DecodeParams& p, bool fp8, bool rope, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    // Pages of 16 tokens take instances without the block arithmetic.
    auto go = [&](auto lp) {
      constexpr bool LP = decltype(lp)::value;
      if (fp8)
        hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, (D == 256 ? 1 : kFp8Batch), true, false, LP>),
                           dim3(p.n_groups), dim3(p.hw * 64), 0, s, p);
      else if (rope) {
        if constexpr (D <= 128)
          hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, kMfmaBatch, false, true, LP>),
                             dim3(p.n_groups), dim3(p.hw * 64), 0, s, p);
        else
          return hipErrorInvalidValue;
      } else
        hipLaunchKernelGGL((decode_mfma_kernel<T, D, G, (D == 256 ? 1 : kMfmaBatch), false, false, LP>),
                           dim3(p.n_groups), dim3(p.hw * 64), 0, s, p);
      return hipSuccess;
    };
    const hipError_t e = p.page_shift > 0 ? go(std::true_type{}) : go(std::false_type{});
    if (e != hipSuccess) return e;
  } else {
    if (fp8 || rope) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_split_kernel<T, D, G, kBatch>), dim3(p.n_splits, p.Hkv, p.B),
                       dim3(kNW * 64), 0, s, p);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_split_g(const DecodeParams& p, int G, bool fp8, bool rope, hipStream_t s) {
  switch (G) {
    case 1: return launch_split_t<T, D, 1>(p, fp8, rope, s);
    case 2: return launch_split_t<T, D, 2>(p, fp8, rope, s);
    case 4: return launch_split_t<T, D, 4>(p, fp8, rope, s);
    case 8: return launch_split_t<T, D, 8>(p, fp8, rope, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_split_d(const DecodeParams& p, int D, int G, bool fp8, bool rope, hipStream_t s) {
  switch (D) {
    case 64: return launch_split_g<T, 64>(p, G, fp8, rope, s);
    case 128: return launch_split_g<T, 128>(p, G, fp8, rope, s);
    case 256:
      if constexpr (sizeof(T) == 2) return launch_split_g<T, 256>(p, G, fp8, rope, s);
      break;
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t launch_combine_t(const DecodeParams& p, hipStream_t s) {
  constexpr int HPB = 256 / D;
  dim3 grid((p.Hq + HPB - 1) / HPB, p.B);
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template <typename E, int D, int G>
void launch_merge_gs(const DecodeParams& p, hipStream_t s) {
  // Segment-parallel merge (16 waves) when a pair is expected to span more
  // than 64 runs, i.e. fewer than one (request, head group) per 64 workgroups.
  // That case gives each query head and each 64 d of it a workgroup of 16
  // waves, so a pair's hundreds of partial states are read by G * D / 64
  // CUs, 16 segments or fewer per wave (one memory round trip).
  if ((long)p.B * p.nhg * 64 < p.n_groups) {
    constexpr int DS = D / 64 > 0 ? D / 64 : 1;
    hipLaunchKernelGGL((decode_merge_kernel<E, D, G, 16, DS, 1>), dim3(p.Hkv, p.B, G * DS), dim3(1024),
                       0, s, p);
  } else {
    hipLaunchKernelGGL((decode_merge_kernel<E, D, G, 1, 1, G>), dim3(p.Hkv, p.B), dim3(G * 64), 0, s, p);
  }
}

template <typename E, int D>
hipError_t launch_merge_g(const DecodeParams& p, int G, hipStream_t s) {
  switch (G) {
    case 1: launch_merge_gs<E, D, 1>(p, s); break;
    case 2: launch_merge_gs<E, D, 2>(p, s); break;
    case 4: launch_merge_gs<E, D, 4>(p, s); break;
    case 8: launch_merge_gs<E, D, 8>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool decode_supported(int dtype, int D, int G, int page_size) {
  const bool d_ok = (dtype == 1 || dtype == 2) ? (D == 64 || D == 128 || D == 256)
                                                : (dtype == 0 && (D == 64 || D == 128));
  // 16-bit paths: pages of 16, 32, ..., 256 tokens; fp32: 16.
  const bool p_ok = page_size == kPage ||
                    (dtype != 0 && page_size <= 16 * kPage && page_size % kPage == 0 &&
                     ((page_size / kPage) & (page_size / kPage - 1)) == 0);
  return d_ok && (G == 1 || G == 2 || G == 4 || G == 8) && p_ok;
}

hipError_t launch_decode_split(const DecodeParams& p, int dtype, int D, int G, bool fp8_kv,
                               bool rope, hipStream_t s) {
  if (dtype == 0)
    return (fp8_kv || rope) ? hipErrorInvalidValue : launch_split_d<float>(p, D, G, false, false, s);
  return dtype == 1 ? launch_split_d<bf16_t>(p, D, G, fp8_kv, rope, s)
                    : launch_split_d<f16_t>(p, D, G, fp8_kv, rope, s);
}

// Partial decode states of attn_decode_paged_noalloc, for callers that
// cannot allocate device memory.  Each GPU the library runs on holds its own
// copy until the process ends; every call on a GPU shares it, so calls that
// overlap on one GPU race.  The decode kernels need no particular contents on
// entry (every slot they read was written earlier in the same call).
static __device__ __align__(256) char scratch[ATTN_DECODE_NOALLOC_SCRATCH_BYTES];

hipError_t decode_scratch(void** ptr, size_t* bytes) {
  // In host code `scratch` names a host-side stand-in: kernels get the device
  // address hipGetSymbolAddress returns, kept per device (racing first calls
  // store the same value).
  static std::atomic<void*> cache[64] = {};
  *bytes = sizeof(scratch);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) {
    void* c = cache[dev].load(std::memory_order_acquire);
    if (c != nullptr) {
      *ptr = c;
      return hipSuccess;
    }
  }
  void* a = nullptr;
  e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64) cache[dev].store(a, std::memory_order_release);
  *ptr = a;
  return hipSuccess;
}

hipError_t launch_decode_combine(const DecodeParams& p, int dtype, int D, int G, hipStream_t s) {
  if (dtype == 0) {
    if (D == 64) return launch_combine_t<float, 64>(p, s);
    if (D == 128) return launch_combine_t<float, 128>(p, s);
    return hipErrorInvalidValue;
  }
  if (dtype == 2) {
    if (D == 64) return launch_merge_g<f16_t, 64>(p, G, s);
    if (D == 128) return launch_merge_g<f16_t, 128>(p, G, s);
    if (D == 256) return launch_merge_g<f16_t, 256>(p, G, s);
    return hipErrorInvalidValue;
  }
  if (D == 64) return launch_merge_g<bf16_t, 64>(p, G, s);
  if (D == 128) return launch_merge_g<bf16_t, 128>(p, G, s);
  if (D == 256) return launch_merge_g<bf16_t, 256>(p, G, s);
  return hipErrorInvalidValue;
}

}  // namespace attn
