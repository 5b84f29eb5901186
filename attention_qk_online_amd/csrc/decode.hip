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
#include "common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int kPage = 16;   // tokens per page handled by this kernel
constexpr int kNW = 4;      // waves per workgroup
#ifndef ATTN_DECODE_BATCH
#define ATTN_DECODE_BATCH 2
#endif
constexpr int kBatch = ATTN_DECODE_BATCH;  // pages whose loads are issued together

template <typename T, int D>
struct Slice {
  static constexpr int VPL = D / 16;                     // elements per lane
  static constexpr int WORDS = VPL * (int)sizeof(T) / 4; // 32-bit words per lane
  uint32_t w[WORDS];

  __device__ __forceinline__ void load(const T* row) {
    const char* p = reinterpret_cast<const char*>(row);
    if constexpr (WORDS % 4 == 0) {
#pragma unroll
      for (int i = 0; i < WORDS / 4; ++i) {
        u32x4 x = *reinterpret_cast<const u32x4*>(p + 16 * i);
        w[4 * i + 0] = x[0]; w[4 * i + 1] = x[1]; w[4 * i + 2] = x[2]; w[4 * i + 3] = x[3];
      }
    } else {
      static_assert(WORDS == 2, "slice of 8 bytes");
      u32x2 x = *reinterpret_cast<const u32x2*>(p);
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

// Number of valid tokens of request b after clamping inconsistent device data
// (negative, above max_kv_len or above the page table's capacity -> bad).
__device__ __forceinline__ int request_len(const DecodeParams& p, int b, bool& bad) {
  int kv = p.kv_lens[b];
  bad = kv < 0 || kv > p.max_kv_len || kv > p.max_pages * kPage;
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
  const size_t row_stride = (size_t)p.Hkv * D;            // elements between tokens
  const size_t lane_off = (size_t)kvh * D + gl * VPL;
  const int32_t* table = p.page_table + (size_t)b * p.max_pages;

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
      const size_t off = ((size_t)pid * kPage + grp * 4 + t) * row_stride + lane_off;
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
      const bool valid = tok0 + t < len;
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

  // Merge the four 16-lane groups of the wave (lane ^ 16, then lane ^ 32).
#pragma unroll
  for (int mask = 16; mask <= 32; mask <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mo = shfl_xor_f32(m[g], mask);
      float lo = shfl_xor_f32(l[g], mask);
      float mn = fmaxf(m[g], mo);
      float mu = mn == kNegInf ? 0.f : mn;
      float a = exp2_fast(m[g] - mu), ao = exp2_fast(mo - mu);
      l[g] = l[g] * a + lo * ao;
#pragma unroll
      for (int e = 0; e < VPL; ++e) o[g][e] = o[g][e] * a + shfl_xor_f32(o[g][e], mask) * ao;
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
hipError_t launch_split_t(const DecodeParams& p, hipStream_t s) {
  dim3 grid(p.n_splits, p.Hkv, p.B);
  hipLaunchKernelGGL((decode_split_kernel<T, D, G, kBatch>), grid, dim3(kNW * 64), 0, s, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_split_g(const DecodeParams& p, int G, hipStream_t s) {
  switch (G) {
    case 1: return launch_split_t<T, D, 1>(p, s);
    case 2: return launch_split_t<T, D, 2>(p, s);
    case 4: return launch_split_t<T, D, 4>(p, s);
    case 8: return launch_split_t<T, D, 8>(p, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_split_d(const DecodeParams& p, int D, int G, hipStream_t s) {
  switch (D) {
    case 64: return launch_split_g<T, 64>(p, G, s);
    case 128: return launch_split_g<T, 128>(p, G, s);
    case 256:
      if constexpr (sizeof(T) == 2) return launch_split_g<T, 256>(p, G, s);
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

template <typename T>
hipError_t launch_combine_d(const DecodeParams& p, int D, hipStream_t s) {
  switch (D) {
    case 64: return launch_combine_t<T, 64>(p, s);
    case 128: return launch_combine_t<T, 128>(p, s);
    case 256:
      if constexpr (sizeof(T) == 2) return launch_combine_t<T, 256>(p, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool decode_supported(int dtype, int D, int G, int page_size) {
  const bool d_ok = dtype == 1 ? (D == 64 || D == 128 || D == 256) : (dtype == 0 && D <= 128 &&
                                                                      (D == 64 || D == 128));
  return d_ok && (G == 1 || G == 2 || G == 4 || G == 8) && page_size == kPage;
}

hipError_t launch_decode_split(const DecodeParams& p, int dtype, int D, int G, hipStream_t s) {
  return dtype == 0 ? launch_split_d<float>(p, D, G, s) : launch_split_d<bf16_t>(p, D, G, s);
}

hipError_t launch_decode_combine(const DecodeParams& p, int dtype, int D, hipStream_t s) {
  return dtype == 0 ? launch_combine_d<float>(p, D, s) : launch_combine_d<bf16_t>(p, D, s);
}

}  // namespace attn
