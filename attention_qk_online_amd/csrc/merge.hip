// Log-sum-exp merge of two attention states over the same (row, head) grid.
//
// For one query row and head, a state (o, lse) is the softmax-weighted sum of
// V over some set of keys and the log of its normaliser.  The state over the
// union of two disjoint key sets follows from the two states alone: with
// m = max(lse_a, lse_b), w_x = exp(lse_x - m),
//   o = (w_a o_a + w_b o_b) / (w_a + w_b),   lse = m + ln(w_a + w_b).
// This is the aggregation step of the online softmax ("FlashAttention-3 内核
// 在最新大模型推理中的集成实践" section 一: partial results aggregated in
// place) applied to two finished partitions; it joins a shared-prefix pass to
// each request's own keys ("FlashInfer内核库深度解析", batch processing layer:
// reuse of a prefix common to several sequences).
//
// One thread per 8 consecutive elements of a row (16-byte loads for 16-bit
// types, two 16-byte loads for float); rows are (token, head) pairs.  An
// empty state (lse = -inf) has weight 0 and its o is not read; both empty
// gives o = 0, lse = -inf; a NaN lse on either side gives NaN.  A row's
// threads lie in one wave and read both lse values before any of them
// stores, so the outputs may overwrite either input in place.
#include "common.h"
#include "launch.h"

namespace attn {

namespace {

template <typename T>
struct Elem8;
template <>
struct Elem8<float> {
  typedef float v __attribute__((ext_vector_type(8)));
};
template <>
struct Elem8<bf16_t> {
  typedef __bf16 v __attribute__((ext_vector_type(8)));
};
template <>
struct Elem8<f16_t> {
  typedef _Float16 v __attribute__((ext_vector_type(8)));
};

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_states_kernel(const void* oa, const float* la,
                                                           const void* ob, const float* lb,
                                                           void* out, float* lse, long rows) {
  using V = typename Elem8<T>::v;
  constexpr int TPR = D / 8;                       // threads per row
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  const long row = t / TPR;
  const int c = (int)(t % TPR);
  if (row >= rows) return;
  const float xa = la[row], xb = lb[row];
  const float mx = fmaxf(xa, xb);
  const bool nan = xa != xa || xb != xb;
  const size_t off = (size_t)row * D + c * 8;
  V r;
  float lr;
  if (nan) {
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = __builtin_nanf("");
    lr = __builtin_nanf("");
  } else if (mx == kNegInf) {
    r = V{};
    lr = kNegInf;
  } else {
    const float wa = exp2_fast((xa - mx) * kLog2e), wb = exp2_fast((xb - mx) * kLog2e);
    const float inv = 1.f / (wa + wb);
    V va{}, vb{};
    if (wa > 0.f) va = *(reinterpret_cast<const V*>(oa) + off / 8);
    if (wb > 0.f) vb = *(reinterpret_cast<const V*>(ob) + off / 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (float(va[e]) * wa + float(vb[e]) * wb) * inv;
    lr = mx + log2_fast(wa + wb) * kLn2;
  }
  *(reinterpret_cast<V*>(out) + off / 8) = r;
  if (c == 0) lse[row] = lr;
}

template <typename T>
hipError_t launch_merge_t(const void* oa, const float* la, const void* ob, const float* lb,
                          void* out, float* lse, long rows, int D, hipStream_t s) {
  const long threads = rows * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  switch (D) {
    case 64: hipLaunchKernelGGL((merge_states_kernel<T, 64>), grid, dim3(256), 0, s, oa, la, ob, lb, out, lse, rows); break;
    case 128: hipLaunchKernelGGL((merge_states_kernel<T, 128>), grid, dim3(256), 0, s, oa, la, ob, lb, out, lse, rows); break;
    case 256: hipLaunchKernelGGL((merge_states_kernel<T, 256>), grid, dim3(256), 0, s, oa, la, ob, lb, out, lse, rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool merge_supported(int dtype, int D) { return dtype >= 0 && dtype <= 2 && (D == 64 || D == 128 || D == 256); }

hipError_t launch_merge_states(const void* oa, const float* la, const void* ob, const float* lb,
                               void* out, float* lse, long rows, int dtype, int D, hipStream_t s) {
  if (dtype == 0) return launch_merge_t<float>(oa, la, ob, lb, out, lse, rows, D, s);
  if (dtype == 1) return launch_merge_t<bf16_t>(oa, la, ob, lb, out, lse, rows, D, s);
  if (dtype == 2) return launch_merge_t<f16_t>(oa, la, ob, lb, out, lse, rows, D, s);
  return hipErrorInvalidValue;
}

}  // namespace attn
