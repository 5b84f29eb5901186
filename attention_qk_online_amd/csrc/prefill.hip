// Ragged causal prefill for gfx950 on bf16 MFMA with fp32 accumulation.
//
// One workgroup = one (query tile of BM = 128 rows, query head) of one
// sequence; four waves own 32 query rows each.  Per key tile of BN = 64:
//   1. K[BN, D] and V^T[D, BN] are staged in LDS (V is transposed on the way
//      in so both MFMA operands read contiguous k-slices); the next tile's
//      global loads are issued into registers before the current tile is
//      computed, so HBM latency hides behind MFMA work.
//   2. S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: Q stays in VGPRs for the
//      whole loop (B operand), K comes from LDS (A operand).  The transposed
//      product puts one query per lane column, so a row max over keys is an
//      in-lane reduction plus one lane^32 exchange.
//   3. Causal/tail mask only on tiles that cross the diagonal or the end of
//      the keys; online softmax in log2 units (running max m, running sum l,
//      O rescaled by 2^(m_old - m_new) only when some row's max moved).
//   4. O^T += V^T . P^T on MFMA: the S^T accumulator is already laid out as
//      the B operand of this product (keys are permuted consistently on both
//      operands), so P never leaves registers.
// Tiles wholly above the causal diagonal are never loaded.  The score
// matrix never reaches memory.
//
// This follows the tiled, fused scheme of "FlashAttention-3 内核在最新大模型
// 推理中的集成实践" (section 一: Q/K/V blocks in on-chip memory, online softmax
// accumulated in place; section 二: varlen packing by cu_seqlens, causal,
// paged blocks; section 四: keep the rescaling, and keep tiles within the
// on-chip budget for head_dim 256) and the three-stage QK^T / softmax / PV
// pipeline of "FlashInfer Attention Kernel技术解析" section 1.3, re-tiled for
// 64-wide waves, 32x32 MFMA tiles and a 160 KiB LDS.
#include "common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int BM = kPrefillBM;   // query rows per workgroup
constexpr int BN = 64;           // keys per tile
constexpr int NWAVE = 4;
constexpr int NT = NWAVE * 64;
constexpr int kPage = 16;

template <int D>
struct Cfg {
  static constexpr int KSTR = D + 8;                 // K row stride in LDS (bf16), padded
  static constexpr int VSTR = BN + 8;                // V^T row stride in LDS (bf16), padded
  static constexpr int K_PER_THREAD = BN * D / 8 / NT;      // 16-byte chunks
  static constexpr int V_PER_THREAD = (BN / 4) * (D / 4) / NT;  // 4x4 blocks
  static constexpr int QK = D / 16;                  // MFMA k-steps over D
  static constexpr int DB = D / 32;                  // 32-row blocks of D in O^T
  static_assert(BN * D / 8 % NT == 0 && (BN / 4) * (D / 4) % NT == 0, "tile split");
  static constexpr int LDS_BYTES = (BN * KSTR + D * VSTR) * 2;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, bool PAGED>
__global__ __launch_bounds__(NT) void prefill_kernel(PrefillParams p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sK[BN * C::KSTR];
  __shared__ __attribute__((aligned(16))) __bf16 sVt[D * C::VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;

  // Heads that share a KV head land on the same XCD (workgroups are dealt
  // round-robin over the 8 XCDs, each with its own L2).
  const int x = blockIdx.x;
  const int head = (p.Hq % 8 == 0) ? (x % 8) * (p.Hq / 8) + x / 8 : x;
  const int kvh = head / (p.Hq / p.Hkv);
  const int b = blockIdx.y;
  const int tile = p.q_tiles - 1 - (int)blockIdx.z;   // heaviest causal tiles first

  // Sequence extents, clamped so every access stays inside the tensors.
  int q_start = min(max(p.cu_q[b], 0), p.total_q);
  int q_end = min(max(p.cu_q[b + 1], q_start), p.total_q);
  const int Lq = q_end - q_start;
  const int r0 = tile * BM;
  if (r0 >= Lq) return;
  bool bad = Lq > p.max_seqlen_q;
  int k_start = 0, Lk;
  const int32_t* table = nullptr;
  if constexpr (PAGED) {
    Lk = p.kv_lens[b];
    if (Lk < 0 || Lk > p.max_pages * kPage) { bad = true; Lk = 0; }
    table = p.page_table + (size_t)b * p.max_pages;
  } else {
    k_start = min(max(p.cu_k[b], 0), p.total_k);
    const int k_end = min(max(p.cu_k[b + 1], k_start), p.total_k);
    Lk = k_end - k_start;
  }
  const int off = Lk - Lq;                       // bottom-right causal offset
  const int r_last = min(r0 + BM, Lq) - 1;
  int kend = p.causal ? min(Lk, r_last + off + 1) : Lk;
  if (kend < 0) kend = 0;
  const int n_kt = (kend + BN - 1) / BN;

  const __bf16* qg = reinterpret_cast<const __bf16*>(p.q);
  const __bf16* kg = reinterpret_cast<const __bf16*>(p.k);
  const __bf16* vg = reinterpret_cast<const __bf16*>(p.v);
  const size_t kv_row = (size_t)p.Hkv * D;       // elements between consecutive tokens

  // Address of key `kj` (0 <= kj < Lk) of this sequence for our KV head.
  auto key_row = [&](int kj, bool& ok) -> size_t {
    if constexpr (PAGED) {
      const int pid = table[kj >> 4];
      ok = (unsigned)pid < (unsigned)p.num_pages;
      return ok ? (((size_t)pid * kPage + (kj & 15)) * kv_row + (size_t)kvh * D) : 0;
    } else {
      ok = true;
      return (size_t)(k_start + kj) * kv_row + (size_t)kvh * D;
    }
  };

  // ---- Q fragments (B operand of S^T = K Q^T): row l32 of this wave's 32 rows.
  const int my_row = r0 + wave * 32 + l32;
  const bool row_ok = my_row < Lq;
  bf16x8 qf[C::QK];
  {
    const __bf16* qr = qg + ((size_t)(q_start + (row_ok ? my_row : 0)) * p.Hq + head) * D + hl * 8;
#pragma unroll
    for (int s = 0; s < C::QK; ++s) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qr + s * 16);
      qf[s] = row_ok ? v : bf16x8{};
    }
  }

  // ---- register staging of the next K/V tile
  u32x4 kreg[C::K_PER_THREAD];
  u32x2 vreg[C::V_PER_THREAD][4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int r = 0; r < C::K_PER_THREAD; ++r) {
      const int c = tid + NT * r;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int kj = k0 + row;
      bool ok = false;
      size_t a = 0;
      if (kj < Lk) a = key_row(kj, ok);
      if (kj < Lk && !ok) bad = true;
      kreg[r] = ok ? *reinterpret_cast<const u32x4*>(kg + a + col) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < C::V_PER_THREAD; ++r) {
      const int bi = tid + NT * r;
      const int dg = bi % (D / 4), kgp = bi / (D / 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kj = k0 + kgp * 4 + i;
        bool ok = false;
        size_t a = 0;
        if (kj < Lk) a = key_row(kj, ok);
        if (kj < Lk && !ok) bad = true;
        vreg[r][i] = ok ? *reinterpret_cast<const u32x2*>(vg + a + dg * 4) : u32x2{0u, 0u};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < C::K_PER_THREAD; ++r) {
      const int c = tid + NT * r;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *reinterpret_cast<u32x4*>(&sK[row * C::KSTR + col]) = kreg[r];
    }
#pragma unroll
    for (int r = 0; r < C::V_PER_THREAD; ++r) {
      const int bi = tid + NT * r;
      const int dg = bi % (D / 4), kgp = bi / (D / 4);
      // 4 keys x 4 dims -> 4 dims x 4 keys (bf16 transpose in registers)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int w = j >> 1;
        const bool hi = j & 1;
        uint32_t e0 = hi ? (vreg[r][0][w] >> 16) : (vreg[r][0][w] & 0xffffu);
        uint32_t e1 = hi ? (vreg[r][1][w] >> 16) : (vreg[r][1][w] & 0xffffu);
        uint32_t e2 = hi ? (vreg[r][2][w] >> 16) : (vreg[r][2][w] & 0xffffu);
        uint32_t e3 = hi ? (vreg[r][3][w] >> 16) : (vreg[r][3][w] & 0xffffu);
        u32x2 t = {e0 | (e1 << 16), e2 | (e3 << 16)};
        *reinterpret_cast<u32x2*>(&sVt[(dg * 4 + j) * C::VSTR + kgp * 4]) = t;
      }
    }
  };

  f32x16 o[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) o[i] = f32x16{};
  float m = kNegInf, lsum = 0.f;
  const float c = p.scale_log2;

  const int w_first = r0 + wave * 32;                       // first row of this wave
  const int w_last = min(w_first + 31, Lq - 1);
  const bool wave_rows = w_first < Lq;

  if (n_kt > 0) load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(k0 + BN);

    const bool wave_sees = wave_rows && (!p.causal || k0 <= w_last + off);
    if (!wave_sees) continue;

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const __bf16* kr = &sK[(kb * 32 + l32) * C::KSTR + hl * 8];
#pragma unroll
      for (int ks = 0; ks < C::QK; ++ks)
        s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(kr + ks * 16), qf[ks], s[kb]);
    }

    // scale to log2 units, mask where needed
    const bool need_mask = (k0 + BN > Lk) || (p.causal && k0 + BN - 1 > w_first + off);
    const int pos = my_row + off;   // last visible key index for this lane's query
    float t[2][16];
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[kb][r] * c;
        if (need_mask) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          if (key >= Lk || (p.causal && key > pos)) v = kNegInf;
        }
        t[kb][r] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = max_halves(mt);
    const float mn = fmaxf(m, mt);
    const float mu = mn == kNegInf ? 0.f : mn;
    const float alpha = exp2_fast(m - mu);
    m = mn;
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = exp2_fast(t[kb][half * 8 + e] - mu);
          psum += pe;
          v[e] = (__bf16)pe;
        }
        pb[kb * 2 + half] = v;
      }
    }
    lsum = lsum * alpha + psum;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const __bf16* vr = &sVt[(db * 32 + l32) * C::VSTR + hl * 4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x4 lo = *reinterpret_cast<const bf16x4*>(vr + ks * 16);
        bf16x4 hi = *reinterpret_cast<const bf16x4*>(vr + ks * 16 + 8);
        bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = mfma32(a, pb[ks], o[db]);
      }
    }
  }

  const bool any_bad = __syncthreads_or(bad);

  // ---- epilogue: O / l, LSE in natural log
  const float ltot = sum_halves(lsum);
  float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  float lse_v = ltot > 0.f ? (m + log2_fast(ltot)) * kLn2 : kNegInf;
  if (any_bad) {
    inv = __builtin_nanf("");
    lse_v = inv;
  }
  if (!row_ok) return;
  const size_t orow = (size_t)(q_start + my_row) * p.Hq + head;
  __bf16* og = reinterpret_cast<__bf16*>(p.out) + orow * D;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      bf16x4 v;
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (__bf16)(o[db][a4 * 4 + j] * inv);
      *reinterpret_cast<bf16x4*>(og + db * 32 + a4 * 8 + hl * 4) = v;
    }
  }
  if (hl == 0) p.lse[orow] = lse_v;
}

template <int D, bool PAGED>
hipError_t launch_t(const PrefillParams& p, hipStream_t s) {
  dim3 grid(p.Hq, p.B, p.q_tiles);
  hipLaunchKernelGGL((prefill_kernel<D, PAGED>), grid, dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool prefill_supported(int dtype, int D) { return dtype == 1 && (D == 128 || D == 256); }

hipError_t launch_prefill(const PrefillParams& p, int D, bool paged, hipStream_t s) {
  if (D == 128) return paged ? launch_t<128, true>(p, s) : launch_t<128, false>(p, s);
  if (D == 256) return paged ? launch_t<256, true>(p, s) : launch_t<256, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace attn
