// Ragged causal prefill for gfx950 on bf16 MFMA with fp32 accumulation.
//
// One workgroup = one (query tile of BM = 128 rows, query head) of one
// sequence; four waves own 32 query rows each, and two workgroups share a CU
// so that one wave's matrix work overlaps another's softmax.  Per key tile
// of BN keys (64 for head_dim 128, 32 for head_dim 256):
//   1. The tile's K and V rows were fetched into registers during the
//      previous tile and are written to one of two LDS stages (row-major,
//      XOR-swizzled so the reads below hit every bank once); the next tile's
//      global loads are issued right after, so HBM latency hides behind a
//      whole tile of MFMA work.  One barrier per tile.
//   2. S^T = K . Q^T on v_mfma_f32_32x32x16_bf16: Q stays in VGPRs for the
//      whole loop (B operand), K comes from LDS (A operand).  The transposed
//      product puts one query per lane column, so a row max over keys is an
//      in-lane reduction plus one lane^32 exchange.
//   3. Causal/tail mask only on tiles that cross the diagonal or the end of
//      the keys; online softmax in log2 units (running max m, running sum l,
//      O rescaled by 2^(m_old - m_new) only when some row's max moved).
//   4. O^T += V^T . P^T on MFMA: the S^T accumulator is already laid out as
//      the B operand (keys permuted identically on both operands), and V^T
//      fragments come from the row-major V tile through ds_read_b64_tr_b16.
// Tiles wholly above the causal diagonal are never loaded.  The score
// matrix never reaches memory.
//
// This follows the tiled, fused scheme of "FlashAttention-3 内核在最新大模型
// 推理中的集成实践" (section 一: Q/K/V blocks in on-chip memory, online softmax
// accumulated in place, loads overlapped with tensor-core work by double
// buffering; section 二: varlen packing by cu_seqlens, causal, paged blocks;
// section 四: keep the rescaling, and keep tiles within the on-chip budget for
// head_dim 256) and the three-stage QK^T / softmax / PV pipeline of "FlashInfer
// Attention Kernel技术解析" section 1.3 (bank-conflict avoidance: section 4),
// re-tiled for 64-wide waves, 32x32 MFMA tiles and a 160 KiB LDS.
#include "common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int BM = kPrefillBM;   // query rows per workgroup
constexpr int NWAVE = 4;
constexpr int NT = NWAVE * 64;
constexpr int kPage = 16;

template <int D>
struct Cfg {
  static constexpr int BN = D == 128 ? 64 : 32;      // keys per tile
  static constexpr int ROWB = D * 2;                  // bytes of one K/V row
  static constexpr int TILEB = BN * ROWB;             // bytes of one K or V tile
  static constexpr int STAGEB = 2 * TILEB;            // K + V
  static constexpr int CH = D / 8;                    // 16-byte chunks per row
  static constexpr int LOADS = BN * CH / NT;          // 16-byte chunks per thread (K or V)
  static constexpr int QK = D / 16;                   // MFMA k-steps over D
  static constexpr int DB = D / 32;                   // 32-row blocks of D in O^T
  static constexpr int KB = BN / 32;                  // 32-key blocks per tile
  static constexpr int PS = BN / 16;                  // 16-key k-steps of P.V
  static_assert(BN * CH % NT == 0, "tile split");
  static_assert(2 * STAGEB <= 80 * 1024, "two workgroups per CU");
};

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

// Byte offset of 16-byte chunk `c` of K row `r` in a K tile: chunk index
// XOR (r mod 16), so 16 consecutive rows read at the same logical chunk land
// in 16 different 16-byte bank groups.
template <int D>
__device__ __forceinline__ int k_off(int r, int c) {
  return r * Cfg<D>::ROWB + ((c ^ (r & 15)) << 4);
}
// Byte offset of 16-byte chunk `c` of V row `r`: its 64-byte block is XORed
// with (r mod 4), so the four rows that one 16-lane group of a transposing
// read touches fall in four different 64-byte bank groups.
template <int D>
__device__ __forceinline__ int v_off(int r, int c) {
  return r * Cfg<D>::ROWB + ((((c >> 2) ^ (r & 3)) << 2 | (c & 3)) << 4);
}

template <int D, bool PAGED>
__global__ __launch_bounds__(NT, D == 128 ? 2 : 1) void prefill_kernel(PrefillParams p) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGEB];

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
  const int q_start = min(max(p.cu_q[b], 0), p.total_q);
  const int q_end = min(max(p.cu_q[b + 1], q_start), p.total_q);
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
  const int n_kt = (kend + C::BN - 1) / C::BN;

  const __bf16* qg = reinterpret_cast<const __bf16*>(p.q);
  const char* kg = reinterpret_cast<const char*>(p.k);
  const char* vg = reinterpret_cast<const char*>(p.v);
  const size_t kv_rowb = (size_t)p.Hkv * C::ROWB;      // bytes between consecutive tokens

  // Byte address of key `kj` (clamped into [0, Lk)) for our KV head.  Keys past
  // the end reuse the last key's row: finite data that the mask zeroes out.
  auto key_addr = [&](int kj) -> size_t {
    kj = min(kj, Lk - 1);
    if constexpr (PAGED) {
      int pid = table[kj >> 4];
      if ((unsigned)pid >= (unsigned)p.num_pages) { bad = true; pid = 0; }
      return ((size_t)pid * kPage + (kj & 15)) * kv_rowb + (size_t)kvh * C::ROWB;
    } else {
      return (size_t)(k_start + kj) * kv_rowb + (size_t)kvh * C::ROWB;
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

  // ---- register staging of one K/V tile: thread owns chunks tid + NT*i
  u32x4 kreg[C::LOADS], vreg[C::LOADS];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int ci = tid + NT * i;
      const int row = ci / C::CH, c = ci % C::CH;
      const size_t a = key_addr(k0 + row) + c * 16;
      kreg[i] = *reinterpret_cast<const u32x4*>(kg + a);
      vreg[i] = *reinterpret_cast<const u32x4*>(vg + a);
    }
  };
  auto store_tile = [&](int stage) {
    char* sk = smem + stage * C::STAGEB;
    char* sv = sk + C::TILEB;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int ci = tid + NT * i;
      const int row = ci / C::CH, c = ci % C::CH;
      *reinterpret_cast<u32x4*>(sk + k_off<D>(row, c)) = kreg[i];
      *reinterpret_cast<u32x4*>(sv + v_off<D>(row, c)) = vreg[i];
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
  const int pos = my_row + off;   // last visible key index for this lane's query

  // transposing-read geometry: 16-lane group g = lane / 16
  const int grp = lane >> 4, gj = lane & 15;
  const int tr_row = 4 * (grp >> 1) + (gj >> 2);           // + 16 * ks (+ 8 for the high half)
  const int tr_col = 16 * (grp & 1) + 4 * (gj & 3);        // d within the 32-wide block

  if (n_kt > 0) {
    load_tile(0);
    store_tile(0);
    if (n_kt > 1) load_tile(C::BN);
  }
  __syncthreads();

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * C::BN;
    const char* sk = smem + (kt & 1) * C::STAGEB;
    const char* sv = sk + C::TILEB;
    const bool wave_sees = wave_rows && (!p.causal || k0 <= w_last + off);

    if (wave_sees) {
      // S^T = K Q^T
      f32x16 s[C::KB];
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) {
        s[kb] = f32x16{};
        const int r = kb * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < C::QK; ++ks)
          s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(sk + k_off<D>(r, ks * 2 + hl)), qf[ks], s[kb]);
      }

      // scale to log2 units, mask where needed, running max
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] *= c;
      if (k0 + C::BN > Lk || (p.causal && k0 + C::BN - 1 > w_first + off)) {
        // keys past the end or above the diagonal; lim = last visible key
        const int lim = p.causal ? min(pos, Lk - 1) : Lk - 1;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            s[kb][r] = key > lim ? kNegInf : s[kb][r];
          }
      }
      float mt = kNegInf;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
      mt = max_halves(mt);
      const float mn = fmaxf(m, mt);
      const float mu = mn == kNegInf ? 0.f : mn;
      const float alpha = exp2_fast(m - mu);
      m = mn;
      float psum = 0.f;
      bf16x8 pb[C::PS];
#pragma unroll
      for (int ps = 0; ps < C::PS; ++ps) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = exp2_fast(s[ps >> 1][(ps & 1) * 8 + e] - mu);
          psum += pe;
          v[e] = (__bf16)pe;
        }
        pb[ps] = v;
      }
      lsum = lsum * alpha + psum;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }

      // O^T += V^T P^T, V^T fragments through the transposing LDS read
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
#pragma unroll
        for (int ps = 0; ps < C::PS; ++ps) {
          const int r = ps * 16 + tr_row;
          const int d = db * 32 + tr_col;     // 4 consecutive d of one 16-byte chunk half
          const int cl = d >> 3, cb = (d & 7) * 2;
          v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)((lds_char*)sv + v_off<D>(r, cl) + cb));
          v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)((lds_char*)sv + v_off<D>(r + 8, cl) + cb));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = mfma32(a, pb[ps], o[db]);
        }
      }
    }

    // stage the next tile and fetch the one after it
    if (kt + 1 < n_kt) {
      store_tile((kt + 1) & 1);
      if (kt + 2 < n_kt) load_tile(k0 + 2 * C::BN);
    }
    __syncthreads();
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
