// Prefill for head_dim 256 on bf16 / fp16 MFMA: eight waves of 16 query rows.
//
// Same tiling, data movement, work order and step structure as the head_dim
// 128 kernel (prefill.hip): one workgroup = one (query tile of BM = 128
// rows, query head); K and V tiles of 64 keys go HBM -> LDS by buffer-load
// DMA into rings of two slots (128 KiB, one workgroup per CU); one wait and
// one barrier per tile; tiles wholly above the causal diagonal are never
// loaded.  What differs: a 32-row wave needs the whole register file at
// head_dim 256 (O^T alone is 128 VGPRs), so it would run alone on its SIMD.
// Here each wave owns 16 query rows, on v_mfma_f32_16x16x32_{bf16,f16}:
//   S^T(16 keys x 16 rows) = K . Q^T      A = K rows from LDS (16 bytes per lane),
//                                          B = Q^T held in VGPRs (32 registers)
//   O^T(16 d x 16 rows)  += V^T . P^T      A = V^T fragments from LDS via
//                                          ds_read_b64_tr_b16, B = P^T
// so a wave needs about half the registers and two waves share each SIMD:
// one wave's exponentials run beside the other's matrix work.  The price is
// twice the LDS operand reads per flop (every K and V fragment now feeds 16
// query rows instead of 32).  Tiles are 64 keys because the fixed cost of a
// step (DMA issue, wait, barrier) is large: 32-key tiles measured 10 %
// slower on long sequences.
//
// Key order inside each 32 keys of a tile: the S^T accumulator of key block
// kb (keys 16 kb .. 16 kb + 15) gives lane (query j = lane % 16, group
// g = lane / 16) keys 16 kb + 4 g .. + 3.  As the B operand of
// O^T += V^T P^T that lane supplies k-elements 8 g .. 8 g + 7, read here as
// keys {4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3}; the V^T fragments are read
// in the same key order, so P^T needs no data movement.
//
// LDS layouts (rows of 512 bytes): K chunks of 16 bytes XOR (row mod 16),
// so the 16 rows of a K fragment read hit every bank once; V units of 32
// bytes XOR (row mod 8), so the 8 rows two lane groups of a transposing read
// touch together land on distinct banks.
//
// This follows the tiled, fused scheme of "FlashAttention-3 内核在最新大模型
// 推理中的集成实践" (section 一: tiles in on-chip memory, online softmax
// accumulated in place, asynchronous copies overlapped with matrix work;
// section 四: keep the rescaling, and size tiles for head_dim 256 within the
// on-chip budget) and the QK^T / softmax / PV stages of "FlashInfer
// Attention Kernel技术解析" section 1.3 (bank conflicts: section 4).
#include "common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int D = 256;
constexpr int BM = kPrefillBM;        // query rows per workgroup
constexpr int NW = 8;                 // waves
constexpr int NT = NW * 64;
constexpr int RW = BM / NW;           // query rows per wave (16)
constexpr int BN = 64;                // keys per tile
constexpr int KB = BN / 16;           // 16-key blocks of S^T
constexpr int PS = BN / 32;           // 32-key k-steps of O^T
constexpr int ROWB = D * 2;           // bytes of one K/V row
constexpr int TILEB = BN * ROWB;      // 32 KiB
constexpr int CH = D / 8;             // 16-byte chunks per row
constexpr int DMA = TILEB / 1024 / NW;  // 1 KiB DMA instructions per wave per tile
constexpr int WROWS = BN / NW;        // tile rows written by one wave
constexpr int QK = D / 32;            // k-steps of S^T
constexpr int DB = D / 16;            // 16-row blocks of O^T
constexpr int R = 2;                  // ring slots per operand
constexpr int kPage = 16;
constexpr float kRescaleSlack = 8.f;
constexpr int kBufferWord3 = 0x00020000;
static_assert(RW == 16 && DMA == 4 && WROWS == 8, "geometry");
static_assert(WROWS <= kPage && kPage % WROWS == 0, "a wave's rows stay inside one page");
static_assert(R == 2 && 2 * R * TILEB <= 160 * 1024, "LDS per CU");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

// Logical 16-byte chunk stored at physical chunk q of K row r / V row r.
__device__ __forceinline__ int k_chunk(int r, int q) { return q ^ (r & 15); }
__device__ __forceinline__ int v_chunk(int r, int q) { return (((q >> 1) ^ (r & 7)) << 1) | (q & 1); }

template <int N>
struct Idx { static constexpr int value = N; };

constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 0xc07f;

// Sum / max over the four 16-lane groups (lanes j, j+16, j+32, j+48).
__device__ __forceinline__ float max_groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  x = fmaxf(__builtin_bit_cast(float, (int)a[0]), __builtin_bit_cast(float, (int)a[1]));
  return max_halves(x);
}
__device__ __forceinline__ float sum_groups(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                            false, false);
  x = __builtin_bit_cast(float, (int)a[0]) + __builtin_bit_cast(float, (int)a[1]);
  return sum_halves(x);
}

template <typename E, bool PAGED, bool LP>
__global__ __launch_bounds__(NT, 1) void prefill16_kernel(PrefillParams p,
                                                         const int32_t* __restrict__ page_table) {
  using H = Half16<E>;
  using elem = typename H::elem;
  using v8 = typename H::v8;
  using v2 = typename H::v2;
  auto mfma = [](v8 a, v8 b, f32x4 c) { return H::mfma16x16x32(a, b, c); };
  __shared__ __attribute__((aligned(1024))) char k_ring0[TILEB];
  __shared__ __attribute__((aligned(1024))) char k_ring1[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_ring0[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_ring1[TILEB];
  auto kslot = [&](auto i) -> char* {
    if constexpr (decltype(i)::value % R == 0) return k_ring0;
    else return k_ring1;
  };
  auto vslot = [&](auto i) -> char* {
    if constexpr (decltype(i)::value % R == 0) return v_ring0;
    else return v_ring1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j16 = lane & 15, grp = lane >> 4;

  // Work order: as the head_dim 128 kernel (XCD c runs the c-th eighth of the
  // (KV head, sequence, tile heaviest first, query head) list).
  int head, kvh, b, tile;
  {
    const int G = p.Hq / p.Hkv;
    const int total = p.Hq * p.B * p.q_tiles;          // fits an int (checked on the host)
    const int chunk = (total + 7) / 8;
    const int w = blockIdx.x;
    int r = (w % 8) * chunk + w / 8;
    if (r >= total) return;
    const int hg = r % G;
    r /= G;
    tile = p.q_tiles - 1 - r % p.q_tiles;
    r /= p.q_tiles;
    b = r % p.B;
    kvh = r / p.B;
    head = kvh * G + hg;
  }

  // Sequence extents, clamped so every access stays inside the tensors.
  const bool fixed = PAGED && p.kv_len_fixed >= 0;
  const int q_start = fixed ? 0 : min(max(p.cu_q[b], 0), p.total_q);
  const int q_end = fixed ? p.total_q : min(max(p.cu_q[b + 1], q_start), p.total_q);
  const int Lq = q_end - q_start;
  const int r0 = tile * BM;
  if (r0 >= Lq) return;
  bool bad = Lq > p.max_seqlen_q;
  int k_start = 0, Lk;
  const int32_t* table = nullptr;
  // LP (pages of 32..256 tokens): table stays at the row start and blk_off
  // counts the 16-token blocks skipped (key offset, window); a block's page is
  // table[block >> page_shift].
  int blk_off = 0;
  if constexpr (PAGED) {
    if (fixed) {
      Lk = p.kv_len_fixed;
      table = page_table;
    } else {
      // kv_len above the table's capacity or above the host bound max_kv_len
      // (max_seqlen_k) marks the request bad and reads nothing.
      Lk = p.kv_lens[b] - p.kv_offset;
      if (Lk < 0 || Lk > p.max_tokens - p.kv_offset || Lk > p.max_seqlen_k - p.kv_offset) {
        bad = true;
        Lk = 0;
      }
      if (p.kv_offset > 0 && p.causal && Lk < Lq) bad = true;
      table = page_table + (size_t)b * p.table_stride + (LP ? 0 : p.kv_offset / kPage);
      if constexpr (LP) blk_off = p.kv_offset / kPage;
    }
  } else {
    k_start = min(max(p.cu_k[b], 0), p.total_k);
    const int k_end = min(max(p.cu_k[b + 1], k_start), p.total_k);
    Lk = k_end - k_start;
    if (Lk > p.max_seqlen_k) { bad = true; Lk = 0; }   // above the host bound max_seqlen_k
  }
  int off = Lk - Lq;                             // bottom-right causal offset
  // Right bound: query i sees keys j <= i + off + rb (causal: rb = 0).
  const int rb = p.causal ? 0 : p.window_right;
  const bool up = rb >= 0;
  const int r_last = min(r0 + BM, Lq) - 1;
  int kend = up ? min(Lk, r_last + off + rb + 1) : Lk;
  if (kend < 0) kend = 0;
  // Sliding window: query i sees keys from i + off - window_left on.  Whole
  // tiles before the first row's window are skipped by moving the key origin
  // (tile-aligned, so paged tiles still start at a page).
  const int win = p.window_left;
  if (win >= 0) {
    const int kt0 = min(max(0, r0 + off - win), kend) / BN;
    const int sh = kt0 * BN;
    if constexpr (PAGED) {
      if constexpr (LP) blk_off += sh / kPage;
      else table += sh / kPage;
    }
    else k_start += sh;
    Lk -= sh;
    off -= sh;
    kend -= sh;
  }
  const int n_kt = (kend + BN - 1) / BN;

  float c = p.scale_log2;
  const bool flip = c < 0.f;
  c = flip ? -c : (c == 0.f ? 1e-30f : c);

  // ---- Q^T fragments (B operand): lane (row j16 of this wave, group grp)
  // holds q[32 ks + 8 grp .. + 8] for k-step ks.
  const int my_row = r0 + wave * RW + j16;
  const bool row_ok = my_row < Lq;
  v8 qf[QK];
  {
    const elem* qr = reinterpret_cast<const elem*>(p.q) +
                     ((size_t)(q_start + (row_ok ? my_row : 0)) * p.Hq + head) * D + grp * 8;
#pragma unroll
    for (int s = 0; s < QK; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qr + s * 32);
      if (flip) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qf[s] = row_ok ? __builtin_bit_cast(v8, v) : v8{};
    }
  }

  // ---- DMA geometry (as prefill.hip): instruction i of this wave fills the
  // 1 KiB at tile byte (wave * DMA + i) * 1024, RPI whole rows.
  constexpr int RPI = 64 / CH;
  const char* kg = reinterpret_cast<const char*>(p.k);
  const char* vg = reinterpret_cast<const char*>(p.v);
  // Bytes between consecutive keys of one head: NHD interleaves the heads of
  // a token, HND (paged only) keeps each head's 16 rows of a page together.
  const int kv_rowb = (PAGED && p.kv_hnd) ? ROWB : p.Hkv * ROWB;
  // A 16-token block is addressed as base + id * page_b + kv head * head_b:
  // with 16-token pages the id is the page id; with larger pages (LP) it is
  // page * m + block (NHD, m = 1 << page_shift) or page * Hkv * m + block (HND).
  const size_t page_b = (LP && p.kv_hnd) ? (size_t)kPage * ROWB : (size_t)kPage * p.Hkv * ROWB;
  const size_t head_b = (PAGED && p.kv_hnd) ? ((size_t)kPage << (LP ? p.page_shift : 0)) * ROWB
                                            : (size_t)ROWB;
  const int wrow0 = wave * WROWS;
  const int lane_row = lane / CH, lane_q = lane % CH;
  const int lane_rowb = lane_row * kv_rowb;
  unsigned klane[DMA], vlane[DMA];
#pragma unroll
  for (int i = 0; i < DMA; ++i) {
    const int rlo = ((wave * DMA + i) * RPI) & 15;
    klane[i] = (unsigned)(lane_rowb + k_chunk(rlo | lane_row, lane_q) * 16);
    vlane[i] = (unsigned)(lane_rowb + v_chunk(rlo | lane_row, lane_q) * 16);
  }
  const int t_full = Lk / BN;
  auto load_pid = [&](int t) -> int {
    int pid = 0;
    if constexpr (PAGED) {
      if constexpr (LP) {
        const int k16 = (min(t * BN + wrow0, Lk - 1) >> 4) + blk_off;
        pid = table[k16 >> p.page_shift];
        if ((unsigned)pid >= (unsigned)p.num_pages) { bad = true; pid = 0; }
        pid = pid * (p.kv_hnd ? p.Hkv << p.page_shift : 1 << p.page_shift) +
              (k16 & ((1 << p.page_shift) - 1));
      } else {
        pid = table[min(t * BN + wrow0, Lk - 1) >> 4];
        if ((unsigned)pid >= (unsigned)p.num_pages) { bad = true; pid = 0; }
      }
    }
    return pid;
  };
  auto dma = [&](int kt, char* dst, bool is_v, int pid, auto full_tag) {
    const int k0 = kt * BN;
    const char* g = is_v ? vg : kg;
    const char* base;
    int nrec;
    if constexpr (PAGED) {
      base = g + (size_t)pid * page_b + (size_t)kvh * head_b;
      nrec = (kPage - 1) * kv_rowb + ROWB;
    } else {
      base = g + ((size_t)(k_start + k0) * kv_rowb + (size_t)kvh * ROWB);
      nrec = (min(BN, Lk - k0) - 1) * kv_rowb + ROWB;
    }
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, nrec, kBufferWord3);
    if (decltype(full_tag)::value || kt < t_full) {   // full_tag: known to be a whole tile
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        const int r0i = (wave * DMA + i) * RPI;
        const int soff = (PAGED ? (r0i & (kPage - 1)) : r0i) * kv_rowb;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (wave * DMA + i) * 1024), 16,
                                                 (int)(is_v ? vlane[i] : klane[i]), soff, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        const int kj = min(k0 + (wave * DMA + i) * RPI + lane_row, Lk - 1);
        const int row = PAGED ? (kj & (kPage - 1)) : kj - k0;
        const int o = row * kv_rowb - lane_rowb + (int)(is_v ? vlane[i] : klane[i]);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (wave * DMA + i) * 1024), 16,
                                                 o, 0, 0, 0);
      }
    }
  };

  // ---- per-lane LDS read offsets
  // K fragment (key block kb, k-step ks): row 16 kb + j16, logical chunk
  // 4 ks + grp.  The swizzle touches chunk bits 0-3, so k-steps 4.. are 256
  // bytes further on and key block 1 is 16 rows further on.
  int kro[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) kro[q] = j16 * ROWB + (k_chunk(j16, 4 * q + grp) << 4);
  // V^T fragment (d block db, keys 4 grp ..): a transposing read in which lane
  // (j16, grp) addresses row 4 grp + j16 / 4, elements 16 db + 4 (j16 % 4) .. + 3.
  // The swizzle touches 32-byte unit bits 0-2, so d blocks 8.. are 256 bytes on.
  const int tr_row = 4 * grp + (j16 >> 2);
  int vro[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) vro[u] = tr_row * ROWB + ((u ^ (tr_row & 7)) << 5) + 8 * (j16 & 3);

  f32x4 o[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) o[i] = f32x4{};
  float m = kNegInf, lsum = 0.f;

  const int w_first = r0 + wave * RW;
  const int w_last = min(w_first + RW - 1, Lq - 1);
  const bool wave_rows = w_first < Lq;
  const int pos = my_row + off;
  int w_kt = 0, w_fast = 0, w_lead = 0;
  if (wave_rows) {
    // tiles before w_lead hold keys left of some row's window
    if (win >= 0) w_lead = max(0, w_last + off - win + BN - 1) / BN;
    const int wkend = up ? max(0, min(Lk, w_last + off + rb + 1)) : Lk;
    w_kt = min(n_kt, (wkend + BN - 1) / BN);
    int lim = t_full;
    if (up) lim = min(lim, max(0, w_first + off + rb + 1) / BN);
    w_fast = min(lim, w_kt);
  }

  auto kfrag = [&](const char* kbuf, int kb, int ks) {
    return *reinterpret_cast<const v8*>(kbuf + kb * 16 * ROWB + (ks >> 2) * 256 + kro[ks & 3]);
  };
  auto qk = [&](const char* kbuf, f32x4 (&s)[KB]) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x4{};
#pragma unroll
      for (int ks = 0; ks < QK; ++ks) s[kb] = mfma(kfrag(kbuf, kb, ks), qf[ks], s[kb]);
    }
  };

  auto mask = [&](int kt, f32x4 (&s)[KB]) {
    const int k0 = kt * BN;
    const int lim = up ? min(pos + rb, Lk - 1) : Lk - 1;
    const int lo = win >= 0 ? pos - win : 0;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 16 * kb + 4 * grp + r;
        s[kb][r] = (key > lim || key < lo) ? kNegInf : s[kb][r];
      }
  };

  auto update_max = [&](f32x4 (&s)[KB]) {
    float mr = kNegInf;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mr = fmaxf(mr, s[kb][r]);
    const float mt = max_groups(mr) * c;
    const bool raise = mt > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float alpha = raise ? exp2_fast(m - mt) : 1.f;
      m = raise ? mt : m;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[db][r] *= alpha;
    }
  };

  // P^T = 2^(s c - m) in the B-operand order {kb 0 keys, kb 1 keys}; the row
  // sum adds the rounded weights.
  auto weights = [&](f32x4 (&s)[KB], v8 (&pb)[PS], float nm) {
    const v2 one = {(elem)1.f, (elem)1.f};
    float psum = 0.f;
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) {
      v8 w;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[e] = (elem)exp2_fast(__builtin_fmaf(s[2 * ps + (e >> 2)][e & 3], c, nm));
#pragma unroll
      for (int e = 0; e < 8; e += 2) psum = H::dot2(v2{w[e], w[e + 1]}, one, psum);
      pb[ps] = w;
    }
    lsum += psum;
  };

  auto vfrag = [&](const char* vbuf, int db, int ps) {
    const int ro = ps * 32 * ROWB + (db >> 3) * 256 + vro[db & 7];
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((lds_char*)vbuf + ro));
    const v4i16 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((lds_char*)vbuf + ro + 16 * ROWB));
    return __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto pv = [&](const char* vbuf, v8 (&pb)[PS]) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) o[db] = mfma(vfrag(vbuf, db, ps), pb[ps], o[db]);
  };

  f32x4 sa[KB], sb[KB];
  int pid_v = 0, pid_k = 0;
  auto step = [&](auto slot_tag, auto fast_tag, int kt, f32x4 (&scur)[KB], f32x4 (&snext)[KB]) {
    constexpr int SLOT = decltype(slot_tag)::value;
    constexpr bool FAST = decltype(fast_tag)::value != 0;
    // 2: a steady-state step whose two DMAs are whole tiles (no clamped rows)
    constexpr int FULL = decltype(fast_tag)::value == 2 ? 1 : 0;
    char* const KDST = kslot(Idx<SLOT>{});
    char* const KNXT = kslot(Idx<SLOT + 1>{});
    char* const VCUR = vslot(Idx<SLOT>{});
    char* const VDST = vslot(Idx<SLOT + R - 1>{});
    if (kt + R - 1 < n_kt) dma(kt + R - 1, VDST, true, pid_v, Idx<FULL>{});
    if (kt + R < n_kt) dma(kt + R, KDST, false, pid_k, Idx<FULL>{});
    v8 pb[PS];
    if constexpr (FAST) {
      update_max(scur);
      qk(KNXT, snext);
      weights(scur, pb, -m);
      pv(VCUR, pb);
      // Issue order: eight K fragment reads ahead of the S^T MFMAs, each S^T
      // MFMA followed by the next K read and two vector ops of the softmax,
      // the first V^T reads behind the last eight S^T MFMAs, then each O^T
      // MFMA with the transposing reads of a later fragment.  (Left to the
      // compiler, the reads ran one or two MFMAs ahead and the waves waited
      // on LDS before almost every MFMA.)
      constexpr int KA = 8;
      __builtin_amdgcn_sched_group_barrier(0x100, KA, 0);             // K reads
#pragma unroll
      for (int i = 0; i < KB * QK - KA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // S^T MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);            // next K read
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);            // softmax
      }
#pragma unroll
      for (int i = 0; i < KA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);            // first V reads
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
      }
#pragma unroll
      for (int i = 0; i < DB * PS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // O^T MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);            // V reads ahead
        __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);
      }
    } else if (kt < w_kt) {
      if (kt < w_lead || kt >= w_fast) mask(kt, scur);
      update_max(scur);
      if (kt + 1 < w_kt) qk(KNXT, snext);
      weights(scur, pb, m == kNegInf ? 0.f : -m);
      pv(VCUR, pb);
    }
    if constexpr (PAGED) {
      pid_v = pid_k;
      if (kt + R + 1 < n_kt) pid_k = load_pid(kt + R + 1);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("s_barrier" ::: "memory");
  };

  int n_fast = t_full;
  if (up) n_fast = min(n_fast, max(0, r0 + off + rb + 1) / BN);
  {
    const int wkend0 = up ? max(0, min(Lk, min(r0 + RW - 1, Lq - 1) + off + rb + 1)) : Lk;
    const int w_kt0 = min(n_kt, (wkend0 + BN - 1) / BN);
    n_fast = max(0, min(n_fast, w_kt0 - 1));
    n_fast -= n_fast % R;
  }
  // Leading tiles that some row's window cuts (from the last row, whose
  // window starts latest) run the masked step too; a multiple of R.
  int n_lead = 0;
  if (win >= 0) {
    n_lead = min(n_kt, max(0, r_last + off - win + BN - 1) / BN);
    n_lead += n_lead % R;
  }
  n_fast = max(n_fast, n_lead);

  // prologue: K(0 .. R-1) and V(0 .. R-2) in LDS, S^T(0) in registers
#pragma unroll
  for (int t = 0; t < R; ++t) {
    if (t < n_kt) {
      const int pid = load_pid(t);
      char* kd = t == 0 ? kslot(Idx<0>{}) : kslot(Idx<1>{});
      char* vd = t == 0 ? vslot(Idx<0>{}) : vslot(Idx<1>{});
      dma(t, kd, false, pid, Idx<0>{});
      if (t + 1 < R) dma(t, vd, true, pid, Idx<0>{});
      else pid_v = pid;
    }
  }
  if (R < n_kt) pid_k = load_pid(R);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  if (n_kt > 0) qk(k_ring0, sa);
  __syncthreads();
  int kt = 0;
  for (; kt < n_lead; kt += R) {
    step(Idx<0>{}, Idx<0>{}, kt, sa, sb);
    if (kt + 1 < n_kt) step(Idx<1>{}, Idx<0>{}, kt + 1, sb, sa);
  }
  // Steady-state steps whose DMAs (tiles kt + R - 1 and kt + R) are whole
  // tiles skip the clamped-row addressing of the last, partial tile.
  for (; kt < n_fast && kt + R + 1 < t_full; kt += R) {
    step(Idx<0>{}, Idx<2>{}, kt, sa, sb);
    step(Idx<1>{}, Idx<2>{}, kt + 1, sb, sa);
  }
  for (; kt < n_fast; kt += R) {
    step(Idx<0>{}, Idx<1>{}, kt, sa, sb);
    step(Idx<1>{}, Idx<1>{}, kt + 1, sb, sa);
  }
  for (; kt < n_kt; kt += R) {
    step(Idx<0>{}, Idx<0>{}, kt, sa, sb);
    if (kt + 1 < n_kt) step(Idx<1>{}, Idx<0>{}, kt + 1, sb, sa);
  }

  const bool any_bad = __syncthreads_or(bad);

  // ---- epilogue: lane (row j16, group grp) holds O^T[16 db + 4 grp + r][row]
  const float ltot = sum_groups(lsum);
  float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  float lse_v = ltot > 0.f ? (m + log2_fast(ltot)) * kLn2 : kNegInf;
  if (any_bad) {
    inv = __builtin_nanf("");
    lse_v = inv;
  }
  if (p.merge_lse == nullptr) {
    // Stage this wave's 16 x D tile through LDS (the K ring is free: every
    // wave is past its last step) and store whole rows, 32 lanes x 16 bytes
    // per row, instead of 8-byte pieces scattered over 16 rows per store.
    // Chunk q of row r sits at chunk q ^ (r mod 16).
    char* stage = (wave < 4 ? k_ring0 : k_ring1) + (wave & 3) * RW * ROWB;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      typename H::v4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (elem)(o[db][r] * inv);
      const int q = 2 * db + (grp >> 1);
      *reinterpret_cast<typename H::v4*>(stage + j16 * ROWB + ((q ^ j16) << 4) + (grp & 1) * 8) = v;
    }
    const int c32 = lane & 31;
#pragma unroll
    for (int i = 0; i < RW / 2; ++i) {
      const int r = i * 2 + (lane >> 5);
      const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * ROWB + ((c32 ^ (r & 15)) << 4));
      const int row = r0 + wave * RW + r;
      if (row < Lq)
        *reinterpret_cast<u32x4*>(reinterpret_cast<elem*>(p.out) +
                                  ((size_t)(q_start + row) * p.Hq + head) * D + c32 * 8) = x;
    }
    if (grp == 0 && row_ok) p.lse[(size_t)(q_start + my_row) * p.Hq + head] = lse_v;
    return;
  }
  if (!row_ok) return;
  const size_t orow = (size_t)(q_start + my_row) * p.Hq + head;
  elem* og = reinterpret_cast<elem*>(p.out) + orow * D + 4 * grp;
  {
    // Merge with another state over disjoint keys (see prefill.hip).
    const float lp = p.merge_lse[orow] * kLog2e;
    const float ls = ltot > 0.f ? m + log2_fast(ltot) : kNegInf;
    const float mx = fmaxf(lp, ls);
    float wo = 0.f, wp = 0.f;
    if (any_bad || lp != lp) {
      wo = __builtin_nanf("");
      lse_v = wo;
    } else if (mx == kNegInf) {
      lse_v = kNegInf;
    } else {
      wp = exp2_fast(lp - mx);
      const float ws = ltot > 0.f ? exp2_fast(m - mx) : 0.f;
      const float den = wp + ws * ltot;
      const float rd = 1.f / den;
      wo = ws * rd;
      wp *= rd;
      lse_v = (mx + log2_fast(den)) * kLn2;
    }
    const elem* pg = reinterpret_cast<const elem*>(p.merge_o) + orow * D + 4 * grp;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      typename H::v4 v;
      typename H::v4 w{};
      if (wp != 0.f) w = *reinterpret_cast<const typename H::v4*>(pg + 16 * db);
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (elem)(o[db][r] * wo + (float)w[r] * wp);
      *reinterpret_cast<typename H::v4*>(og + 16 * db) = v;
    }
  }
  if (grp == 0) p.lse[orow] = lse_v;
}

template <typename E, bool PAGED>
hipError_t launch16_t(const PrefillParams& p, hipStream_t s) {
  const int total = p.Hq * p.B * p.q_tiles;
  dim3 grid(8 * ((total + 7) / 8));
  if (PAGED && p.page_shift > 0)
    hipLaunchKernelGGL((prefill16_kernel<E, PAGED, PAGED>), grid, dim3(NT), 0, s, p, p.page_table);
  else
    hipLaunchKernelGGL((prefill16_kernel<E, PAGED, false>), grid, dim3(NT), 0, s, p, p.page_table);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_d256(const PrefillParams& p, int dtype, bool paged, hipStream_t s) {
  if (dtype == 1) return paged ? launch16_t<bf16_t, true>(p, s) : launch16_t<bf16_t, false>(p, s);
  if (dtype == 2) return paged ? launch16_t<f16_t, true>(p, s) : launch16_t<f16_t, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace attn
