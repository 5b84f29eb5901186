// Prefill for head_dim 256 on bf16 / fp16 MFMA: four pairs of waves, each
// pair owning 32 query rows.
//
// Tiling, data movement and work order follow the head_dim 128 kernel
// (prefill.hip): one workgroup = one (query tile of BM = 128 rows, query
// head); K and V tiles of 64 keys go HBM -> LDS by buffer-load DMA into rings
// of two slots (128 KiB, one workgroup per CU); tiles wholly above the causal
// diagonal are never loaded.  At head_dim 256 a wave cannot hold Q, O^T and
// the scores of 32 rows in the 256 registers that two waves per SIMD allow,
// and a 16-row wave reads every K and V fragment for only 16 rows.  Here the
// two waves of a pair share 32 rows and split the work of a tile:
//   wave h:  S^T_h (keys 32 h .. +31 x 32 rows) = K_h . Q^T on
//            v_mfma_f32_32x32x16 (Q^T in 64 registers): its half of the
//            tile's scores;
//   both:    the running max agreed from the two waves' tile maxima (posted
//            in LDS one step ahead), P_h = 2^(s c - m) posted in LDS;
//   wave h:  O^T_h (d 128 h .. +127 x 32 rows) += V^T_h . P^T over its own
//            32 keys, then, after a barrier, over its partner's.
// A wave reads half a K tile and half a V tile per step: half the LDS
// operand bytes per flop of 16-row waves, with the register budget of two
// waves per SIMD (Q 64, O^T 64, two S^T blocks 32 registers).  Two barriers
// per tile: P posted, and the ring barrier.  The scores of tile kt + 1 are
// computed beside the exponentials of tile kt.
//
// Key order: as in the head_dim 128 kernel the S^T accumulator is the P^T
// operand as is; the V^T fragments are read in the same key order.
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
constexpr int PR = 32;                // query rows per pair of waves
constexpr int BN = 64;                // keys per tile
constexpr int ROWB = D * 2;           // bytes of one K/V row
constexpr int TILEB = BN * ROWB;      // 32 KiB
constexpr int CH = D / 8;             // 16-byte chunks per row
constexpr int DMA = TILEB / 1024 / NW;  // 1 KiB DMA instructions per wave per tile
constexpr int WROWS = BN / NW;        // tile rows written by one wave
constexpr int QK = D / 16;            // 16-element k-steps of S^T
constexpr int DBH = D / 2 / 32;       // 32-wide d blocks of a wave's half of O^T
constexpr int PS = BN / 16;           // 16-key k-steps of O^T
constexpr int R = 2;                  // ring slots per operand
constexpr int PB = 64 * 32;           // bytes of one wave's P (32 per lane)
constexpr int kPage = 16;
constexpr float kRescaleSlack = 8.f;
constexpr int kBufferWord3 = 0x00020000;
static_assert(BM == 4 * PR && DMA == 4 && WROWS == 8 && DBH == 4 && PS == 4, "geometry");
static_assert(WROWS <= kPage && kPage % WROWS == 0, "a wave's rows stay inside one page");
static_assert(2 * R * TILEB + NW * PB + 2 * NW * PR * 4 <= 160 * 1024, "LDS per CU");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

// Logical 16-byte chunk stored at physical chunk q of K row r / V row r.
__device__ __forceinline__ int k_chunk(int r, int q) { return q ^ (r & 15); }
__device__ __forceinline__ int v_chunk(int r, int q) { return (((q >> 2) ^ (r & 3)) << 2) | (q & 3); }

template <int N>
struct Idx { static constexpr int value = N; };

constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 0xc07f;

template <typename E, bool PAGED, bool LP>
__global__ __launch_bounds__(NT, 1) void prefill256_kernel(PrefillParams p,
                                                         const int32_t* __restrict__ page_table) {
  using H = Half16<E>;
  using elem = typename H::elem;
  using v8 = typename H::v8;
  using v2 = typename H::v2;
  auto mfma32 = [](v8 a, v8 b, f32x16 c) { return H::mfma32x32x16(a, b, c); };
  __shared__ __attribute__((aligned(1024))) char k_ring0[TILEB];
  __shared__ __attribute__((aligned(1024))) char k_ring1[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_ring0[TILEB];
  __shared__ __attribute__((aligned(1024))) char v_ring1[TILEB];
  __shared__ __attribute__((aligned(1024))) char p_buf[NW * PB];   // each wave's P^T, lane-linear
  __shared__ float m_buf[2][NW][PR];                               // tile maxima (by tile parity)
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
  const int pair = wave >> 1, half = wave & 1, partner = wave ^ 1;
  const int l32 = lane & 31, hl = lane >> 5;

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

  // ---- Q^T fragments (B operand): lane (row l32 of the pair, half hl) holds
  // q[16 ks + 8 hl .. + 8] for k-step ks.
  const int my_row = r0 + pair * PR + l32;
  const bool row_ok = my_row < Lq;
  v8 qf[QK];
  {
    const elem* qr = reinterpret_cast<const elem*>(p.q) +
                     ((size_t)(q_start + (row_ok ? my_row : 0)) * p.Hq + head) * D + hl * 8;
#pragma unroll
    for (int s = 0; s < QK; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qr + s * 16);
      if (flip) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qf[s] = row_ok ? __builtin_bit_cast(v8, v) : v8{};
    }
  }

  // ---- DMA geometry: instruction i of this wave fills the 1 KiB at tile
  // byte (wave * DMA + i) * 1024, RPI whole rows.
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
  // K fragment (k-step ks) of this wave's 32 keys: row l32 of the half,
  // logical chunk 2 ks + hl; k-steps 8.. are 256 bytes further on.
  const int kbase = half * 32 * ROWB;
  int kro[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kro[ks] = kbase + l32 * ROWB + (k_chunk(l32, 2 * ks + hl) << 4);
  // V^T fragment (d block db of this wave's half, key step ps): transposing
  // reads of rows 16 ps + tr_row (+ 8), d = 128 half + 32 db + tr_col.
  const int grp = lane >> 4, gj = lane & 15;
  const int tr_row = 4 * (grp >> 1) + (gj >> 2);
  const int tr_col = 16 * (grp & 1) + 4 * (gj & 3);
  int vro[DBH];
#pragma unroll
  for (int db = 0; db < DBH; ++db) {
    const int d = db * 32 + tr_col;
    vro[db] = half * 256 + tr_row * ROWB + (v_chunk(tr_row, d >> 3) << 4) + (d & 7) * 2;
  }
  // P^T pieces: 16-byte piece k of lane L at k * 1024 + L * 16 (conflict-free).
  char* const p_mine = p_buf + wave * PB + lane * 16;
  const char* const p_pair = p_buf + pair * 2 * PB + lane * 16;

  f32x16 o[DBH];
#pragma unroll
  for (int i = 0; i < DBH; ++i) o[i] = f32x16{};
  float m = kNegInf, lsum = 0.f;

  const int w_first = r0 + pair * PR;
  const int w_last = min(w_first + PR - 1, Lq - 1);
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

  auto qk = [&](const char* kbuf) {
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < QK; ++ks)
      s = mfma32(*reinterpret_cast<const v8*>(kbuf + (ks >> 3) * 256 + kro[ks & 7]), qf[ks], s);
    return s;
  };

  // Scores of this wave's keys past the end, right of the lane's diagonal or
  // left of its window -> -inf.
  auto mask = [&](int kt, f32x16& s) {
    const int k0 = kt * BN + half * 32;
    const int lim = up ? min(pos + rb, Lk - 1) : Lk - 1;
    const int lo = win >= 0 ? pos - win : 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 8 * (r >> 2) + 4 * hl + (r & 3);
      s[r] = (key > lim || key < lo) ? kNegInf : s[r];
    }
  };

  // Running max agreed by the pair: the larger of the two tile maxima; raised
  // (O, l rescaled) only past the slack.  Both waves see the same values.
  auto agree_max = [&](float mine, float theirs) {
    const float mt = fmaxf(mine, theirs) * c;
    const bool raise = mt > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float alpha = raise ? exp2_fast(m - mt) : 1.f;
      m = raise ? mt : m;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DBH; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
  };

  // P^T of this wave's 32 keys (two 16-key k-steps): kept for this wave's
  // O^T and posted to LDS for the partner; the row sum adds the rounded weights.
  auto weights = [&](const f32x16& s, float nm, v8 (&pw)[2]) {
    const v2 one = {(elem)1.f, (elem)1.f};
    float psum = 0.f;
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      v8 w;
#pragma unroll
      for (int e = 0; e < 8; ++e) w[e] = (elem)exp2_fast(__builtin_fmaf(s[ps * 8 + e], c, nm));
#pragma unroll
      for (int e = 0; e < 8; e += 2) psum = H::dot2(v2{w[e], w[e + 1]}, one, psum);
      *reinterpret_cast<v8*>(p_mine + ps * 1024) = w;
      pw[ps] = w;
    }
    lsum += psum;
  };

  // O^T += V^T . P^T over one wave's 32 keys: key half kh of the tile (this
  // wave's own, or its partner's), P^T given.
  auto pv_half = [&](const char* vbuf, int kh, const v8 (&pw)[2]) {
    const char* vb = vbuf + kh * 32 * ROWB;
#pragma unroll
    for (int db = 0; db < DBH; ++db)
#pragma unroll
      for (int ps = 0; ps < 2; ++ps) {
        const int ro = ps * 16 * ROWB + vro[db];
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((lds_char*)vb + ro));
        const v4i16 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((lds_char*)vb + ro + 8 * ROWB));
        o[db] = mfma32(__builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7)),
                       pw[ps], o[db]);
      }
  };

  auto barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("s_barrier" ::: "memory");
  };

  // One tile step.  On entry S^T(kt) of this wave is in registers and both
  // waves' tile maxima are in m_buf[kt % 2]; K(kt + 1) and V(kt) are in LDS.
  // The step starts the DMA of V(kt + 1) and K(kt + 2) (slots last read in
  // step kt - 1), agrees the running max and posts this wave's P(kt), computes
  // S^T(kt + 1) beside those exponentials and posts its maxima, accumulates
  // O^T over its own P(kt) and, after a barrier, over its partner's.  FAST:
  // tiles kt and kt + 1 unmasked and needed by every row.  (No issue-order
  // hints: those of the head_dim 128 kernel measured 1.5 % slower here, and
  // hints for the K reads alone were within 1 % of the compiler's order.)
  int pid_v = 0, pid_k = 0;     // pages of V(kt + 1) and K(kt + 2) for the next DMA
  float mine = kNegInf;         // this wave's tile max of S^T(kt)
  auto step = [&](auto slot_tag, auto fast_tag, int kt, f32x16& scur, f32x16& snext) {
    constexpr int SLOT = decltype(slot_tag)::value;
    constexpr bool FAST = decltype(fast_tag)::value != 0;
    constexpr int FULL = decltype(fast_tag)::value == 2 ? 1 : 0;
    if (kt + 1 < n_kt) dma(kt + 1, vslot(Idx<SLOT + 1>{}), true, pid_v, Idx<FULL>{});
    if (kt + 2 < n_kt) dma(kt + 2, kslot(Idx<SLOT>{}), false, pid_k, Idx<FULL>{});
    const bool need = FAST || kt < w_kt;
    const bool need_n = FAST || kt + 1 < w_kt;
    v8 pw[2];
    if (need) {
      agree_max(mine, m_buf[kt & 1][partner][l32]);
      weights(scur, FAST ? -m : (m == kNegInf ? 0.f : -m), pw);
    }
    mine = kNegInf;
    if (need_n) {
      snext = qk(kslot(Idx<SLOT + 1>{}));
      if (!FAST && (kt + 1 < w_lead || kt + 1 >= w_fast)) mask(kt + 1, snext);
      float mr = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mr = fmaxf(mr, snext[r]);
      mine = max_halves(mr);
    }
    if (hl == 0) m_buf[(kt + 1) & 1][wave][l32] = mine;
    if (need) pv_half(vslot(Idx<SLOT>{}), half, pw);     // this wave's own keys first
    barrier();
    if (need) {
      v8 pp[2];
#pragma unroll
      for (int ps = 0; ps < 2; ++ps) pp[ps] = *reinterpret_cast<const v8*>(p_pair + (half ^ 1) * PB + ps * 1024);
      pv_half(vslot(Idx<SLOT>{}), half ^ 1, pp);
    }
    if constexpr (PAGED) {
      pid_v = pid_k;
      if (kt + 3 < n_kt) pid_k = load_pid(kt + 3);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    barrier();
  };

  // Tiles that every row of the workgroup sees whole and unmasked; a FAST
  // step also computes the scores of the next tile, so it needs two of them.
  int n_fast = t_full;
  if (up) n_fast = min(n_fast, max(0, r0 + off + rb + 1) / BN);
  n_fast = max(0, min(n_fast, n_kt) - 1);
  n_fast -= n_fast % R;
  // Leading tiles that some row's window cuts run the masked step; a multiple of R.
  int n_lead = 0;
  if (win >= 0) {
    n_lead = min(n_kt, max(0, r_last + off - win + BN - 1) / BN);
    n_lead += n_lead % R;
  }
  n_fast = max(n_fast, n_lead);

  // prologue: K(0), V(0) in slot 0 and K(1) in slot 1; S^T(0) and its maxima.
  if (n_kt > 0) {
    const int pid = load_pid(0);
    dma(0, k_ring0, false, pid, Idx<0>{});
    dma(0, v_ring0, true, pid, Idx<0>{});
  }
  if (1 < n_kt) {
    pid_v = load_pid(1);
    dma(1, k_ring1, false, pid_v, Idx<0>{});
  }
  if (2 < n_kt) pid_k = load_pid(2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  f32x16 sa = {}, sb = {};
  if (n_kt > 0 && 0 < w_kt) {
    sa = qk(k_ring0);
    if (0 < w_lead || 0 >= w_fast) mask(0, sa);
    float mr = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mr = fmaxf(mr, sa[r]);
    mine = max_halves(mr);
  }
  if (hl == 0) m_buf[0][wave][l32] = mine;
  __syncthreads();
  int kt = 0;
  for (; kt < n_lead; kt += R) {
    step(Idx<0>{}, Idx<0>{}, kt, sa, sb);
    if (kt + 1 < n_kt) step(Idx<1>{}, Idx<0>{}, kt + 1, sb, sa);
  }
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

  // ---- epilogue: the pair's row sums (each wave summed its own keys)
  const float lmine = sum_halves(lsum);
  if (hl == 0) m_buf[0][wave][l32] = lmine;
  __syncthreads();
  const float ltot = lmine + m_buf[0][partner][l32];
  float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  float lse_v = ltot > 0.f ? (m + log2_fast(ltot)) * kLn2 : kNegInf;
  if (any_bad) {
    inv = __builtin_nanf("");
    lse_v = inv;
  }
  // Lane (row l32, hl) holds O^T[128 half + 32 db + 8 (r / 4) + 4 hl + r % 4][row].
  if (p.merge_lse == nullptr) {
    // Stage this wave's 32 rows x 128 d through LDS (the K ring is free: every
    // wave is past its last step) and store whole 256-byte row halves, 16
    // lanes x 16 bytes per row.  Chunk q of row r sits at chunk q ^ (r mod 16).
    char* stage = (wave < 4 ? k_ring0 : k_ring1) + (wave & 3) * PR * 256;
#pragma unroll
    for (int db = 0; db < DBH; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        typename H::v4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (elem)(o[db][4 * rq + r] * inv);
        const int q = 4 * db + rq;
        *reinterpret_cast<typename H::v4*>(stage + l32 * 256 + ((q ^ (l32 & 15)) << 4) + hl * 8) = v;
      }
    const int c16 = lane & 15;
#pragma unroll
    for (int i = 0; i < PR / 4; ++i) {
      const int r = i * 4 + (lane >> 4);
      const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * 256 + ((c16 ^ (r & 15)) << 4));
      const int row = w_first + r;
      if (row < Lq)
        *reinterpret_cast<u32x4*>(reinterpret_cast<elem*>(p.out) +
                                  ((size_t)(q_start + row) * p.Hq + head) * D + half * 128 + c16 * 8) = x;
    }
    if (half == 0 && hl == 0 && row_ok) p.lse[(size_t)(q_start + my_row) * p.Hq + head] = lse_v;
    return;
  }
  if (!row_ok) return;
  const size_t orow = (size_t)(q_start + my_row) * p.Hq + head;
  elem* og = reinterpret_cast<elem*>(p.out) + orow * D + half * 128 + 4 * hl;
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
    const elem* pg = reinterpret_cast<const elem*>(p.merge_o) + orow * D + half * 128 + 4 * hl;
#pragma unroll
    for (int db = 0; db < DBH; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = 32 * db + 8 * rq;
        typename H::v4 v;
        typename H::v4 w{};
        if (wp != 0.f) w = *reinterpret_cast<const typename H::v4*>(pg + d);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (elem)(o[db][4 * rq + r] * wo + (float)w[r] * wp);
        *reinterpret_cast<typename H::v4*>(og + d) = v;
      }
  }
  if (half == 0 && hl == 0) p.lse[orow] = lse_v;
}

template <typename E, bool PAGED>
hipError_t launch16_t(const PrefillParams& p, hipStream_t s) {
  const int total = p.Hq * p.B * p.q_tiles;
  dim3 grid(8 * ((total + 7) / 8));
  if (PAGED && p.page_shift > 0)
    hipLaunchKernelGGL((prefill256_kernel<E, PAGED, PAGED>), grid, dim3(NT), 0, s, p, p.page_table);
  else
    hipLaunchKernelGGL((prefill256_kernel<E, PAGED, false>), grid, dim3(NT), 0, s, p, p.page_table);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_d256(const PrefillParams& p, int dtype, bool paged, hipStream_t s) {
  if (dtype == 1) return paged ? launch16_t<bf16_t, true>(p, s) : launch16_t<bf16_t, false>(p, s);
  if (dtype == 2) return paged ? launch16_t<f16_t, true>(p, s) : launch16_t<f16_t, false>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace attn
