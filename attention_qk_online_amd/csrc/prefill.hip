// Ragged causal prefill for gfx950 on bf16 / fp16 MFMA with fp32 accumulation,
// head_dim 128 (head_dim 256: prefill256.hip).
//
// One workgroup = one (query tile of BM = 128 rows, query head) of one
// sequence; four waves own 32 query rows each.  Key tiles have BN = 64 keys.
// Two workgroups run per CU, so one wave's matrix work overlaps another's
// vector work.
//
// Data movement: K and V tiles go from HBM straight into LDS with
// buffer_load_dwordx4 ... lds (no register staging), into rings of R = 2
// slots: while tile j is processed, the
// DMA for K(j+R) and V(j+R-1) is in flight; one wait and one barrier per
// tile.  Each lane loads the 16-byte chunk that belongs at its LDS position
// under an XOR swizzle (K: chunk XOR row mod 16; V: 64-byte block XOR row mod
// 4), so the MFMA operand reads below hit every bank once.
//
// Per tile j (the loop is unrolled by R so every LDS address is a per-lane
// constant plus an immediate):
//   1. S^T(j+1) = K(j+1) . Q^T on v_mfma_f32_32x32x16_bf16 (_f16), issued alongside
//      the softmax of tile j (independent work, interleaved on the SIMD).
//      Q stays in VGPRs (B operand); the transposed product gives each lane
//      one query column, so a row max is in-lane plus one lane^32 exchange.
//   2. Softmax of S^T(j) in log2 units: masks only on tiles crossing the
//      diagonal or the end of the keys (a separate, generic step); p =
//      2^(s*c - m) with one FMA; the running max m is raised (and O, l
//      rescaled) only when a row's tile max exceeds it by more than 2^8, so
//      rescaling is rare while p stays below 256.
//   3. O^T += V^T(j) . P^T(j) on MFMA: the S^T accumulator is already laid
//      out as the B operand (keys permuted identically on both operands), and
//      V^T fragments come from the row-major V tile through ds_read_b64_tr_b16.
// Tiles wholly above the causal diagonal are never loaded.  The score
// matrix never reaches memory.
//
// This follows the tiled, fused scheme of "FlashAttention-3 内核在最新大模型
// 推理中的集成实践" (section 一: Q/K/V blocks in on-chip memory, online softmax
// accumulated in place, asynchronous global-to-shared copies overlapped with
// tensor-core work by double buffering; section 二: varlen packing by
// cu_seqlens, causal, paged blocks; section 四: keep the rescaling) and the
// three-stage QK^T /
// softmax / PV pipeline of "FlashInfer Attention Kernel技术解析" section 1.3
// (bank-conflict avoidance: section 4), re-tiled for 64-wide waves, 32x32
// MFMA tiles and a 160 KiB LDS.
#include "common.h"
#include "launch.h"

namespace attn {

namespace {

constexpr int BM = kPrefillBM;   // query rows per workgroup
constexpr int NWAVE = 4;
constexpr int NT = NWAVE * 64;
constexpr int kPage = 16;
constexpr float kRescaleSlack = 8.f;   // log2 units the running max may lag behind
constexpr int kBufferWord3 = 0x00020000;   // buffer descriptor word 3 for gfx950 (32-bit data format)

template <int D>
struct Cfg {
  static_assert(D == 128, "head_dim 256 has its own kernel");
  static constexpr int BN = 64;                       // keys per tile
  static constexpr int ROWB = D * 2;                  // bytes of one K/V row
  static constexpr int TILEB = BN * ROWB;             // bytes of one K or V tile
  static constexpr int CH = D / 8;                    // 16-byte chunks per row
  static constexpr int DMA = TILEB / 1024 / NWAVE;    // 1 KiB DMA instructions per wave per tile
  static constexpr int WROWS = BN / NWAVE;            // tile rows written by one wave
  static constexpr int QK = D / 16;                   // MFMA k-steps over D
  static constexpr int DB = D / 32;                   // 32-row blocks of D in O^T
  static constexpr int KB = BN / 32;                  // 32-key blocks per tile
  static constexpr int PS = BN / 16;                  // 16-key k-steps of P.V
  static constexpr int VALU_PER_QK = 6;               // vector work issued per S^T MFMA
  static constexpr int R = 2;                         // ring slots per operand
  static constexpr int LDSB = 2 * R * TILEB;
  static_assert(TILEB % (1024 * NWAVE) == 0, "tile split into 1 KiB DMA instructions");
  static_assert(WROWS <= kPage && kPage % WROWS == 0, "a wave's rows stay inside one page");
  static_assert(LDSB <= 80 * 1024, "two workgroups per CU");
};


typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

// Logical 16-byte chunk stored at physical chunk q of K row r / V row r.
__device__ __forceinline__ int k_chunk(int r, int q) { return q ^ (r & 15); }
__device__ __forceinline__ int v_chunk(int r, int q) { return (((q >> 2) ^ (r & 3)) << 2) | (q & 3); }

template <int N>
struct Idx { static constexpr int value = N; };

// s_waitcnt immediates (gfx9 encoding): vmcnt(n) with expcnt and lgkmcnt
// unconstrained, and lgkmcnt(0) alone.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 0xc07f;

// The page table comes as its own restrict-qualified argument so that its
// wave-uniform reads compile to scalar loads.
template <typename E, int D, bool PAGED, bool LP>
__global__ __launch_bounds__(NT, 2) void prefill_kernel(
    PrefillParams p, const int32_t* __restrict__ page_table) {
  using C = Cfg<D>;
  using H = Half16<E>;            // bf16 or fp16 inputs
  using elem = typename H::elem;
  using v8 = typename H::v8;
  using v2 = typename H::v2;
  auto mfma32 = [](v8 a, v8 b, f32x16 c) { return H::mfma32x32x16(a, b, c); };
  // One array per ring slot (not one array): the compiler can then tell that a
  // DMA into one slot does not alias operand reads from another, and does not
  // stall those reads on the DMA's completion.
  __shared__ __attribute__((aligned(1024))) char k_ring0[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char k_ring1[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v_ring0[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v_ring1[C::TILEB];
  auto kslot = [&](auto i) -> char* {
    if constexpr (decltype(i)::value % C::R == 0) return k_ring0;
    else return k_ring1;
  };
  auto vslot = [&](auto i) -> char* {
    if constexpr (decltype(i)::value % C::R == 0) return v_ring0;
    else return v_ring1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;

  // Work order.  Workgroups are dealt round-robin over the 8 XCDs (each with
  // its own L2); XCD c takes the c-th contiguous eighth of the work items
  // ordered by (KV head, sequence, query tile heaviest first, query head of
  // the KV head's group).  Workgroups running together on one XCD then share
  // their K/V reads: the query heads of one KV head, the tiles of one sequence.
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
  const bool fixed = PAGED && p.kv_len_fixed >= 0;   // all rows, one key range
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
    const int kt0 = min(max(0, r0 + off - win), kend) / C::BN;
    const int sh = kt0 * C::BN;
    if constexpr (PAGED) {
      if constexpr (LP) blk_off += sh / kPage;
      else table += sh / kPage;
    }
    else k_start += sh;
    Lk -= sh;
    off -= sh;
    kend -= sh;
  }
  const int n_kt = (kend + C::BN - 1) / C::BN;

  // Scores are used as s * c with c > 0: a negative scale flips the sign of Q,
  // a zero scale becomes a tiny one (every weight rounds to exactly 1).
  float c = p.scale_log2;
  const bool flip = c < 0.f;
  c = flip ? -c : (c == 0.f ? 1e-30f : c);

  // ---- Q fragments (B operand of S^T = K Q^T): row l32 of this wave's 32 rows.
  const int my_row = r0 + wave * 32 + l32;
  const bool row_ok = my_row < Lq;
  v8 qf[C::QK];
  {
    const elem* qr = reinterpret_cast<const elem*>(p.q) +
                       ((size_t)(q_start + (row_ok ? my_row : 0)) * p.Hq + head) * D + hl * 8;
#pragma unroll
    for (int s = 0; s < C::QK; ++s) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qr + s * 16);
      if (flip) v ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
      qf[s] = row_ok ? __builtin_bit_cast(v8, v) : v8{};
    }
  }

  // ---- DMA geometry.  Instruction i of this wave fills the 1 KiB of LDS at
  // tile byte (wave * DMA + i) * 1024: RPI whole rows, lane -> row
  // (wave * DMA + i) * RPI + lane / CH, physical chunk lane % CH, fetching the
  // logical chunk that the swizzle puts there.
  constexpr int RPI = 64 / C::CH;                      // rows per DMA instruction
  const char* kg = reinterpret_cast<const char*>(p.k);
  const char* vg = reinterpret_cast<const char*>(p.v);
  // Bytes between consecutive keys of one head: NHD interleaves the heads of
  // a token, HND (paged only) keeps each head's 16 rows of a page together.
  const int kv_rowb = (PAGED && p.kv_hnd) ? C::ROWB : p.Hkv * C::ROWB;
  // A 16-token block is addressed as base + id * page_b + kv head * head_b:
  // with 16-token pages the id is the page id; with larger pages (LP) it is
  // page * m + block (NHD, m = 1 << page_shift) or page * Hkv * m + block (HND).
  const size_t page_b = (LP && p.kv_hnd) ? (size_t)kPage * C::ROWB : (size_t)kPage * p.Hkv * C::ROWB;
  const size_t head_b = (PAGED && p.kv_hnd) ? ((size_t)kPage << (LP ? p.page_shift : 0)) * C::ROWB
                                            : (size_t)C::ROWB;
  const int wrow0 = wave * C::WROWS;                   // first tile row of this wave
  const int lane_row = lane / C::CH, lane_q = lane % C::CH;
  const int lane_rowb = lane_row * kv_rowb;
  // Per-lane part of each DMA address (row within the instruction + swizzled
  // chunk); the instruction's first row is wave-uniform and goes in the base.
  unsigned klane[C::DMA], vlane[C::DMA];
#pragma unroll
  for (int i = 0; i < C::DMA; ++i) {
    const int rlo = ((wave * C::DMA + i) * RPI) & 15;  // a multiple of RPI, so OR adds lane_row
    klane[i] = (unsigned)(lane_rowb + k_chunk(rlo | lane_row, lane_q) * 16);
    vlane[i] = (unsigned)(lane_rowb + v_chunk(rlo | lane_row, lane_q) * 16);
  }
  const int t_full = Lk / C::BN;                       // tiles wholly inside the keys
  // Issue the DMA of K (is_v = false) or V rows k0 .. k0 + BN - 1 into LDS tile `dst`
  // with buffer loads (a wave-uniform descriptor whose range ends at the last
  // row this tile may touch, so the hardware drops anything past it).  The
  // last, partial tile repeats the last key in rows past the end (finite data
  // that the mask drops).
  // Physical page holding this wave's rows of tile t (paged; clamped rows
  // past the end stay in the same page); an out-of-range entry marks the
  // request bad and reads page 0 instead.
  auto load_pid = [&](int t) -> int {
    int pid = 0;
    if constexpr (PAGED) {
      if constexpr (LP) {
        const int k16 = (min(t * C::BN + wrow0, Lk - 1) >> 4) + blk_off;
        pid = table[k16 >> p.page_shift];
        if ((unsigned)pid >= (unsigned)p.num_pages) { bad = true; pid = 0; }
        pid = pid * (p.kv_hnd ? p.Hkv << p.page_shift : 1 << p.page_shift) +
              (k16 & ((1 << p.page_shift) - 1));
      } else {
        pid = table[min(t * C::BN + wrow0, Lk - 1) >> 4];
        if ((unsigned)pid >= (unsigned)p.num_pages) { bad = true; pid = 0; }
      }
    }
    return pid;
  };
  auto dma = [&](int kt, char* dst, bool is_v, int pid, auto full_tag) {
    const int k0 = kt * C::BN;
    const char* g = is_v ? vg : kg;
    const char* base;
    int nrec;
    if constexpr (PAGED) {
      base = g + (size_t)pid * page_b + (size_t)kvh * head_b;
      nrec = (kPage - 1) * kv_rowb + C::ROWB;
    } else {
      base = g + ((size_t)(k_start + k0) * kv_rowb + (size_t)kvh * C::ROWB);
      nrec = (min(C::BN, Lk - k0) - 1) * kv_rowb + C::ROWB;
    }
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, nrec, kBufferWord3);
    if (decltype(full_tag)::value || kt < t_full) {   // full_tag: known to be a whole tile
#pragma unroll
      for (int i = 0; i < C::DMA; ++i) {
        const int r0i = (wave * C::DMA + i) * RPI;     // first tile row of instruction i
        const int soff = (PAGED ? (r0i & (kPage - 1)) : r0i) * kv_rowb;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (wave * C::DMA + i) * 1024), 16,
                                                 (int)(is_v ? vlane[i] : klane[i]), soff, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < C::DMA; ++i) {
        const int kj = min(k0 + (wave * C::DMA + i) * RPI + lane_row, Lk - 1);
        const int row = PAGED ? (kj & (kPage - 1)) : kj - k0;
        const int o = row * kv_rowb - lane_rowb + (int)(is_v ? vlane[i] : klane[i]);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (wave * C::DMA + i) * 1024), 16,
                                                 o, 0, 0, 0);
      }
    }
  };

  // ---- per-lane LDS read offsets (the buffer and block go in the immediate)
  // K: row l32 of a 32-key block, logical chunk 2 ks + hl.  The swizzle only
  // touches the low four chunk bits, so k-steps 8.. are 256 bytes further on.
  int kro[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) kro[ks] = l32 * C::ROWB + (k_chunk(l32, 2 * ks + hl) << 4);
  const int grp = lane >> 4, gj = lane & 15;
  const int tr_row = 4 * (grp >> 1) + (gj >> 2);       // + 16 ps (+ 8 for the high half)
  const int tr_col = 16 * (grp & 1) + 4 * (gj & 3);    // d within a 32-wide block
  // V: the swizzle touches 64-byte block bits 0-1 only, so 32-wide d blocks
  // 4.. are 256 bytes further on.
  int vro[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int d = db * 32 + tr_col;
    vro[db] = tr_row * C::ROWB + (v_chunk(tr_row, d >> 3) << 4) + (d & 7) * 2;
  }

  f32x16 o[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) o[i] = f32x16{};
  float m = kNegInf, lsum = 0.f;

  const int w_first = r0 + wave * 32;                       // first row of this wave
  const int w_last = min(w_first + 31, Lq - 1);
  const bool wave_rows = w_first < Lq;
  const int pos = my_row + off;   // last visible key index for this lane's query
  // Tiles this wave needs (keys up to its last row's diagonal), and the
  // leading ones in which every row of the wave sees every key (no mask).
  int w_kt = 0, w_fast = 0, w_lead = 0;
  if (wave_rows) {
    // tiles before w_lead hold keys left of some row's window
    if (win >= 0) w_lead = max(0, w_last + off - win + C::BN - 1) / C::BN;
    const int wkend = up ? max(0, min(Lk, w_last + off + rb + 1)) : Lk;
    w_kt = min(n_kt, (wkend + C::BN - 1) / C::BN);
    int lim = t_full;
    if (up) lim = min(lim, max(0, w_first + off + rb + 1) / C::BN);
    w_fast = min(lim, w_kt);
  }

  auto qk = [&](const char* kbuf, f32x16 (&s)[C::KB]) {
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::QK; ++ks)
        s[kb] = mfma32(*reinterpret_cast<const v8*>(kbuf + kb * 32 * C::ROWB + (ks >> 3) * 256 + kro[ks & 7]),
                       qf[ks], s[kb]);
    }
  };

  // Scores past the end of the keys, right of this lane's diagonal or left of
  // its window -> -inf.
  auto mask = [&](int kt, f32x16 (&s)[C::KB]) {
    const int k0 = kt * C::BN;
    const int lim = up ? min(pos + rb, Lk - 1) : Lk - 1;
    const int lo = win >= 0 ? pos - win : 0;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        s[kb][r] = (key > lim || key < lo) ? kNegInf : s[kb][r];
      }
  };

  // Row max of the tile; raise the running max (and rescale O, l) only when
  // some row's tile max passes it by more than the slack.
  auto update_max = [&](f32x16 (&s)[C::KB]) {
    float mr = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mr = fmaxf(mr, s[kb][r]);
    const float mt = max_halves(mr) * c;                 // tile max in log2 units
    const bool raise = mt > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      // Lanes that do not raise keep alpha = 1 (m may still be -inf there);
      // a raise from m = -inf gives alpha = 0.
      const float alpha = raise ? exp2_fast(m - mt) : 1.f;
      m = raise ? mt : m;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
  };

  // P = 2^(s c - m) rounded to the input type (laid out as the B operand of O^T += V^T P^T);
  // the row sum adds the rounded weights, the ones that multiply V.
  auto weights = [&](f32x16 (&s)[C::KB], v8 (&pb)[C::PS], float nm) {
    float psum = 0.f;
    const v2 one = {(elem)1.f, (elem)1.f};
#pragma unroll
    for (int ps = 0; ps < C::PS; ++ps) {
      v8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = (elem)exp2_fast(__builtin_fmaf(s[ps >> 1][(ps & 1) * 8 + e], c, nm));
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        psum = H::dot2(v2{v[e], v[e + 1]}, one, psum);
      pb[ps] = v;
    }
    lsum += psum;
  };

  auto pv = [&](const char* vbuf, v8 (&pb)[C::PS]) {
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int ps = 0; ps < C::PS; ++ps) {
        const int ro = ps * 16 * C::ROWB + (db >> 2) * 256 + vro[db & 3];
        v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)((lds_char*)vbuf + ro));
        v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)((lds_char*)vbuf + ro + 8 * C::ROWB));
        const v8 a = __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = mfma32(a, pb[ps], o[db]);
      }
    }
  };

  // One tile step.  SLOT = kt % R picks the ring slots at compile time: K(kt+1)
  // is in slot kt+1, V(kt) in slot kt; this step starts the DMA of V(kt+R-1)
  // into slot kt-1 and of K(kt+R) into slot kt, both last read in the step
  // before.  FAST steps are the steady state: no row of any wave masks tile
  // kt, and every wave needs tile kt + 1.
  f32x16 sa[C::KB], sb[C::KB];
  int pid_v = 0, pid_k = 0;     // pages of V(kt+R-1) and K(kt+R) for the next step
  auto step = [&](auto slot_tag, auto fast_tag, int kt, f32x16 (&scur)[C::KB],
                  f32x16 (&snext)[C::KB]) {
    constexpr int SLOT = decltype(slot_tag)::value;
    constexpr bool FAST = decltype(fast_tag)::value != 0;
    // 2: a steady-state step whose two DMAs are whole tiles (no clamped rows)
    constexpr int FULL = decltype(fast_tag)::value == 2 ? 1 : 0;
    char* const KDST = kslot(Idx<SLOT>{});
    char* const KNXT = kslot(Idx<SLOT + 1>{});
    char* const VCUR = vslot(Idx<SLOT>{});
    char* const VDST = vslot(Idx<SLOT + C::R - 1>{});
    if (kt + C::R - 1 < n_kt) dma(kt + C::R - 1, VDST, true, pid_v, Idx<FULL>{});
    if (kt + C::R < n_kt) dma(kt + C::R, KDST, false, pid_k, Idx<FULL>{});
    v8 pb[C::PS];
    if constexpr (FAST) {
      // One block in which the S^T(kt+1) MFMAs hide the exponentials of tile kt.
      update_max(scur);
      qk(KNXT, snext);
      weights(scur, pb, -m);                 // m is finite once a tile is unmasked
      pv(VCUR, pb);
      // Issue order: K fragment reads ahead of the S^T MFMAs, each MFMA
      // followed by a share of the vector work, then the V^T fragment reads
      // ahead of the O^T MFMAs.
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);              // 4 K reads
#pragma unroll
      for (int i = 0; i < C::KB * C::QK - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // S^T MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);            // next K read
        __builtin_amdgcn_sched_group_barrier(0x002, C::VALU_PER_QK, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);            // first V reads
        __builtin_amdgcn_sched_group_barrier(0x002, C::VALU_PER_QK, 0);
      }
#pragma unroll
      for (int i = 0; i < C::DB * C::PS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);            // O^T MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);            // V reads ahead
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
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
      if (kt + C::R + 1 < n_kt) pid_k = load_pid(kt + C::R + 1);
    }
    // The next step reads K(kt+2) and V(kt+1), whose DMAs this step issued.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // this wave's LDS reads (and page ids) are done
    // Every wave's DMA for the next step has landed and every read of the
    // slots refilled next has completed.  (A workgroup fence here would also
    // wait for the DMAs still in flight, so the barrier stands alone; the
    // memory clobber keeps the compiler from moving LDS accesses across it.)
    asm volatile("s_barrier" ::: "memory");
  };

  // Steady-state steps: [0, n_fast), a multiple of R.  Wave 0 has the fewest
  // unmasked and needed tiles (its rows come first); waves past the last
  // row compute on zero queries and store nothing.
  int n_fast = t_full;
  if (up) n_fast = min(n_fast, max(0, r0 + off + rb + 1) / C::BN);
  {
    const int wkend0 = up ? max(0, min(Lk, min(r0 + 31, Lq - 1) + off + rb + 1)) : Lk;
    const int w_kt0 = min(n_kt, (wkend0 + C::BN - 1) / C::BN);
    n_fast = max(0, min(n_fast, w_kt0 - 1));
    n_fast -= n_fast % C::R;
  }
  // Leading tiles that some row's window cuts (from the last row, whose
  // window starts latest) run the masked step too; a multiple of R.
  int n_lead = 0;
  if (win >= 0) {
    n_lead = min(n_kt, max(0, r_last + off - win + C::BN - 1) / C::BN);
    n_lead += n_lead % C::R;
  }
  n_fast = max(n_fast, n_lead);

  // prologue: K(0 .. R-1) and V(0 .. R-2) in LDS, S^T(0) in registers
#pragma unroll
  for (int t = 0; t < C::R; ++t) {
    if (t < n_kt) {
      const int pid = load_pid(t);
      char* kd = t == 0 ? kslot(Idx<0>{}) : kslot(Idx<1>{});
      char* vd = t == 0 ? vslot(Idx<0>{}) : vslot(Idx<1>{});
      dma(t, kd, false, pid, Idx<0>{});
      if (t + 1 < C::R) dma(t, vd, true, pid, Idx<0>{});
      else pid_v = pid;
    }
  }
  if (C::R < n_kt) pid_k = load_pid(C::R);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  if (n_kt > 0) qk(k_ring0, sa);
  __syncthreads();   // every wave is done with K(0) before step 0 refills its slot
  int kt = 0;
  for (; kt < n_lead; kt += C::R) {
    step(Idx<0>{}, Idx<0>{}, kt, sa, sb);
    if (kt + 1 < n_kt) step(Idx<1>{}, Idx<0>{}, kt + 1, sb, sa);
  }
  // Steady-state steps whose DMAs (tiles kt + C::R - 1 and kt + C::R) are whole
  // tiles skip the clamped-row addressing of the last, partial tile.
  for (; kt < n_fast && kt + C::R + 1 < t_full; kt += C::R) {
    step(Idx<0>{}, Idx<2>{}, kt, sa, sb);
    step(Idx<1>{}, Idx<2>{}, kt + 1, sb, sa);
  }
  for (; kt < n_fast; kt += C::R) {
    step(Idx<0>{}, Idx<1>{}, kt, sa, sb);
    step(Idx<1>{}, Idx<1>{}, kt + 1, sb, sa);
  }
  for (; kt < n_kt; kt += C::R) {
    step(Idx<0>{}, Idx<0>{}, kt, sa, sb);
    if (kt + 1 < n_kt) step(Idx<1>{}, Idx<0>{}, kt + 1, sb, sa);
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
  if (p.merge_lse == nullptr) {
    // Stage this wave's 32 x D tile through LDS (the K ring is free: every
    // wave is past its last step) and store whole rows, 16 lanes x 16 bytes
    // per row: written straight from the O^T layout, each store instruction
    // would scatter 8-byte pieces over 32 rows.  Chunk q of row r sits at
    // chunk q ^ (r mod 16) so both passes spread over the banks.
    char* stage = (wave < 2 ? k_ring0 : k_ring1) + (wave & 1) * 32 * C::ROWB;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        typename H::v4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (elem)(o[db][a4 * 4 + j] * inv);
        const int q = db * 4 + a4;
        *reinterpret_cast<typename H::v4*>(stage + l32 * C::ROWB + ((q ^ (l32 & 15)) << 4) + hl * 8) = v;
      }
    }
    const int c16 = lane & 15;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = i * 4 + (lane >> 4);
      const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * C::ROWB + ((c16 ^ (r & 15)) << 4));
      const int row = r0 + wave * 32 + r;
      if (row < Lq)
        *reinterpret_cast<u32x4*>(reinterpret_cast<elem*>(p.out) +
                                  ((size_t)(q_start + row) * p.Hq + head) * D + c16 * 8) = x;
    }
    if (hl == 0 && row_ok) p.lse[(size_t)(q_start + my_row) * p.Hq + head] = lse_v;
    return;
  }
  if (!row_ok) return;
  const size_t orow = (size_t)(q_start + my_row) * p.Hq + head;
  elem* og = reinterpret_cast<elem*>(p.out) + orow * D;
  {
    // Merge with another state over disjoint keys: with x = log2 of each
    // normaliser and mx their max, the weights are 2^(x - mx).  Here the
    // accumulator is unnormalised, so its weight per unit is 2^(m - mx).
    // An empty state (lse -inf) contributes nothing; a NaN on either side,
    // or an invalid request, gives NaN.
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
      const float r = 1.f / den;
      wo = ws * r;
      wp *= r;
      lse_v = (mx + log2_fast(den)) * kLn2;
    }
    const elem* pg = reinterpret_cast<const elem*>(p.merge_o) + orow * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = db * 32 + a4 * 8 + hl * 4;
        typename H::v4 v;
        typename H::v4 w{};
        if (wp != 0.f) w = *reinterpret_cast<const typename H::v4*>(pg + d0);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (elem)(o[db][a4 * 4 + j] * wo + (float)w[j] * wp);
        *reinterpret_cast<typename H::v4*>(og + d0) = v;
      }
    }
  }
  if (hl == 0) p.lse[orow] = lse_v;
}

template <typename E, int D, bool PAGED>
hipError_t launch_t(const PrefillParams& p, hipStream_t s) {
  const int total = p.Hq * p.B * p.q_tiles;
  dim3 grid(8 * ((total + 7) / 8));
  if (PAGED && p.page_shift > 0)
    hipLaunchKernelGGL((prefill_kernel<E, D, PAGED, PAGED>), grid, dim3(NT), 0, s, p, p.page_table);
  else
    hipLaunchKernelGGL((prefill_kernel<E, D, PAGED, false>), grid, dim3(NT), 0, s, p, p.page_table);
  return hipGetLastError();
}

}  // namespace

bool prefill_supported(int dtype, int D) { return (dtype == 1 || dtype == 2) && (D == 128 || D == 256); }

template <typename E>
hipError_t launch_e(const PrefillParams& p, bool paged, hipStream_t s) {
  return paged ? launch_t<E, 128, true>(p, s) : launch_t<E, 128, false>(p, s);
}

hipError_t launch_prefill(const PrefillParams& p, int dtype, int D, bool paged, hipStream_t s) {
  if (D == 256) return launch_prefill_d256(p, dtype, paged, s);
  if (D != 128) return hipErrorInvalidValue;
  if (dtype == 1) return launch_e<bf16_t>(p, paged, s);
  if (dtype == 2) return launch_e<f16_t>(p, paged, s);
  return hipErrorInvalidValue;
}

}  // namespace attn
