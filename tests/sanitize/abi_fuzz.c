/*
 * Argument fuzz of the C ABI for a host build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure; no GPU needed).
 *
 * Every entry point is called from a valid base configuration, then with each
 * integer argument replaced in turn by edge values (negative, zero, powers of
 * two and their neighbours, the 2^30 token limit, INT_MAX and INT_MIN), then
 * with many random mixtures of edge values, non-finite and extreme floats,
 * NULL and misaligned pointers.  Device pointers are fake addresses that host
 * code must never dereference (a dereference is a segmentation fault the
 * sanitizer reports).  Without a GPU, a call that passes every check fails at
 * its launch with ATTN_E_HIP; with a GPU visible the program exits (77)
 * without calling anything, since such a call would launch a kernel on the
 * fake addresses.
 *
 * Checked on every call: the status is one of attn_status; a failing call
 * leaves a non-empty attn_last_error(); attn_last_hip_error() is non-empty
 * exactly when the status is ATTN_E_HIP; a decode or cascade call given the
 * workspace its size query reports never returns ATTN_E_WORKSPACE, and the
 * allocation-free decode returns it exactly when that size exceeds the static
 * scratch.  The sanitizers abort the run on any memory error or undefined
 * behaviour (signed overflow, bad shift, misaligned access, ...).
 */
#include "attn.h"

#include <hip/hip_runtime_api.h>

#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static const int kEdge[] = {INT_MIN, INT_MIN + 1, -65536, -2, -1, 0, 1, 2, 3, 4, 7, 8, 15, 16,
                            17, 31, 32, 63, 64, 96, 127, 128, 129, 255, 256, 257, 4096, 65535,
                            65536, 1 << 24, (1 << 30) - 1, 1 << 30, (1 << 30) + 1,
                            INT_MAX - 256, INT_MAX - 8, INT_MAX - 1, INT_MAX};
#define NEDGE ((int)(sizeof kEdge / sizeof kEdge[0]))
static const float kFloat[] = {0.0883883f, 1.f, 0.f, -0.f, -1.f, 1e-30f, 1e30f, FLT_MAX,
                               -FLT_MAX, INFINITY, -INFINITY, NAN};
#define NFLOAT ((int)(sizeof kFloat / sizeof kFloat[0]))

static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(uint32_t n) {
  g_rng ^= g_rng << 13;
  g_rng ^= g_rng >> 7;
  g_rng ^= g_rng << 17;
  return (uint32_t)(g_rng >> 11) % n;
}

/* Fake device addresses, 256-byte aligned and distinct. */
#define NPTR 10
static void* g_ptr[NPTR];
static void reset_ptrs(void) {
  for (int i = 0; i < NPTR; ++i) g_ptr[i] = (void*)(uintptr_t)(0x10000000u + 0x100000u * (unsigned)i);
}

static long g_calls = 0, g_failures = 0;
static long g_status[ATTN_E_HIP + 1];

static void check(const char* name, attn_status st, const int* a, int n) {
  ++g_calls;
  if ((int)st >= ATTN_OK && (int)st <= ATTN_E_HIP) ++g_status[st];
  const char* why = NULL;
  const char* msg = attn_last_error();
  const char* hip = attn_last_hip_error();
  if ((int)st < ATTN_OK || (int)st > ATTN_E_HIP) why = "status outside attn_status";
  else if (st != ATTN_OK && (msg == NULL || msg[0] == 0)) why = "failure without attn_last_error text";
  else if (hip == NULL || ((st == ATTN_E_HIP) != (hip[0] != 0))) why = "attn_last_hip_error inconsistent with the status";
  else if (attn_status_string(st) == NULL) why = "no status string";
  if (why) {
    ++g_failures;
    if (g_failures <= 20) {
      fprintf(stderr, "FAIL %s: %s (status %d, '%s'); ints:", name, why, (int)st, msg ? msg : "(null)");
      for (int i = 0; i < n; ++i) fprintf(stderr, " %d", a[i]);
      fprintf(stderr, "\n");
    }
  }
}

static void expect(int cond, const char* name, const char* what, const int* a, int n) {
  if (cond) return;
  ++g_failures;
  if (g_failures <= 20) {
    fprintf(stderr, "FAIL %s: %s; ints:", name, what);
    for (int i = 0; i < n; ++i) fprintf(stderr, " %d", a[i]);
    fprintf(stderr, " (%s)\n", attn_last_error());
  }
}

/* ---- decode family ---------------------------------------------------- */
/* ints: dtype B Hq Hkv D page_size num_pages max_pages_per_req max_kv_len split_pages kv_layout window_left */
enum { DT, DB, DHQ, DHKV, DD, DPS, DNP, DMP, DMKV, DSP, DLAY, DWIN, DN };
/* floats: scale k_scale v_scale rope_theta rope_scale */
enum { FS, FK, FV, FT, FR, FN };

typedef enum { DEC, DEC_HND, DEC_WIN, DEC_ROPE, DEC_FP8, DEC_FP8_HND, DEC_FP8_WIN, DEC_NOALLOC, DEC_KINDS } dec_kind;
static const char* kDecName[DEC_KINDS] = {"decode_paged", "decode_paged_hnd", "decode_paged_window",
                                          "decode_paged_rope", "decode_paged_fp8", "decode_paged_fp8_hnd",
                                          "decode_paged_fp8_window", "decode_paged_noalloc"};

static attn_status call_decode(dec_kind k, const int* a, const float* f, size_t ws_bytes) {
  void** p = g_ptr;
  const attn_dtype dt = (attn_dtype)a[DT];
  switch (k) {
    case DEC:
      return attn_decode_paged(dt, p[0], p[1], p[2], (const int32_t*)p[3], (const int32_t*)p[4], a[DB], a[DHQ],
                               a[DHKV], a[DD], a[DPS], a[DNP], a[DMP], a[DMKV], a[DSP], f[FS], p[5],
                               (float*)p[6], p[7], ws_bytes, NULL);
    case DEC_HND:
      return attn_decode_paged_hnd(dt, p[0], p[1], p[2], (const int32_t*)p[3], (const int32_t*)p[4], a[DB],
                                   a[DHQ], a[DHKV], a[DD], a[DPS], a[DNP], a[DMP], a[DMKV], a[DSP], f[FS],
                                   p[5], (float*)p[6], p[7], ws_bytes, NULL);
    case DEC_WIN:
      return attn_decode_paged_window(dt, a[DLAY], a[DWIN], p[0], p[1], p[2], (const int32_t*)p[3],
                                      (const int32_t*)p[4], a[DB], a[DHQ], a[DHKV], a[DD], a[DPS], a[DNP],
                                      a[DMP], a[DMKV], a[DSP], f[FS], p[5], (float*)p[6], p[7], ws_bytes,
                                      NULL);
    case DEC_ROPE:
      return attn_decode_paged_rope(dt, a[DLAY], a[DWIN], f[FT], f[FR], p[0], p[1], p[2],
                                    (const int32_t*)p[3], (const int32_t*)p[4], a[DB], a[DHQ], a[DHKV], a[DD],
                                    a[DPS], a[DNP], a[DMP], a[DMKV], a[DSP], f[FS], p[5], (float*)p[6], p[7],
                                    ws_bytes, NULL);
    case DEC_FP8:
      return attn_decode_paged_fp8(dt, p[0], p[1], p[2], (const int32_t*)p[3], (const int32_t*)p[4], a[DB],
                                   a[DHQ], a[DHKV], a[DD], a[DPS], a[DNP], a[DMP], a[DMKV], a[DSP], f[FS],
                                   f[FK], f[FV], p[5], (float*)p[6], p[7], ws_bytes, NULL);
    case DEC_FP8_HND:
      return attn_decode_paged_fp8_hnd(dt, p[0], p[1], p[2], (const int32_t*)p[3], (const int32_t*)p[4],
                                       a[DB], a[DHQ], a[DHKV], a[DD], a[DPS], a[DNP], a[DMP], a[DMKV],
                                       a[DSP], f[FS], f[FK], f[FV], p[5], (float*)p[6], p[7], ws_bytes,
                                       NULL);
    case DEC_FP8_WIN:
      return attn_decode_paged_fp8_window(dt, a[DLAY], a[DWIN], p[0], p[1], p[2], (const int32_t*)p[3],
                                          (const int32_t*)p[4], a[DB], a[DHQ], a[DHKV], a[DD], a[DPS],
                                          a[DNP], a[DMP], a[DMKV], a[DSP], f[FS], f[FK], f[FV], p[5],
                                          (float*)p[6], p[7], ws_bytes, NULL);
    case DEC_NOALLOC:
    default:
      return attn_decode_paged_noalloc(dt, p[0], p[1], p[2], (const int32_t*)p[3], (const int32_t*)p[4],
                                       a[DB], a[DHQ], a[DHKV], a[DD], a[DPS], a[DNP], a[DMP], a[DMKV],
                                       a[DSP], f[FS], p[5], (float*)p[6], NULL);
  }
}

static void run_decode(dec_kind k, const int* a, const float* f, int ws_mode) {
  const size_t need = attn_decode_paged_workspace_size((attn_dtype)a[DT], a[DB], a[DHQ], a[DHKV], a[DD],
                                                       a[DPS], a[DMKV], a[DSP]);
  size_t bytes = ws_mode == 0 ? need : ws_mode == 1 ? 0 : SIZE_MAX;
  const attn_status st = call_decode(k, a, f, bytes);
  check(kDecName[k], st, a, DN);
  if (k == DEC_NOALLOC) {
    /* Reached the workspace check: a partial state larger than the scratch
       array is the only ATTN_E_WORKSPACE of this entry point. */
    if (st == ATTN_E_WORKSPACE)
      expect(need > (size_t)ATTN_DECODE_NOALLOC_SCRATCH_BYTES, kDecName[k],
             "E_WORKSPACE although the plan fits the scratch array", a, DN);
  } else if (ws_mode == 0 && need != SIZE_MAX && g_ptr[7] != NULL) {
    expect(st != ATTN_E_WORKSPACE, kDecName[k], "E_WORKSPACE with the queried workspace size", a, DN);
  }
}

static const int kDecBase[][DN] = {
    /* dtype B  Hq Hkv D   P    pages  mp  mkv   sp lay win */
    {1, 4, 32, 8, 128, 16, 1024, 64, 1000, 0, 0, -1},
    {2, 3, 8, 8, 64, 64, 300, 20, 1200, 0, 1, 100},
    {1, 1, 16, 2, 256, 256, 40, 40, 10000, 8, 0, 4095},
    {0, 5, 8, 1, 128, 16, 500, 100, 1600, 0, 0, -1},
    {0, 2, 4, 4, 64, 16, 100, 50, 800, 4, 0, 31},
};
#define NDECBASE ((int)(sizeof kDecBase / sizeof kDecBase[0]))

static void fuzz_decode(int random_rounds) {
  const float f0[FN] = {0.0883883f, 0.5f, 2.f, 10000.f, 1.f};
  for (int k = 0; k < DEC_KINDS; ++k) {
    for (int b = 0; b < NDECBASE; ++b) {
      int a[DN];
      float f[FN];
      memcpy(f, f0, sizeof f);
      memcpy(a, kDecBase[b], sizeof a);
      reset_ptrs();
      /* A base configuration passes every host check: without a GPU it
         fails only at the HIP runtime. */
      expect(call_decode((dec_kind)k, a, f,
                         attn_decode_paged_workspace_size((attn_dtype)a[DT], a[DB], a[DHQ], a[DHKV], a[DD],
                                                          a[DPS], a[DMKV], a[DSP])) == ATTN_E_HIP ||
                 (k == DEC_ROPE && (a[DT] == 0 || a[DD] == 256)) ||
                 ((k == DEC_FP8 || k == DEC_FP8_HND || k == DEC_FP8_WIN) && a[DT] == 0),
             kDecName[k], "base configuration does not reach the launch", a, DN);
      for (int m = 0; m < 3; ++m) run_decode((dec_kind)k, a, f, m);
      for (int i = 0; i < DN; ++i)
        for (int e = 0; e < NEDGE; ++e) {
          memcpy(a, kDecBase[b], sizeof a);
          a[i] = kEdge[e];
          run_decode((dec_kind)k, a, f, 0);
        }
      for (int j = 0; j < FN; ++j)
        for (int e = 0; e < NFLOAT; ++e) {
          memcpy(a, kDecBase[b], sizeof a);
          memcpy(f, f0, sizeof f);
          f[j] = kFloat[e];
          run_decode((dec_kind)k, a, f, 0);
        }
    }
    for (int r = 0; r < random_rounds; ++r) {
      int a[DN];
      float f[FN];
      memcpy(a, kDecBase[rnd(NDECBASE)], sizeof a);
      memcpy(f, f0, sizeof f);
      for (int i = 0; i < DN; ++i)
        if (rnd(3) == 0) a[i] = kEdge[rnd(NEDGE)];
      for (int j = 0; j < FN; ++j)
        if (rnd(6) == 0) f[j] = kFloat[rnd(NFLOAT)];
      reset_ptrs();
      const uint32_t pm = rnd(8);
      if (pm == 0) g_ptr[rnd(8)] = NULL;
      if (pm == 1) g_ptr[rnd(8)] = (char*)g_ptr[0] + 8;
      run_decode((dec_kind)k, a, f, (int)rnd(3));
    }
  }
  reset_ptrs();
}

/* ---- prefill family --------------------------------------------------- */
/* ints: dtype B Hq Hkv D total_q total_k max_seqlen_q max_seqlen_k causal
         page_size num_pages max_pages_per_req max_kv_len kv_layout window_left window_right shared_prefix */
enum { PT, PB, PHQ, PHKV, PD, PTQ, PTK, PMQ, PMK, PC, PPS, PNP, PMP, PMKV, PLAY, PWL, PWR, PSP, PN };
typedef enum { VARLEN, VARLEN_WIN, PAGED, PAGED_HND, PAGED_WIN, CASCADE, CASCADE_HND, PRE_KINDS } pre_kind;
static const char* kPreName[PRE_KINDS] = {"prefill_varlen", "prefill_varlen_window", "prefill_paged",
                                          "prefill_paged_hnd", "prefill_paged_window",
                                          "prefill_paged_cascade", "prefill_paged_cascade_hnd"};

static attn_status call_prefill(pre_kind k, const int* a, float scale, size_t ws_bytes) {
  void** p = g_ptr;
  const attn_dtype dt = (attn_dtype)a[PT];
  const int32_t* cq = (const int32_t*)p[3];
  const int32_t* ck = (const int32_t*)p[4];
  const int32_t* table = (const int32_t*)p[8];
  const int32_t* lens = (const int32_t*)p[9];
  switch (k) {
    case VARLEN:
      return attn_prefill_varlen(dt, p[0], p[1], p[2], cq, ck, a[PB], a[PHQ], a[PHKV], a[PD], a[PTQ], a[PTK],
                                 a[PMQ], a[PMK], a[PC], scale, p[5], (float*)p[6], NULL);
    case VARLEN_WIN:
      return attn_prefill_varlen_window(dt, p[0], p[1], p[2], cq, ck, a[PB], a[PHQ], a[PHKV], a[PD], a[PTQ],
                                        a[PTK], a[PMQ], a[PMK], a[PC], a[PWL], a[PWR], scale, p[5],
                                        (float*)p[6], NULL);
    case PAGED:
      return attn_prefill_paged(dt, p[0], cq, p[1], p[2], table, lens, a[PB], a[PHQ], a[PHKV], a[PD], a[PTQ],
                                a[PPS], a[PNP], a[PMP], a[PMQ], a[PMKV], a[PC], scale, p[5], (float*)p[6],
                                NULL);
    case PAGED_HND:
      return attn_prefill_paged_hnd(dt, p[0], cq, p[1], p[2], table, lens, a[PB], a[PHQ], a[PHKV], a[PD],
                                    a[PTQ], a[PPS], a[PNP], a[PMP], a[PMQ], a[PMKV], a[PC], scale, p[5],
                                    (float*)p[6], NULL);
    case PAGED_WIN:
      return attn_prefill_paged_window(dt, a[PLAY], p[0], cq, p[1], p[2], table, lens, a[PB], a[PHQ], a[PHKV],
                                       a[PD], a[PTQ], a[PPS], a[PNP], a[PMP], a[PMQ], a[PMKV], a[PC], a[PWL],
                                       a[PWR], scale, p[5], (float*)p[6], NULL);
    case CASCADE:
      return attn_prefill_paged_cascade(dt, p[0], cq, p[1], p[2], table, lens, a[PB], a[PHQ], a[PHKV], a[PD],
                                        a[PTQ], a[PPS], a[PNP], a[PMP], a[PMQ], a[PMKV], a[PSP], a[PC], scale,
                                        p[5], (float*)p[6], p[7], ws_bytes, NULL);
    case CASCADE_HND:
    default:
      return attn_prefill_paged_cascade_hnd(dt, p[0], cq, p[1], p[2], table, lens, a[PB], a[PHQ], a[PHKV],
                                            a[PD], a[PTQ], a[PPS], a[PNP], a[PMP], a[PMQ], a[PMKV], a[PSP],
                                            a[PC], scale, p[5], (float*)p[6], p[7], ws_bytes, NULL);
  }
}

static void run_prefill(pre_kind k, const int* a, float scale, int ws_mode) {
  const size_t need = attn_prefill_paged_cascade_workspace_size((attn_dtype)a[PT], a[PTQ], a[PHQ], a[PD]);
  const size_t bytes = ws_mode == 0 ? need : ws_mode == 1 ? 0 : SIZE_MAX;
  const attn_status st = call_prefill(k, a, scale, bytes);
  check(kPreName[k], st, a, PN);
  if ((k == CASCADE || k == CASCADE_HND) && ws_mode == 0 && need != SIZE_MAX && g_ptr[7] != NULL)
    expect(st != ATTN_E_WORKSPACE, kPreName[k], "E_WORKSPACE with the queried workspace size", a, PN);
}

static const int kPreBase[][PN] = {
    /* dt B Hq Hkv D  tq   tk   mq   mk  c  P   pages mp  mkv  lay wl   wr  sp */
    {1, 3, 8, 2, 128, 700, 900, 300, 400, 1, 16, 200, 40, 600, 0, -1, -1, 256},
    {2, 2, 16, 16, 256, 512, 512, 256, 256, 0, 64, 64, 32, 2048, 1, 127, 3, 1024},
    {1, 1, 4, 1, 128, 129, 4096, 129, 4096, 1, 256, 16, 16, 4096, 0, 1000, 0, 512},
};
#define NPREBASE ((int)(sizeof kPreBase / sizeof kPreBase[0]))

static void fuzz_prefill(int random_rounds) {
  for (int k = 0; k < PRE_KINDS; ++k) {
    for (int b = 0; b < NPREBASE; ++b) {
      int a[PN];
      memcpy(a, kPreBase[b], sizeof a);
      reset_ptrs();
      expect(call_prefill((pre_kind)k, a, 0.0883883f,
                          attn_prefill_paged_cascade_workspace_size((attn_dtype)a[PT], a[PTQ], a[PHQ],
                                                                    a[PD])) == ATTN_E_HIP,
             kPreName[k], "base configuration does not reach the launch", a, PN);
      for (int m = 0; m < 3; ++m) run_prefill((pre_kind)k, a, 0.0883883f, m);
      for (int i = 0; i < PN; ++i)
        for (int e = 0; e < NEDGE; ++e) {
          memcpy(a, kPreBase[b], sizeof a);
          a[i] = kEdge[e];
          run_prefill((pre_kind)k, a, 0.0883883f, 0);
        }
      for (int e = 0; e < NFLOAT; ++e) {
        memcpy(a, kPreBase[b], sizeof a);
        run_prefill((pre_kind)k, a, kFloat[e], 0);
      }
    }
    for (int r = 0; r < random_rounds; ++r) {
      int a[PN];
      memcpy(a, kPreBase[rnd(NPREBASE)], sizeof a);
      for (int i = 0; i < PN; ++i)
        if (rnd(3) == 0) a[i] = kEdge[rnd(NEDGE)];
      reset_ptrs();
      const uint32_t pm = rnd(8);
      if (pm == 0) g_ptr[rnd(NPTR)] = NULL;
      if (pm == 1) g_ptr[rnd(NPTR)] = (char*)g_ptr[0] + 8;
      run_prefill((pre_kind)k, a, rnd(8) == 0 ? kFloat[rnd(NFLOAT)] : 0.0883883f, (int)rnd(3));
    }
  }
  reset_ptrs();
}

/* ---- merge, size queries, timing, text -------------------------------- */
static void fuzz_misc(int random_rounds) {
  /* ints: dtype rows D */
  const int base[3] = {1, 1000, 128};
  for (int i = 0; i < 3; ++i)
    for (int e = 0; e < NEDGE; ++e) {
      int a[3] = {base[0], base[1], base[2]};
      a[i] = kEdge[e];
      for (int pm = 0; pm < 3; ++pm) {
        reset_ptrs();
        if (pm == 1) g_ptr[rnd(6)] = NULL;
        if (pm == 2) g_ptr[rnd(3) * 2] = (char*)g_ptr[0] + 8;
        void** p = g_ptr;
        const attn_status st = attn_merge_states((attn_dtype)a[0], p[0], (const float*)p[1], p[2],
                                                 (const float*)p[3], a[1], a[2], p[4], (float*)p[5], NULL);
        check("merge_states", st, a, 3);
      }
    }
  for (int r = 0; r < random_rounds; ++r) {
    int a[8];
    for (int i = 0; i < 8; ++i) a[i] = kEdge[rnd(NEDGE)];
    (void)attn_decode_paged_workspace_size((attn_dtype)(a[0] & 3), a[1], a[2], a[3], a[4], a[5], a[6], a[7]);
    (void)attn_prefill_paged_cascade_workspace_size((attn_dtype)(a[0] & 3), a[1], a[2], a[3]);
    (void)attn_decode_paged_workspace_size((attn_dtype)a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7]);
    ++g_calls;
  }
  /* The size queries saturate instead of wrapping. */
  {
    const int a[1] = {0};
    expect(attn_decode_paged_workspace_size(ATTN_BF16, INT_MAX, INT_MAX, 1, INT_MAX, 16, INT_MAX, 0) == SIZE_MAX,
           "decode_paged_workspace_size", "no saturation at SIZE_MAX", a, 1);
    expect(attn_decode_paged_workspace_size(ATTN_F32, INT_MAX, INT_MAX, 1, INT_MAX, 16, INT_MAX, 1) == SIZE_MAX,
           "decode_paged_workspace_size", "no saturation at SIZE_MAX (f32)", a, 1);
    expect(attn_prefill_paged_cascade_workspace_size(ATTN_F32, INT_MAX, INT_MAX, INT_MAX) == SIZE_MAX,
           "prefill_paged_cascade_workspace_size", "no saturation at SIZE_MAX", a, 1);
  }
  for (int e = 0; e < NEDGE; ++e) {
    const int cap = kEdge[e];
    /* Capacities above the limit must be refused without creating events. */
    if (cap > 0 && cap <= ATTN_TIMING_MAX_LAUNCHES && cap > 64) continue;
    const attn_status st = attn_timing_begin(cap);
    check("timing_begin", st, &cap, 1);
    if (cap <= 0 || cap > ATTN_TIMING_MAX_LAUNCHES)
      expect(st == ATTN_E_SHAPE, "timing_begin", "capacity outside the limit not refused", &cap, 1);
    double ms[ATTN_KERNEL_KINDS];
    int n[ATTN_KERNEL_KINDS];
    check("timing_end", attn_timing_end(ms, n), &cap, 1);
    check("timing_end", attn_timing_end(NULL, NULL), &cap, 1);
  }
  for (int s = -3; s < 12; ++s) {
    const char* t = attn_status_string((attn_status)s);
    const int a[1] = {s};
    expect(t != NULL && strlen(t) > 0, "status_string", "empty text", a, 1);
    const char* kn = attn_kernel_name((attn_kernel_kind)s);
    expect(kn != NULL && strlen(kn) > 0, "kernel_name", "empty text", a, 1);
  }
}

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? atoi(argv[1]) : 3000;
  /* Calls that pass the host checks launch kernels on fake addresses: run
     only where the HIP runtime sees no device. */
  int devices = 0;
  if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
    printf("abi_fuzz: %d GPU(s) visible; this fuzz runs only without a GPU\n", devices);
    return 77;
  }
  reset_ptrs();
  fuzz_decode(rounds);
  fuzz_prefill(rounds);
  fuzz_misc(rounds);
  printf("abi_fuzz: %ld calls, %ld failures; statuses:", g_calls, g_failures);
  for (int i = 0; i <= ATTN_E_HIP; ++i) printf(" %s=%ld", attn_status_string((attn_status)i), g_status[i]);
  printf("\n");
  return g_failures == 0 ? 0 : 1;
}
