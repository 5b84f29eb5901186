/*
 * A plain C client of the C ABI (include/attn.h): device memory from
 * hipMalloc, a stream from hipStreamCreate, no Python and no torch.  It
 * shows that the library stands on its own and lets the tests check it end
 * to end against the oracle.
 *
 *   attn_client decode  DIR B Hq Hkv D page_size num_pages max_pages max_kv_len scale
 *     reads  DIR/q.bin [B,Hq,D] bf16, DIR/k.bin DIR/v.bin [num_pages,page_size,Hkv,D] bf16,
 *            DIR/table.bin [B,max_pages] int32, DIR/lens.bin [B] int32
 *   attn_client prefill DIR B Hq Hkv D total_q total_k max_seqlen_q max_seqlen_k causal scale
 *     reads  DIR/q.bin [total_q,Hq,D] bf16, DIR/k.bin DIR/v.bin [total_k,Hkv,D] bf16,
 *            DIR/cuq.bin DIR/cuk.bin [B+1] int32
 *   both write DIR/out.bin (bf16, shaped like q) and DIR/lse.bin (float32, [rows, Hq]).
 *
 * Exit status: 0 on success, 1 on a usage, file or HIP runtime error, 2 when
 * the library returns a status other than ATTN_OK (its text is printed).
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "attn.h"

static int fail_hip(hipError_t e, const char* what) {
  fprintf(stderr, "attn_client: %s: %s\n", what, hipGetErrorString(e));
  return 1;
}

/* Reads exactly `bytes` bytes of DIR/name into a new device buffer. */
static int upload(const char* dir, const char* name, size_t bytes, void** dev) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "attn_client: cannot open %s\n", path);
    return 1;
  }
  void* host = malloc(bytes ? bytes : 1);
  size_t got = bytes ? fread(host, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    fprintf(stderr, "attn_client: %s holds fewer than %zu bytes\n", path, bytes);
    free(host);
    return 1;
  }
  *dev = NULL;
  if (bytes) {
    hipError_t e = hipMalloc(dev, bytes);
    if (e == hipSuccess) e = hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      free(host);
      return fail_hip(e, name);
    }
  }
  free(host);
  return 0;
}

static int download(const char* dir, const char* name, const void* dev, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  void* host = malloc(bytes ? bytes : 1);
  if (bytes) {
    hipError_t e = hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
      free(host);
      return fail_hip(e, name);
    }
  }
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(host, 1, bytes, f) != bytes) {
    fprintf(stderr, "attn_client: cannot write %s\n", path);
    if (f) fclose(f);
    free(host);
    return 1;
  }
  fclose(f);
  free(host);
  return 0;
}

static int report(attn_status s) {
  if (s == ATTN_OK) return 0;
  fprintf(stderr, "attn_client: %s: %s\n", attn_status_string(s), attn_last_error());
  return 2;
}

static int run_decode(const char* dir, char** a) {
  const int B = atoi(a[0]), Hq = atoi(a[1]), Hkv = atoi(a[2]), D = atoi(a[3]);
  const int P = atoi(a[4]), num_pages = atoi(a[5]), max_pages = atoi(a[6]), max_kv = atoi(a[7]);
  const float scale = (float)atof(a[8]);
  const size_t qb = (size_t)B * Hq * D * 2, kvb = (size_t)num_pages * P * Hkv * D * 2;
  void *q, *k, *v, *table, *lens, *out = NULL, *lse = NULL, *ws = NULL;
  if (upload(dir, "q.bin", qb, &q) || upload(dir, "k.bin", kvb, &k) || upload(dir, "v.bin", kvb, &v) ||
      upload(dir, "table.bin", (size_t)B * max_pages * 4, &table) ||
      upload(dir, "lens.bin", (size_t)B * 4, &lens))
    return 1;
  const size_t wsb = attn_decode_paged_workspace_size(ATTN_BF16, B, Hq, Hkv, D, P, max_kv, 0);
  hipError_t e = hipMalloc(&out, qb ? qb : 1);
  if (e == hipSuccess) e = hipMalloc(&lse, (size_t)B * Hq * 4 + 4);
  if (e == hipSuccess && wsb) e = hipMalloc(&ws, wsb);
  if (e != hipSuccess) return fail_hip(e, "hipMalloc");
  hipStream_t s;
  if ((e = hipStreamCreate(&s)) != hipSuccess) return fail_hip(e, "hipStreamCreate");
  const int rc = report(attn_decode_paged(ATTN_BF16, q, k, v, (const int32_t*)table,
                                          (const int32_t*)lens, B, Hq, Hkv, D, P, num_pages,
                                          max_pages, max_kv, 0, scale, out, (float*)lse, ws, wsb,
                                          (void*)s));
  if (rc) return rc;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return fail_hip(e, "decode");
  return download(dir, "out.bin", out, qb) || download(dir, "lse.bin", lse, (size_t)B * Hq * 4);
}

static int run_prefill(const char* dir, char** a) {
  const int B = atoi(a[0]), Hq = atoi(a[1]), Hkv = atoi(a[2]), D = atoi(a[3]);
  const int Tq = atoi(a[4]), Tk = atoi(a[5]), mq = atoi(a[6]), mk = atoi(a[7]), causal = atoi(a[8]);
  const float scale = (float)atof(a[9]);
  const size_t qb = (size_t)Tq * Hq * D * 2, kb = (size_t)Tk * Hkv * D * 2;
  void *q, *k, *v, *cuq, *cuk, *out = NULL, *lse = NULL;
  if (upload(dir, "q.bin", qb, &q) || upload(dir, "k.bin", kb, &k) || upload(dir, "v.bin", kb, &v) ||
      upload(dir, "cuq.bin", (size_t)(B + 1) * 4, &cuq) ||
      upload(dir, "cuk.bin", (size_t)(B + 1) * 4, &cuk))
    return 1;
  hipError_t e = hipMalloc(&out, qb ? qb : 1);
  if (e == hipSuccess) e = hipMalloc(&lse, (size_t)Tq * Hq * 4 + 4);
  if (e != hipSuccess) return fail_hip(e, "hipMalloc");
  hipStream_t s;
  if ((e = hipStreamCreate(&s)) != hipSuccess) return fail_hip(e, "hipStreamCreate");
  const int rc = report(attn_prefill_varlen(ATTN_BF16, q, k, v, (const int32_t*)cuq,
                                            (const int32_t*)cuk, B, Hq, Hkv, D, Tq, Tk, mq, mk,
                                            causal, scale, out, (float*)lse, (void*)s));
  if (rc) return rc;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return fail_hip(e, "prefill");
  return download(dir, "out.bin", out, qb) || download(dir, "lse.bin", lse, (size_t)Tq * Hq * 4);
}

int main(int argc, char** argv) {
  if (argc == 12 && strcmp(argv[1], "decode") == 0) return run_decode(argv[2], argv + 3);
  if (argc == 13 && strcmp(argv[1], "prefill") == 0) return run_prefill(argv[2], argv + 3);
  fprintf(stderr,
          "usage: attn_client decode  DIR B Hq Hkv D page_size num_pages max_pages max_kv_len scale\n"
          "       attn_client prefill DIR B Hq Hkv D total_q total_k max_seqlen_q max_seqlen_k "
          "causal scale\n");
  return 1;
}
