/*
 * A plain C11 client of libxattn (test infrastructure): it includes only xattn.h and
 * the HIP runtime's C API, and links against libxattn.so.
 *
 *   xattn_client --host-only   calls the entry points that need no GPU (schedule,
 *                              validation errors, destroy of NULL) and checks them
 *   xattn_client <dir>         reads a workload from <dir> (meta.txt and raw arrays),
 *                              plans and runs it on device 0 and writes out.bin and
 *                              lse.bin to <dir>
 *
 * meta.txt holds, on one line: batch num_qo_heads num_kv_heads head_dim page_size
 * num_pages mask_mode block_size dtype q_rows has_page_indices has_last_page_len
 * sm_scale. The arrays are qo_indptr.bin and kv_indptr.bin (int32, batch + 1 each),
 * kv_page_indices.bin and kv_last_page_len.bin (int32, when flagged), and q.bin,
 * k.bin, v.bin in the plan's dtype (bf16 as raw 16-bit words). Exit status 0 on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "xattn.h"

static int fail(const char* what) {
  fprintf(stderr, "xattn_client: %s\n", what);
  return 1;
}

static void* read_all(const char* dir, const char* name, size_t* bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  if (fseek(f, 0, SEEK_END) != 0) {
    fclose(f);
    return NULL;
  }
  const long n = ftell(f);
  if (n < 0 || fseek(f, 0, SEEK_SET) != 0) {
    fclose(f);
    return NULL;
  }
  void* p = malloc(n > 0 ? (size_t)n : 1);
  if (p && n > 0 && fread(p, 1, (size_t)n, f) != (size_t)n) {
    free(p);
    p = NULL;
  }
  fclose(f);
  if (p) *bytes = (size_t)n;
  return p;
}

static int write_all(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  const int bad = fwrite(p, 1, bytes, f) != bytes;
  return fclose(f) != 0 || bad;
}

/* The entry points that need no GPU. */
static int host_only(void) {
  /* two requests: query lengths 1 and 3, contexts of 16 and 40 keys in pages of 4 */
  const int32_t qo[3] = {0, 1, 4}, kv[3] = {0, 4, 14}, last[2] = {4, 4};
  int32_t pages[14];
  for (int i = 0; i < 14; ++i) pages[i] = 13 - i;
  xattn_schedule_info info;
  memset(&info, 0, sizeof info);
  int rc = xattn_schedule(qo, kv, pages, last, 2, 2, 2, 16, 4, 14, XATTN_MASK_NONE, 0, XATTN_F32, 0,
                          &info, NULL, NULL);
  if (rc != XATTN_OK) return fail("xattn_schedule rejected a valid workload");
  if (info.total_kv_tokens != 56) return fail("total_kv_tokens != 56");
  /* every query sees its whole context: (1 * 16 + 3 * 40) keys x 2 heads */
  if (info.visible_pairs != 272) return fail("visible_pairs != 272");

  /* 3 query heads over 2 KV heads: rejected in validation, with a message */
  rc = xattn_schedule(qo, kv, pages, last, 2, 3, 2, 16, 4, 14, XATTN_MASK_NONE, 0, XATTN_F32, 0,
                      &info, NULL, NULL);
  if (rc != XATTN_ERR_INVALID_ARG) return fail("head counts 3/2 not rejected");
  if (strlen(xattn_last_error()) == 0) return fail("no message for a rejected schedule");

  /* bf16 supports head_dim 64 and 128 only */
  rc = xattn_schedule(qo, kv, pages, last, 2, 2, 2, 16, 4, 14, XATTN_MASK_NONE, 0, XATTN_BF16, 0,
                      &info, NULL, NULL);
  if (rc != XATTN_ERR_UNSUPPORTED) return fail("bf16 head_dim 16 not reported unsupported");

  /* a last-page length past page_size: xattn_plan fails before creating a handle */
  const int32_t bad_last[2] = {4, 9};
  xattn_plan_t h = NULL;
  rc = xattn_plan(&h, qo, kv, pages, bad_last, 2, 2, 2, 16, 4, 14, XATTN_MASK_NONE, 0, 0.f, XATTN_F32,
                  NULL);
  if (rc != XATTN_ERR_INVALID_ARG || h != NULL) return fail("bad kv_last_page_len not rejected");

  xattn_plan_destroy(NULL);
  printf("host-only ok\n");
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 2) return fail("usage: xattn_client --host-only | xattn_client <dir>");
  if (strcmp(argv[1], "--host-only") == 0) return host_only();
  const char* dir = argv[1];

  size_t n = 0;
  char* meta = (char*)read_all(dir, "meta.txt", &n);
  if (!meta) return fail("cannot read meta.txt");
  char* text = (char*)realloc(meta, n + 1);
  if (!text) return fail("out of memory");
  text[n] = '\0';
  int b, hq, hkv, d, ps, mask, block, dtype, q_rows, has_pages, has_last;
  long long num_pages;
  float scale;
  const int got = sscanf(text, "%d %d %d %d %d %lld %d %d %d %d %d %d %f", &b, &hq, &hkv, &d, &ps,
                         &num_pages, &mask, &block, &dtype, &q_rows, &has_pages, &has_last, &scale);
  free(text);
  if (got != 13 || b < 0 || hq < 1 || hkv < 1 || d < 1 || ps < 1 || num_pages < 0 || q_rows < 0)
    return fail("bad meta.txt");

  size_t nb;
  int32_t* qo = (int32_t*)read_all(dir, "qo_indptr.bin", &nb);
  if (!qo || nb != (size_t)(b + 1) * 4) return fail("bad qo_indptr.bin");
  int32_t* kv = (int32_t*)read_all(dir, "kv_indptr.bin", &nb);
  if (!kv || nb != (size_t)(b + 1) * 4) return fail("bad kv_indptr.bin");
  if (qo[b] != q_rows) return fail("qo_indptr does not end at q_rows");
  int32_t* pages = NULL;
  if (has_pages) {
    pages = (int32_t*)read_all(dir, "kv_page_indices.bin", &nb);
    if (!pages || nb != (size_t)kv[b] * 4) return fail("bad kv_page_indices.bin");
  }
  int32_t* last = NULL;
  if (has_last) {
    last = (int32_t*)read_all(dir, "kv_last_page_len.bin", &nb);
    if (!last || nb != (size_t)b * 4) return fail("bad kv_last_page_len.bin");
  }
  const size_t elt = dtype == XATTN_BF16 ? 2 : 4;
  const size_t q_bytes = (size_t)q_rows * hq * d * elt;
  const size_t pool_bytes = (size_t)num_pages * ps * hkv * d * elt;
  size_t qb, kb, vb;
  void* hq_host = read_all(dir, "q.bin", &qb);
  void* hk_host = read_all(dir, "k.bin", &kb);
  void* hv_host = read_all(dir, "v.bin", &vb);
  if (!hq_host || !hk_host || !hv_host || qb != q_bytes || kb != pool_bytes || vb != pool_bytes)
    return fail("bad q.bin, k.bin or v.bin");

  void *dq = NULL, *dk = NULL, *dv = NULL, *dout = NULL;
  float* dlse = NULL;
  const size_t lse_bytes = (size_t)q_rows * hq * sizeof(float);
  if (hipMalloc(&dq, q_bytes ? q_bytes : 16) != hipSuccess || hipMalloc(&dk, pool_bytes ? pool_bytes : 16) != hipSuccess ||
      hipMalloc(&dv, pool_bytes ? pool_bytes : 16) != hipSuccess || hipMalloc(&dout, q_bytes ? q_bytes : 16) != hipSuccess ||
      hipMalloc((void**)&dlse, lse_bytes ? lse_bytes : 16) != hipSuccess)
    return fail("hipMalloc failed");
  if (hipMemcpy(dq, hq_host, q_bytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dk, hk_host, pool_bytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dv, hv_host, pool_bytes, hipMemcpyHostToDevice) != hipSuccess)
    return fail("hipMemcpy to the device failed");

  xattn_plan_t h = NULL;
  int rc = xattn_plan(&h, qo, kv, pages, last, b, hq, hkv, d, ps, num_pages, mask, block, scale, dtype, NULL);
  if (rc != XATTN_OK) {
    fprintf(stderr, "xattn_plan: %d %s\n", rc, xattn_last_error());
    return 1;
  }
  rc = xattn_run(h, dq, dk, dv, dout, dlse, NULL);
  if (rc != XATTN_OK) {
    fprintf(stderr, "xattn_run: %d %s\n", rc, xattn_last_error());
    return 1;
  }
  if (hipDeviceSynchronize() != hipSuccess) return fail("hipDeviceSynchronize failed");
  void* hout = malloc(q_bytes ? q_bytes : 1);
  float* hlse = (float*)malloc(lse_bytes ? lse_bytes : 1);
  if (!hout || !hlse) return fail("out of memory");
  if (hipMemcpy(hout, dout, q_bytes, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(hlse, dlse, lse_bytes, hipMemcpyDeviceToHost) != hipSuccess)
    return fail("hipMemcpy from the device failed");
  xattn_plan_destroy(h);
  if (write_all(dir, "out.bin", hout, q_bytes) || write_all(dir, "lse.bin", hlse, lse_bytes))
    return fail("cannot write the outputs");
  (void)hipFree(dq);
  (void)hipFree(dk);
  (void)hipFree(dv);
  (void)hipFree(dout);
  (void)hipFree(dlse);
  free(hout);
  free(hlse);
  free(hq_host);
  free(hk_host);
  free(hv_host);
  free(qo);
  free(kv);
  free(pages);
  free(last);
  printf("ran %d requests\n", b);
  return 0;
}
