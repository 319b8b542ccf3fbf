// Drives every host-side validation path of the C ABI (include/infini_attn.h)
// on a machine without a GPU, for a build of the host code instrumented with
// AddressSanitizer and UndefinedBehaviorSanitizer: descriptor and argument
// checks, workspace sizing at extreme sizes (where 32-bit arithmetic would
// overflow), handle creation without a device, null handles on every entry
// point, and the status strings. Exits non-zero on any unexpected status; the
// sanitizers abort on any memory or undefined-behaviour error they detect.
#include <limits.h>
#include <stdio.h>
#include <string.h>

#include "infini_attn.h"

static int failures = 0;

static void expect(const char *what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

static infini_attn_desc base() {
  infini_attn_desc d;
  memset(&d, 0, sizeof(d));
  d.batch = 1;
  d.n_q_heads = 32;
  d.n_kv_heads = 8;
  d.seq_len = 32768;
  d.d_k = 128;
  d.d_v = 128;
  d.dtype = INFINI_ATTN_BF16;
  d.eps = 1e-6f;
  d.stream = NULL;
  d.device = 0;
  return d;
}

int main() {
  infini_attn_desc d = base();
  expect("check valid", infini_attn_check(&d, 2048, INFINI_ATTN_DELTA), INFINI_ATTN_OK);
  expect("check null desc", infini_attn_check(NULL, 64, 0), INFINI_ATTN_ERR_INVALID);
  expect("check seg_len 0", infini_attn_check(&d, 0, 0), INFINI_ATTN_ERR_INVALID);
  expect("check seg_len max", infini_attn_check(&d, INT32_MAX, 1), INFINI_ATTN_OK);
  expect("check bad mode", infini_attn_check(&d, 64, 7), INFINI_ATTN_ERR_INVALID);
  {
    infini_attn_desc e = d;
    e.n_kv_heads = 3;
    expect("check heads not divisible", infini_attn_check(&e, 64, 0), INFINI_ATTN_ERR_INVALID);
    e = d;
    e.d_k = e.d_v = 96;
    expect("check d=96", infini_attn_check(&e, 64, 0), INFINI_ATTN_ERR_UNSUPPORTED);
    e = d;
    e.eps = 0.f;
    expect("check eps 0", infini_attn_check(&e, 64, 0), INFINI_ATTN_ERR_INVALID);
    e = d;
    e.seq_len = (1 << 30) + 1;
    expect("check L > 2^30", infini_attn_check(&e, 1 << 30, 0), INFINI_ATTN_ERR_UNSUPPORTED);
    e = d;
    e.seq_len = 1 << 30;
    expect("check 2^30 rows in 1 segment", infini_attn_check(&e, INT32_MAX, 0), INFINI_ATTN_OK);
    expect("check 2^30 rows, 2^15 segments", infini_attn_check(&e, 1 << 15, 0), INFINI_ATTN_OK);
    expect("check too many segments", infini_attn_check(&e, 1, 0), INFINI_ATTN_ERR_UNSUPPORTED);
    e = d;
    e.batch = 65535;
    e.n_q_heads = 2;
    e.n_kv_heads = 1;
    expect("check B*Hq > 65535", infini_attn_check(&e, 64, 0), INFINI_ATTN_ERR_UNSUPPORTED);
  }

  // Workspace sizes at the extremes: the largest descriptor the checks accept.
  size_t bytes = 0;
  expect("workspace null out", infini_attn_workspace_size(&d, 2048, NULL), INFINI_ATTN_ERR_INVALID);
  expect("workspace 8B shape", infini_attn_workspace_size(&d, 2048, &bytes), INFINI_ATTN_OK);
  size_t one = 0;
  expect("workspace seg = L", infini_attn_workspace_size(&d, 32768, &one), INFINI_ATTN_OK);
  size_t big = 0;
  expect("workspace seg = INT32_MAX", infini_attn_workspace_size(&d, INT32_MAX, &big), INFINI_ATTN_OK);
  if (big != one) {
    printf("FAIL workspace of seg_len >= L differs from seg_len = L: %zu vs %zu\n", big, one);
    ++failures;
  }
  {
    infini_attn_desc e = d;
    e.batch = 2047;  // B * Hq = 65504
    e.seq_len = 1 << 30;
    size_t huge = 0;
    expect("workspace 2^30 rows x 2047 batch", infini_attn_workspace_size(&e, 1 << 15, &huge),
           INFINI_ATTN_OK);
    if (huge < (size_t)1 << 40) {
      printf("FAIL workspace of 2^30 rows x 2047 batch is only %zu bytes\n", huge);
      ++failures;
    }
    e.dtype = INFINI_ATTN_F32;
    e.d_k = e.d_v = 32;
    expect("workspace fp32", infini_attn_workspace_size(&e, 1 << 15, &huge), INFINI_ATTN_OK);
  }

  // Handles: no device here, so create reports a HIP error and hands back NULL.
  infini_attn_t *h = (infini_attn_t *)0x1;
  expect("create null out", infini_attn_create(NULL, &d), INFINI_ATTN_ERR_INVALID);
  expect("create null desc", infini_attn_create(&h, NULL), INFINI_ATTN_ERR_INVALID);
  if (h != NULL) {
    printf("FAIL create left a non-null handle after an error\n");
    ++failures;
  }
  {
    infini_attn_desc e = d;
    e.d_k = e.d_v = 48;
    expect("create unsupported d", infini_attn_create(&h, &e), INFINI_ATTN_ERR_UNSUPPORTED);
  }
  const int st = infini_attn_create(&h, &d);
  if (st != INFINI_ATTN_ERR_HIP && st != INFINI_ATTN_OK) {
    printf("FAIL create without a device: status %d\n", st);
    ++failures;
  }
  if (st == INFINI_ATTN_OK) infini_attn_destroy(h);

  // Every entry point rejects a null handle before touching anything.
  float f = 0.f;
  void *p = &f;
  expect("forward null handle",
         infini_attn_forward(NULL, p, p, p, &f, &f, &f, 64, 0, p), INFINI_ATTN_ERR_INVALID);
  expect("update null handle", infini_attn_update(NULL, p, p, &f, &f, 0), INFINI_ATTN_ERR_INVALID);
  expect("decode null handle", infini_attn_decode(NULL, p, 1, p, p, 0, &f, &f, &f, p),
         INFINI_ATTN_ERR_INVALID);
  expect("decode_noalloc null handle",
         infini_attn_decode_noalloc(NULL, p, 1, p, p, 0, &f, &f, &f, p), INFINI_ATTN_ERR_INVALID);
  expect("block null handle",
         infini_attn_block_forward(NULL, 64, p, p, p, p, p, &f, &f, &f, 64, 0, p),
         INFINI_ATTN_ERR_INVALID);
  expect("backward null handle",
         infini_attn_backward(NULL, p, p, p, &f, &f, &f, 64, 0, p, NULL, NULL, &f, &f, &f, &f, &f,
                              &f),
         INFINI_ATTN_ERR_INVALID);
  expect("set_timing null handle", infini_attn_set_timing(NULL, 1), INFINI_ATTN_ERR_INVALID);
  expect("get_timing null handle", infini_attn_get_timing(NULL, NULL, NULL, NULL),
         INFINI_ATTN_ERR_INVALID);
  expect("destroy null handle", infini_attn_destroy(NULL), INFINI_ATTN_OK);
  for (int s = -8; s <= 1; ++s) {
    const char *txt = infini_attn_strerror(s);
    if (!txt || !txt[0]) {
      printf("FAIL strerror(%d) empty\n", s);
      ++failures;
    }
  }
  printf("%s: %d failure(s)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
