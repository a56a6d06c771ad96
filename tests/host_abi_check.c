/*
 * Host-side check of the C ABI under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py builds the
 * library's host code instrumented and runs this program; no GPU is used).
 * It exercises the argument validation, workspace sizing and bookkeeping
 * entry points, which must reject bad input with a status and a message
 * before touching any device memory.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "hstu_attn.h"

static int failures = 0;

#define EXPECT(cond, what)                                                     \
  do {                                                                         \
    if (!(cond)) {                                                             \
      fprintf(stderr, "FAIL %s (line %d): %s\n", what, __LINE__, hstu_last_error()); \
      ++failures;                                                              \
    }                                                                          \
  } while (0)

static hstu_attn_desc good_desc(void) {
  hstu_attn_desc d;
  memset(&d, 0, sizeof(d));
  d.batch = 2; d.heads = 2; d.d_qk = 64; d.d_v = 64; d.max_len = 100;
  d.n_time_buckets = 16; d.rab_heads = 1; d.dtype = HSTU_DTYPE_BF16; d.total_tokens = 50;
  d.stride_q = d.stride_k = d.stride_v = d.stride_u = 128;
  return d;
}

/* never dereferenced: every call below fails validation first */
static void* const FAKE = (void*)4096;

static hstu_status fwd(const hstu_attn_desc* d, size_t ws_bytes) {
  return hstu_attn_fwd(d, FAKE, NULL, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL,
                       (void*)(1 << 20), ws_bytes, NULL);
}

int main(void) {
  /* workspace sizing: valid shapes give sizes that grow with T */
  size_t prev = 0;
  for (int64_t T = 0; T <= 1 << 16; T = T ? T * 4 : 1) {
    hstu_attn_desc d = good_desc();
    d.total_tokens = T;
    size_t f = 0, b = 0, bmin = 0;
    EXPECT(hstu_attn_fwd_workspace_size(&d, &f) == HSTU_OK, "fwd workspace size");
    EXPECT(hstu_attn_bwd_workspace_size(&d, &b) == HSTU_OK, "bwd workspace size");
    EXPECT(hstu_attn_bwd_workspace_size_min(&d, &bmin) == HSTU_OK, "bwd min workspace size");
    EXPECT(bmin <= b, "min <= preferred");
    EXPECT(f >= prev, "fwd workspace grows with T");
    prev = f;
    d.deterministic = 1;
    EXPECT(hstu_attn_bwd_workspace_size_min(&d, &bmin) == HSTU_OK, "deterministic min size");
  }
  /* invalid descriptors */
  {
    hstu_attn_desc d = good_desc();
    size_t n = 0;
    EXPECT(hstu_attn_fwd_workspace_size(NULL, &n) != HSTU_OK, "null desc");
    d.heads = 0;
    EXPECT(fwd(&d, 1 << 30) == HSTU_EINVAL, "heads 0");
    d = good_desc(); d.d_qk = 48;
    EXPECT(fwd(&d, 1 << 30) == HSTU_EUNSUPPORTED, "d_qk 48");
    d = good_desc(); d.stride_k = 130;
    EXPECT(fwd(&d, 1 << 30) == HSTU_EINVAL, "misaligned stride");
    d = good_desc(); d.stride_v = ((int64_t)1 << 22) + 8;
    EXPECT(fwd(&d, 1 << 30) == HSTU_EUNSUPPORTED, "stride beyond the tile range");
    d = good_desc(); d.total_tokens = (int64_t)1 << 31;
    EXPECT(fwd(&d, 1 << 30) == HSTU_EINVAL, "T >= 2^31");
    d = good_desc(); d.n_time_buckets = 2000;
    EXPECT(fwd(&d, 1 << 30) == HSTU_EINVAL, "too many time buckets");
    d = good_desc(); d.deterministic = 2;
    EXPECT(fwd(&d, 1 << 30) == HSTU_EINVAL, "deterministic flag");
    d = good_desc();
    EXPECT(fwd(&d, 16) == HSTU_EWORKSPACE, "workspace too small");
    EXPECT(strlen(hstu_last_error()) > 0, "error message set");
    /* a long message must not overflow the error buffer */
    d = good_desc(); d.stride_q = 64;
    EXPECT(fwd(&d, 1 << 30) == HSTU_EINVAL, "stride below heads*d");
    EXPECT(strlen(hstu_last_error()) < 4096, "bounded message");
  }
  /* backward, allocation-free forward, cached scoring and exports reject bad input */
  {
    hstu_attn_desc d = good_desc();
    d.heads = -3;
    EXPECT(hstu_attn_bwd(&d, FAKE, NULL, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                         FAKE, FAKE, FAKE, NULL, FAKE, FAKE, 1 << 30, NULL) != HSTU_OK, "bwd heads");
    EXPECT(hstu_attn_fwd_noalloc(&d, FAKE, NULL, FAKE, NULL, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL, NULL)
               != HSTU_OK, "noalloc heads");
    EXPECT(hstu_rab_pair_offsets(NULL, FAKE, NULL, FAKE, NULL) != HSTU_OK, "pair offsets null desc");
    d = good_desc(); d.max_len = 40000;
    EXPECT(hstu_rab_bucketize(&d, FAKE, NULL, FAKE, FAKE, FAKE, NULL, NULL) != HSTU_OK, "bucketize max_len");
    hstu_attn_bwd_info info;
    d = good_desc(); d.batch = -1;
    EXPECT(hstu_attn_bwd_report(&d, FAKE, 1 << 30, &info, NULL) != HSTU_OK, "report bad desc");
  }
  /* layer and FP8 entry points */
  EXPECT(hstu_linear(10, 48, 128, FAKE, 48, FAKE, NULL, FAKE, 1, NULL) == HSTU_EUNSUPPORTED, "linear K");
  EXPECT(hstu_linear(-1, 64, 128, FAKE, 64, FAKE, NULL, FAKE, 1, NULL) != HSTU_OK, "linear M");
  EXPECT(hstu_layernorm_gate(4, 100, FAKE, FAKE, 100, 1e-5f, FAKE, NULL) != HSTU_OK, "layernorm N");
  EXPECT(hstu_fp8_quantize_rows(10, 24, FAKE, 24, FAKE, FAKE, NULL) == HSTU_EUNSUPPORTED, "fp8 quantize K");
  EXPECT(hstu_fp8_linear(10, 24, 16, FAKE, FAKE, FAKE, FAKE, NULL, FAKE, 0, NULL) == HSTU_EUNSUPPORTED,
         "fp8 linear K");
  /* bookkeeping */
  const int32_t n = hstu_kernel_count();
  EXPECT(n > 0, "kernel count");
  for (int32_t i = 0; i < n; ++i) EXPECT(hstu_kernel_name(i) != NULL, "kernel name");
  EXPECT(hstu_kernel_name(n) != NULL && hstu_kernel_name(n)[0] == 0, "kernel name past the end");

  if (failures) {
    fprintf(stderr, "%d host ABI check(s) failed\n", failures);
    return 1;
  }
  printf("host ABI checks passed\n");
  return 0;
}
