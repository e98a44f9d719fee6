/* libaqua's C ABI called from C, for a host build under AddressSanitizer
 * (tests/test_abi_asan.py): the size queries, and every entry point with arguments it must
 * reject before any HIP call.  No pointer passed here is dereferenced by a rejecting call; the
 * error text of each rejection is read in full.  Prints "ok" and exits 0, or names the first
 * mismatch and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "aqua.h"

static int failures = 0;

#define FAKE ((void *)(uintptr_t)0x10000) /* 16-byte aligned, never dereferenced */
#define FAKE_AT(off) ((void *)((uintptr_t)0x10000 + (off)))

static void expect(const char *what, aqua_status got, aqua_status want) {
  if (got != want) {
    printf("%s: status %d, expected %d\n", what, (int)got, (int)want);
    ++failures;
    return;
  }
  if (want != AQUA_OK) {
    const char *msg = aqua_last_error();
    if (msg == NULL || strlen(msg) == 0) {
      printf("%s: no error text\n", what);
      ++failures;
    }
  }
}

static aqua_cache cache(int32_t B, int32_t Hkv, int32_t d_head, int32_t d_store, int32_t T_cap,
                        int32_t len, int32_t dtype) {
  aqua_cache c;
  c.kp = FAKE;
  c.v = FAKE;
  c.B = B;
  c.Hkv = Hkv;
  c.d_head = d_head;
  c.d_store = d_store;
  c.T_cap = T_cap;
  c.len = len;
  c.dtype = dtype;
  return c;
}

int main(void) {
  const char *ver = aqua_version();
  if (ver == NULL || strstr(ver, "gfx950") == NULL) {
    printf("version: %s\n", ver ? ver : "(null)");
    ++failures;
  }

  /* size queries (host arithmetic only) */
  aqua_cache c = cache(2, 2, 128, 128, 256, 10, AQUA_BF16);
  size_t n = 0;
  expect("decode_workspace", aqua_decode_workspace(&c, 8, &n), AQUA_OK);
  if (n == 0) {
    printf("decode_workspace: 0 bytes\n");
    ++failures;
  }
  expect("decode_workspace Hq", aqua_decode_workspace(&c, 6, &n), AQUA_ERR_SHAPE);
  expect("prefill_workspace", aqua_prefill_workspace(&c, 8, 4, &n), AQUA_OK);
  expect("gram_workspace", aqua_gram_workspace(AQUA_BF16, 1000, 128, &n), AQUA_OK);
  if (n != (size_t)8 * 128 * 128 * 4) {
    printf("gram_workspace: %zu bytes\n", n);
    ++failures;
  }
  expect("gram_workspace d", aqua_gram_workspace(AQUA_BF16, 1000, 96, &n), AQUA_ERR_SHAPE);
  expect("gram_workspace null", aqua_gram_workspace(AQUA_F32, 10, 64, NULL), AQUA_ERR_NULL);

  /* decode */
  const size_t big = (size_t)1 << 30;
  expect("decode Hq", aqua_decode(&c, 6, FAKE, FAKE, 0.1f, NULL, FAKE, FAKE, big, NULL),
         AQUA_ERR_SHAPE);
  c.len = 300;
  expect("decode capacity", aqua_decode(&c, 8, FAKE, FAKE, 0.1f, NULL, FAKE, FAKE, big, NULL),
         AQUA_ERR_CAPACITY);
  c.len = 10;
  c.dtype = 5;
  expect("decode dtype", aqua_decode(&c, 8, FAKE, FAKE, 0.1f, NULL, FAKE, FAKE, big, NULL),
         AQUA_ERR_DTYPE);
  c.dtype = AQUA_BF16;
  expect("decode null", aqua_decode(&c, 8, NULL, FAKE, 0.1f, NULL, FAKE, FAKE, big, NULL),
         AQUA_ERR_NULL);
  expect("decode align", aqua_decode(&c, 8, FAKE, FAKE, 0.1f, NULL, FAKE_AT(4), FAKE, big, NULL),
         AQUA_ERR_ALIGN);
  expect("decode workspace", aqua_decode(&c, 8, FAKE, FAKE, 0.1f, NULL, FAKE, FAKE, 16, NULL),
         AQUA_ERR_WORKSPACE);

  /* key projection and selection */
  expect("project capacity", aqua_project_keys(&c, FAKE, FAKE, FAKE, 247, NULL, NULL),
         AQUA_ERR_CAPACITY);
  expect("project null", aqua_project_keys(&c, NULL, FAKE, FAKE, 4, NULL, NULL), AQUA_ERR_NULL);
  expect("select k", aqua_select_dims(FAKE, AQUA_BF16, 4, 128, FAKE, 128, 0, FAKE, FAKE, NULL,
                                      NULL),
         AQUA_ERR_SHAPE);
  expect("select dtype", aqua_select_dims(FAKE, 7, 4, 128, FAKE, 128, 96, FAKE, FAKE, NULL, NULL),
         AQUA_ERR_DTYPE);

  /* the fused step (a rejected step appends nothing) */
  c.len = 256;
  expect("step capacity", aqua_decode_step(&c, 8, FAKE, FAKE, FAKE, FAKE, 128, 96, 0.1f, NULL,
                                           FAKE, NULL, NULL, FAKE, big, NULL),
         AQUA_ERR_CAPACITY);
  if (c.len != 256) {
    printf("step capacity: len changed to %d\n", c.len);
    ++failures;
  }
  c.len = 10;
  expect("step workspace", aqua_decode_step(&c, 8, FAKE, FAKE, FAKE, FAKE, 128, 96, 0.1f, NULL,
                                            FAKE, NULL, NULL, FAKE, 16, NULL),
         AQUA_ERR_WORKSPACE);
  expect("step noalloc k", aqua_decode_step_noalloc(&c, 8, FAKE, FAKE, FAKE, FAKE, 128, 0, 0.1f,
                                                    NULL, FAKE, NULL, NULL, NULL),
         AQUA_ERR_SHAPE);
  aqua_cache huge = cache(64, 32, 128, 128, 8192, 100, AQUA_BF16);
  expect("step noalloc scratch",
         aqua_decode_step_noalloc(&huge, 128, FAKE, FAKE, FAKE, FAKE, 128, 96, 0.1f, FAKE, FAKE,
                                  NULL, NULL, NULL),
         AQUA_ERR_WORKSPACE);

  /* prefill */
  expect("prefill pos0", aqua_prefill_chunk(&c, 8, FAKE, 4, 8, FAKE, 128, 96, 0.1f, FAKE, NULL,
                                            NULL, FAKE, big, NULL),
         AQUA_ERR_CAPACITY);
  c.dtype = AQUA_F32;
  expect("prefill dtype", aqua_prefill_chunk(&c, 8, FAKE, 4, 0, FAKE, 128, 96, 0.1f, FAKE, NULL,
                                             NULL, FAKE, big, NULL),
         AQUA_ERR_DTYPE);
  c.dtype = AQUA_BF16;

  /* H2O */
  expect("victim null", aqua_h2o_victim(NULL, FAKE, 1, 1, 4, 10, 2, FAKE, NULL), AQUA_ERR_NULL);
  expect("victim align", aqua_h2o_victim(FAKE, FAKE_AT(8), 1, 1, 4, 10, 2, FAKE, NULL),
         AQUA_ERR_ALIGN);
  aqua_cache full = cache(1, 8, 128, 96, 32768, 32768, AQUA_BF16);
  aqua_cache compact = cache(1, 8, 128, 96, 1280, 1280, AQUA_BF16);
  expect("h2o_init heavy", aqua_h2o_init(&full, FAKE, 1000, 256, &compact, FAKE, FAKE, NULL),
         AQUA_ERR_SHAPE);
  aqua_cache slots = cache(2, 2, 128, 96, 256, 256, AQUA_BF16);
  expect("h2o_step recent", aqua_h2o_step(&slots, 8, FAKE, FAKE, FAKE, FAKE, 96, 64, 0.1f, FAKE,
                                          FAKE, 300, -1, FAKE, FAKE, NULL, NULL, FAKE, big, NULL),
         AQUA_ERR_SHAPE);

  /* calibration Gram matrix and the bandwidth probe */
  expect("gram align", aqua_gram(AQUA_F32, FAKE_AT(4), 10, 64, FAKE, FAKE, (size_t)1 << 24, NULL),
         AQUA_ERR_ALIGN);
  expect("probe size", aqua_stream_read_probe(FAKE, 1000, 4, FAKE, NULL), AQUA_ERR_SHAPE);

  if (failures) {
    printf("%d failure(s)\n", failures);
    return 1;
  }
  printf("ok\n");
  return 0;
}
