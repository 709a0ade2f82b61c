/* Drives the host layer of libhs2 (argument validation, workspace sizing and
 * launch set-up) under AddressSanitizer and UndefinedBehaviorSanitizer on a
 * machine without a GPU.  Pointers are fake, 256-byte aligned device
 * addresses; they are never dereferenced on the host.  Calls whose arguments
 * pass validation reach the HIP launch, which fails without a device and must
 * come back as HS2_ERR_HIP.  Every integer argument is swept over edge values,
 * where a signed overflow in a check would be undefined behaviour.  Exit code
 * 0 and no sanitizer report means the host layer is clean. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "hs2.h"

#define FAKE ((void*)(uintptr_t)0x7F0000000000ull)
#define MIS ((void*)(uintptr_t)0x7F0000000008ull)

static int n_checked = 0, n_failed = 0, n_launched = 0;

static void expect(const char* what, int got, int want) {
  ++n_checked;
  if (got != want) {
    ++n_failed;
    fprintf(stderr, "FAIL %s: got %d (%s) want %d; last error: %s\n", what, got, hs2_status_str(got), want,
            hs2_last_error());
  }
}

static void expect_status(const char* what, int got) {
  ++n_checked;
  if (got > 0 || got < HS2_ERR_HIP || got == HS2_OK) {
    ++n_failed;
    fprintf(stderr, "FAIL %s: got %d, want an error (no device here)\n", what, got);
  }
  n_launched += got == HS2_ERR_HIP;
  (void)strlen(hs2_last_error());
}

static const int64_t I64S[] = {-1, 0, 1, 127, 128, 1152, 4096, 65535, 65536, 1 << 20, 0x7FFFFFFFll, 0x80000000ll,
                               (int64_t)1 << 40, INT64_MAX - 1, INT64_MAX, INT64_MIN};
static const int INTS[] = {-1, 0, 1, 2, 3, 4, 16, 17, 64, 65, 256, 4096, 4097, 65536, 0x7FFFFFFF, (int)0x80000000};
#define N64 (int)(sizeof(I64S) / sizeof(I64S[0]))
#define NI (int)(sizeof(INTS) / sizeof(INTS[0]))

int main(void) {
  char buf[64];
  /* ---- status strings and version */
  for (int c = -10; c <= 2; ++c) (void)strlen(hs2_status_str(c));
  expect("version", hs2_version() >= 10000, 1);

  /* ---- workspace queries over every edge combination */
  size_t acc = 0;
  for (int a = 0; a < NI; ++a)
    for (int b = 0; b < NI; ++b)
      for (int c = 0; c < NI; ++c) {
        acc += hs2_sparse_workspace_bytes(INTS[a], INTS[b], INTS[c] % 17, INTS[c]);
        for (int t = 0; t < N64; ++t) {
          acc += hs2_full_attn_workspace_bytes(INTS[a], INTS[b], INTS[c] % 17, I64S[t], c % 4);
          acc += hs2_select_workspace_bytes(INTS[a], INTS[b], I64S[t], I64S[(t + c) % N64]);
          acc += hs2_select_blocks_workspace_bytes(INTS[a], INTS[b], I64S[t], I64S[(t + c) % N64], INTS[c],
                                                   INTS[(a + c) % NI]);
        }
      }
  printf("workspace queries done (%zu)\n", acc & 0xff);

  /* ---- fixed rejections (one reason each) */
  expect("full: null q", hs2_full_attn_scored(NULL, HS2_BF16, 1, 1, 16, 256, FAKE, FAKE, HS2_BF16, NULL, NULL, 100, 99,
                                              0.0625f, FAKE, FAKE, FAKE, 100, FAKE, 1 << 30, NULL), HS2_ERR_NULL);
  expect("full: H=3", hs2_full_attn_scored(FAKE, HS2_BF16, 1, 1, 3, 256, FAKE, FAKE, HS2_BF16, NULL, NULL, 100, 99,
                                           0.0625f, FAKE, FAKE, FAKE, 100, FAKE, 1 << 30, NULL), HS2_ERR_UNSUPPORTED);
  expect("full: misaligned q", hs2_full_attn_scored(MIS, HS2_BF16, 1, 1, 16, 256, FAKE, FAKE, HS2_BF16, NULL, NULL, 100,
                                                    99, 0.0625f, FAKE, FAKE, FAKE, 100, FAKE, 1 << 30, NULL),
         HS2_ERR_ALIGN);
  expect("select: window 0", hs2_select_topk_window(FAKE, 1152, 1, 1, 1152, 1151, 0, 1024, FAKE, FAKE, NULL, 0, NULL),
         HS2_ERR_SHAPE);
  expect("sparse: max_sel 0", hs2_sparse_attn_reuse(FAKE, HS2_BF16, 1, 1, 16, 256, FAKE, FAKE, HS2_BF16, NULL, NULL,
                                                    100, FAKE, FAKE, 0, 0.0625f, FAKE, NULL, FAKE, 1 << 30, NULL),
         HS2_ERR_SHAPE);
  expect("noalloc: too many pieces", hs2_sparse_attn_reuse_noalloc(FAKE, HS2_BF16, 64, 1, 16, 256, FAKE, FAKE,
                                                                    HS2_BF16, NULL, NULL, 100000, FAKE, FAKE, 4096,
                                                                    0.0625f, FAKE, FAKE, NULL),
         HS2_ERR_WORKSPACE);
  expect("swa: window 0", hs2_swa_attn(FAKE, 1, 16, 16, 256, FAKE, FAKE, 100, 50, 0, 0.0625f, FAKE, FAKE, NULL),
         HS2_ERR_SHAPE);
  expect("rope: dims not a multiple of 8", hs2_rope_partial(FAKE, FAKE, 100, 16, 256, 0, 60, 10000.0, NULL),
         HS2_ERR_UNSUPPORTED);
  expect("rope: overlapping x and y", hs2_rope_partial(FAKE, (char*)FAKE + 512, 100, 16, 256, 0, 64, 10000.0, NULL),
         HS2_ERR_SHAPE);
  expect("bridge: D=16", hs2_bridge_kv_proj(FAKE, 4096, 16, FAKE, FAKE, 4, 256, FAKE, FAKE, 4096 * 256, NULL),
         HS2_ERR_SHAPE);
  expect("bridge8: null scale", hs2_bridge_kv_proj_fp8(FAKE, 4096, 2048, FAKE, FAKE, 4, 256, FAKE, FAKE, NULL, FAKE,
                                                       4096 * 256, 4096, NULL), HS2_ERR_NULL);

  /* ---- sweeps: every call returns a status (an argument error, or HS2_ERR_HIP
   * where the arguments are valid: no device) and leaves no sanitizer report */
  for (int a = 0; a < NI; ++a)
    for (int t = 0; t < N64; ++t)
      for (int u = 0; u < N64; u += 3) {
        const int nq = INTS[a];
        const int64_t T = I64S[t], q0 = I64S[u];
        snprintf(buf, sizeof buf, "full n_q=%d T=%lld q0=%lld", nq, (long long)T, (long long)q0);
        for (int H = 1; H <= 16; H *= 4) {
          expect_status(buf, hs2_full_attn_scored(FAKE, HS2_BF16, 1, nq, H, 256, FAKE, FAKE, HS2_BF16, NULL, NULL, T,
                                                  q0, 0.0625f, FAKE, FAKE, FAKE, I64S[(t + u) % N64], FAKE,
                                                  (size_t)1 << 40, NULL));
          expect_status(buf, hs2_full_attn_scored(FAKE, HS2_BF16, nq, 1, H, 256, FAKE, FAKE, HS2_FP8E4M3, FAKE, FAKE,
                                                  T, q0, 0.0625f, FAKE, NULL, FAKE, T, FAKE, (size_t)1 << 40, NULL));
          expect_status(buf, hs2_sparse_attn_reuse(FAKE, HS2_F32, nq, INTS[(a + 3) % NI], H, 256, FAKE, FAKE,
                                                   HS2_F32, NULL, NULL, T, FAKE, FAKE, (int)(q0 & 0x7FFFFFFF),
                                                   0.0625f, FAKE, FAKE, FAKE, (size_t)1 << 40, NULL));
          expect_status("noalloc", hs2_sparse_attn_reuse_noalloc(FAKE, HS2_BF16, 1, nq, H, 256, FAKE, FAKE,
                                                                 HS2_FP8E4M3, FAKE, FAKE, T, FAKE, FAKE,
                                                                 (int)(q0 & 0x7FFFFFFF), 0.0625f, FAKE, FAKE, NULL));
          expect_status("swa", hs2_swa_attn(FAKE, INTS[(a + 5) % NI], nq, H, 256, FAKE, FAKE, T, q0,
                                            INTS[(t + u) % NI], 0.0625f, FAKE, FAKE, NULL));
          {
            /* rope_dims 0 in place has nothing to do: that valid call returns HS2_OK without a launch */
            const int rd = INTS[(a + t) % NI];
            const int rc = hs2_rope_partial(FAKE, FAKE, T, H, 256, q0, rd, 10000.0, NULL);
            if (rd == 0 && rc == HS2_OK)
              ++n_checked;
            else
              expect_status("rope", rc);
          }
        }
        for (int w = 0; w < NI; w += 5) {
          expect_status(buf, hs2_select_topk_window(FAKE, I64S[(t + u) % N64], 1, nq, T, q0, INTS[w],
                                                    INTS[(w + a) % NI], FAKE, FAKE, FAKE, (size_t)1 << 40, NULL));
          expect_status(buf, hs2_select_blocks_window(FAKE, T, INTS[w], nq, T, q0, 128, 1024, INTS[(w + u) % NI],
                                                      FAKE, FAKE, FAKE, (size_t)1 << 40, NULL));
        }
        expect_status(buf, hs2_bridge_kv_proj(FAKE, T, INTS[a], FAKE, FAKE, INTS[u % NI], 256, FAKE, FAKE, q0, NULL));
        expect_status(buf, hs2_bridge_kv_proj_fp8(FAKE, T, 2048, FAKE, FAKE, 4, 256, FAKE, FAKE, FAKE, FAKE, q0,
                                                  I64S[(t + u) % N64], NULL));
      }
  printf("checked %d calls (%d reached a launch), %d failed\n", n_checked, n_launched, n_failed);
  return n_failed || n_launched == 0 ? 1 : 0;
}
