/* Pure-C check of libgqa's boundary: every validation error is returned
 * before anything touches a device, so this runs on a machine with no GPU.
 * Pointers here are fake host addresses that are never dereferenced. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gqa.h"

static int failures = 0;

static void expect(const char* what, gqa_status_t got, gqa_status_t want) {
  if (got != want) {
    printf("FAIL %s: got %d want %d (%s)\n", what, got, want, gqa_last_error());
    ++failures;
  } else {
    printf("ok   %s -> %d (%s)\n", what, got, gqa_last_error());
  }
}

int main(void) {
  void* P = (void*)(uintptr_t)0x10000;  /* aligned, never dereferenced */
  void* M = (void*)(uintptr_t)0x10002;  /* misaligned */
  const int64_t s[3] = {4096, 1024, 64};
  const int64_t bad[3] = {4096, 1024, 60};
  size_t ws = 0;

  if (gqa_abi_version() != GQA_ABI_VERSION) { printf("FAIL abi version\n"); ++failures; }
  expect("workspace size", gqa_attention_workspace_size(16, 32, 1, 8192, 128, 1024, &ws), GQA_OK);
  if (ws != (size_t)16 * 32 * 8 * 130 * 4) { printf("FAIL workspace bytes %zu\n", ws); ++failures; }
  expect("workspace size tile 0", gqa_attention_workspace_size(1, 1, 1, 1, 64, 0, &ws), GQA_OK);
  if (ws != 0) { printf("FAIL tile-0 workspace %zu\n", ws); ++failures; }
  expect("workspace size NULL out", gqa_attention_workspace_size(1, 1, 1, 1, 64, 64, NULL),
         GQA_ERR_INVALID_ARGUMENT);

#define PREFILL(q, qs, d, hq, hkv, scale, causal, tile, w, wb) \
  gqa_attention_prefill(q, qs, P, s, P, s, P, s, 1, hq, hkv, 16, 128, d, NULL, scale, NULL, \
                        causal, tile, w, wb, NULL)
  expect("NULL q", PREFILL(NULL, s, 64, 4, 1, 0.125f, 0, 0, NULL, 0), GQA_ERR_INVALID_ARGUMENT);
  expect("misaligned q", PREFILL(M, s, 64, 4, 1, 0.125f, 0, 0, NULL, 0), GQA_ERR_UNSUPPORTED);
  expect("stride not x8", PREFILL(P, bad, 64, 4, 1, 0.125f, 0, 0, NULL, 0), GQA_ERR_UNSUPPORTED);
  expect("NULL strides", PREFILL(P, NULL, 64, 4, 1, 0.125f, 0, 0, NULL, 0), GQA_ERR_INVALID_ARGUMENT);
  {
    /* Key-row strides: a 64-key tile spans 63 rows of 32-bit byte offsets
     * from its first row, so the bound is 2^25 elements.  Just below it the
     * stride check passes and the call stops at the (missing) workspace;
     * at the bound and above it is refused. */
    const int64_t big = ((int64_t)1 << 25) - 8;
    const int64_t at[3] = {(int64_t)1 << 40, (int64_t)1 << 34, (int64_t)1 << 25};
    const int64_t below[3] = {(int64_t)1 << 40, (int64_t)1 << 34, big};
    const int64_t huge[3] = {(int64_t)1 << 40, (int64_t)1 << 34, (int64_t)1 << 26};
    expect("k row stride 2^26",
           gqa_attention_prefill(P, s, P, huge, P, s, P, s, 1, 4, 1, 16, 128, 64, NULL, 0.125f,
                                 NULL, 0, 0, NULL, 0, NULL), GQA_ERR_UNSUPPORTED);
    expect("k row stride 2^25",
           gqa_attention_prefill(P, s, P, at, P, s, P, s, 1, 4, 1, 16, 128, 64, NULL, 0.125f,
                                 NULL, 0, 64, NULL, 0, NULL), GQA_ERR_UNSUPPORTED);
    expect("k row stride 2^25 - 8 passes (stops at the workspace)",
           gqa_attention_prefill(P, s, P, below, P, s, P, s, 1, 4, 1, 16, 128, 64, NULL, 0.125f,
                                 NULL, 0, 64, NULL, 0, NULL), GQA_ERR_WORKSPACE);
    expect("v row stride 2^25",
           gqa_attention_prefill(P, s, P, s, P, at, P, s, 1, 4, 1, 16, 128, 64, NULL, 0.125f,
                                 NULL, 0, 64, NULL, 0, NULL), GQA_ERR_UNSUPPORTED);
    expect("v row stride 2^25 - 8 passes (stops at the workspace)",
           gqa_attention_prefill(P, s, P, s, P, below, P, s, 1, 4, 1, 16, 128, 64, NULL, 0.125f,
                                 NULL, 0, 64, NULL, 0, NULL), GQA_ERR_WORKSPACE);
    expect("paged row stride 2^26",
           gqa_attention_paged(P, 4096, 128, P, P, P, (int64_t)1 << 33, (int64_t)1 << 26, 128, P,
                               64, P, P, 4096, 128, 8, 32, 1, 128, 64, 100, 64, 0.088f, NULL, 0, 0,
                               NULL, 0, NULL), GQA_ERR_UNSUPPORTED);
    expect("paged row stride 2^25",
           gqa_attention_paged(P, 4096, 128, P, P, P, (int64_t)1 << 33, (int64_t)1 << 25, 128, P,
                               64, P, P, 4096, 128, 8, 32, 1, 128, 64, 100, 64, 0.088f, NULL, 0,
                               512, NULL, 0, NULL), GQA_ERR_UNSUPPORTED);
    expect("paged row stride 2^25 - 8 passes (stops at the workspace)",
           gqa_attention_paged(P, 4096, 128, P, P, P, (int64_t)1 << 33, big, 128, P, 64, P, P,
                               4096, 128, 8, 32, 1, 128, 64, 100, 64, 0.088f, NULL, 0, 512, NULL,
                               0, NULL), GQA_ERR_WORKSPACE);
  }
  expect("d = 96", PREFILL(P, s, 96, 4, 1, 0.125f, 0, 0, NULL, 0), GQA_ERR_UNSUPPORTED);
  expect("d = 1024", PREFILL(P, s, 1024, 4, 1, 0.125f, 0, 0, NULL, 0), GQA_ERR_UNSUPPORTED);
  expect("Hq % Hkv", PREFILL(P, s, 64, 6, 4, 0.125f, 0, 0, NULL, 0), GQA_ERR_INVALID_ARGUMENT);
  expect("Hkv = 0", PREFILL(P, s, 64, 4, 0, 0.125f, 0, 0, NULL, 0), GQA_ERR_INVALID_ARGUMENT);
  expect("scale 0", PREFILL(P, s, 64, 4, 1, 0.0f, 0, 0, NULL, 0), GQA_ERR_INVALID_ARGUMENT);
  expect("scale nan", PREFILL(P, s, 64, 4, 1, NAN, 0, 0, NULL, 0), GQA_ERR_INVALID_ARGUMENT);
  expect("causal 2", PREFILL(P, s, 64, 4, 1, 0.125f, 2, 0, NULL, 0), GQA_ERR_INVALID_ARGUMENT);
  expect("tile 100", PREFILL(P, s, 64, 4, 1, 0.125f, 0, 100, NULL, 0), GQA_ERR_INVALID_ARGUMENT);
  expect("split, no workspace", PREFILL(P, s, 64, 4, 1, 0.125f, 0, 64, NULL, 0), GQA_ERR_WORKSPACE);
  expect("split, small workspace", PREFILL(P, s, 64, 4, 1, 0.125f, 0, 64, P, 1024), GQA_ERR_WORKSPACE);
  expect("split, misaligned workspace", PREFILL(P, s, 64, 4, 1, 0.125f, 0, 64, M, 1 << 20),
         GQA_ERR_WORKSPACE);
  expect("negative B",
         gqa_attention_prefill(P, s, P, s, P, s, P, s, -1, 4, 1, 16, 128, 64, NULL, 0.125f, NULL,
                               0, 0, NULL, 0, NULL), GQA_ERR_INVALID_ARGUMENT);
  expect("decode tile 0",
         gqa_attention_decode_splitkv(P, s, P, s, P, s, P, s, 16, 32, 8, 8192, 128, NULL,
                                      0.088f, NULL, 0, P, 1 << 30, NULL), GQA_ERR_INVALID_ARGUMENT);
  expect("decode no workspace",
         gqa_attention_decode_splitkv(P, s, P, s, P, s, P, s, 16, 32, 8, 8192, 128, NULL,
                                      0.088f, NULL, 1024, NULL, 0, NULL), GQA_ERR_WORKSPACE);
  expect("partial no workspace",
         gqa_attention_splitkv_partial(P, s, P, s, P, s, 2, 8, 2, 3, 300, 64, NULL, 0.125f, 0, 64,
                                       NULL, 0, NULL), GQA_ERR_WORKSPACE);
  expect("merge small workspace",
         gqa_attention_splitkv_merge(P, 256, P, s, 2, 8, 3, 64, 5, NULL, NULL), GQA_ERR_WORKSPACE);
  expect("merge n_split 0",
         gqa_attention_splitkv_merge(P, 1 << 20, P, s, 2, 8, 3, 64, 0, NULL, NULL),
         GQA_ERR_INVALID_ARGUMENT);
  /* 64 heads x 2^26 rows: 2^30 merge workgroups of 256 work-items, more
   * than one dispatch can count */
  expect("merge grid beyond 2^32 work-items",
         gqa_attention_splitkv_merge(P, SIZE_MAX, P, s, 1, 64, 1 << 26, 64, 1, NULL, NULL),
         GQA_ERR_UNSUPPORTED);
#define PAGED(cu, pt, kvl, page, d, causal) \
  gqa_attention_paged(P, 4096, 128, cu, P, P, 8192, 128, 128, pt, 64, kvl, P, 4096, 128, 8, 32, \
                      1, d, page, 100, 64, 0.088f, NULL, causal, 0, NULL, 0, NULL)
  expect("paged page 32", PAGED(P, P, P, 32, 128, 0), GQA_ERR_UNSUPPORTED);
  expect("paged NULL cu", PAGED(NULL, P, P, 64, 128, 0), GQA_ERR_INVALID_ARGUMENT);
  expect("paged NULL table", PAGED(P, NULL, P, 64, 128, 0), GQA_ERR_INVALID_ARGUMENT);
  expect("paged NULL kv_len", PAGED(P, P, NULL, 64, 128, 0), GQA_ERR_INVALID_ARGUMENT);
  expect("paged d 1024", PAGED(P, P, P, 64, 1024, 0), GQA_ERR_UNSUPPORTED);
  expect("paged d 48", PAGED(P, P, P, 64, 48, 0), GQA_ERR_UNSUPPORTED);
  expect("paged causal 3", PAGED(P, P, P, 64, 128, 3), GQA_ERR_INVALID_ARGUMENT);
  expect("paged split, no workspace",
         gqa_attention_paged(P, 4096, 128, P, P, P, 8192, 128, 128, P, 64, P, P, 4096, 128, 8, 32,
                             1, 128, 64, 100, 64, 0.088f, NULL, 0, 512, NULL, 0, NULL),
         GQA_ERR_WORKSPACE);
  expect("paged tile 100",
         gqa_attention_paged(P, 4096, 128, P, P, P, 8192, 128, 128, P, 64, P, P, 4096, 128, 8, 32,
                             1, 128, 64, 100, 64, 0.088f, NULL, 0, 100, P, 1 << 30, NULL),
         GQA_ERR_INVALID_ARGUMENT);
  /* append: B 8, Hq 32, Hkv 8 (G 4), d 128, total_q 8, max_q_len mq */
#define APPEND(kn, vn, nst, mq) \
  gqa_attention_paged_append(P, 4096, 128, P, P, P, 8192, 128, 128, P, 64, P, kn, vn, nst, 128, \
                             P, 4096, 128, 8, 32, 8, 128, 64, 8, mq, 0.088f, NULL, 0, 0, NULL, 0, \
                             NULL)
  expect("append NULL k_new", APPEND(NULL, P, 1024, 1), GQA_ERR_INVALID_ARGUMENT);
  expect("append NULL v_new", APPEND(P, NULL, 1024, 1), GQA_ERR_INVALID_ARGUMENT);
  expect("append misaligned k_new", APPEND(M, P, 1024, 1), GQA_ERR_UNSUPPORTED);
  expect("append new stride 1020", APPEND(P, P, 1020, 1), GQA_ERR_UNSUPPORTED);
  expect("append 36 rows per kv head", APPEND(P, P, 1024, 9), GQA_ERR_UNSUPPORTED);
  expect("append d 512",
         gqa_attention_paged_append(P, 4096, 128, P, P, P, 8192, 128, 128, P, 64, P, P, P, 1024,
                                    128, P, 4096, 128, 8, 32, 8, 512, 64, 8, 1, 0.044f, NULL, 0, 0,
                                    NULL, 0, NULL),
         GQA_ERR_UNSUPPORTED);
  expect("append new stride 2^26", APPEND(P, P, (int64_t)1 << 26, 1), GQA_ERR_UNSUPPORTED);
  expect("append new stride 2^25", APPEND(P, P, (int64_t)1 << 25, 1), GQA_ERR_UNSUPPORTED);
  expect("append new stride 2^25 - 8 passes (stops at the workspace)",
         gqa_attention_paged_append(P, 4096, 128, P, P, P, 8192, 128, 128, P, 64, P, P, P,
                                    ((int64_t)1 << 25) - 8, 128, P, 4096, 128, 8, 32, 8, 128, 64,
                                    8, 1, 0.088f, NULL, 0, 512, NULL, 0, NULL),
         GQA_ERR_WORKSPACE);
  expect("append empty batch",
         gqa_attention_paged_append(NULL, 0, 0, NULL, NULL, NULL, 0, 0, 0, NULL, 0, NULL, NULL,
                                    NULL, 0, 0, NULL, 0, 0, 0, 32, 8, 128, 64, 0, 0, 0.088f, NULL,
                                    0, 0, NULL, 0, NULL),
         GQA_OK);
  {
    int32_t* T = (int32_t*)P;
    expect("fused NULL tickets",
           gqa_attention_decode_splitkv_fused(P, s, P, s, P, s, P, s, 16, 32, 8, 8192, 128, NULL,
                                              0.088f, NULL, 1024, P, 1 << 30, NULL, 512, NULL),
           GQA_ERR_INVALID_ARGUMENT);
    expect("fused 511 tickets",
           gqa_attention_decode_splitkv_fused(P, s, P, s, P, s, P, s, 16, 32, 8, 8192, 128, NULL,
                                              0.088f, NULL, 1024, P, 1 << 30, T, 511, NULL),
           GQA_ERR_WORKSPACE);
    expect("fused group 64",
           gqa_attention_decode_splitkv_fused(P, s, P, s, P, s, P, s, 16, 64, 1, 8192, 128, NULL,
                                              0.088f, NULL, 1024, P, 1 << 30, T, 1024, NULL),
           GQA_ERR_UNSUPPORTED);
    expect("fused d 512",
           gqa_attention_decode_splitkv_fused(P, s, P, s, P, s, P, s, 16, 32, 8, 8192, 512, NULL,
                                              0.044f, NULL, 1024, P, 1 << 30, T, 512, NULL),
           GQA_ERR_UNSUPPORTED);
    expect("fused tile 0",
           gqa_attention_decode_splitkv_fused(P, s, P, s, P, s, P, s, 16, 32, 8, 8192, 128, NULL,
                                              0.088f, NULL, 0, P, 1 << 30, T, 512, NULL),
           GQA_ERR_INVALID_ARGUMENT);
    expect("fused small workspace",
           gqa_attention_decode_splitkv_fused(P, s, P, s, P, s, P, s, 16, 32, 8, 8192, 128, NULL,
                                              0.088f, NULL, 1024, P, 1024, T, 512, NULL),
           GQA_ERR_WORKSPACE);
  }
  /* the allocation-free decode refuses partial states beyond its scratch
   * (and every other bad argument) before touching a device */
  expect("noalloc tile 0",
         gqa_attention_decode_splitkv_noalloc(P, s, P, s, P, s, P, s, 16, 32, 8, 8192, 128, NULL,
                                              0.088f, NULL, 0, NULL), GQA_ERR_INVALID_ARGUMENT);
  expect("noalloc d 96",
         gqa_attention_decode_splitkv_noalloc(P, s, P, s, P, s, P, s, 16, 32, 8, 8192, 96, NULL,
                                              0.088f, NULL, 1024, NULL), GQA_ERR_UNSUPPORTED);
  expect("noalloc NULL o",
         gqa_attention_decode_splitkv_noalloc(P, s, P, s, P, s, NULL, s, 16, 32, 8, 8192, 128,
                                              NULL, 0.088f, NULL, 1024, NULL),
         GQA_ERR_INVALID_ARGUMENT);
  /* 64 x 32 rows x 8 splits x 130 floats = 8,519,680 bytes > 8 MiB */
  expect("noalloc beyond the scratch",
         gqa_attention_decode_splitkv_noalloc(P, s, P, s, P, s, P, s, 64, 32, 8, 8192, 128, NULL,
                                              0.088f, NULL, 1024, NULL), GQA_ERR_WORKSPACE);
  expect("noalloc empty batch",
         gqa_attention_decode_splitkv_noalloc(NULL, s, NULL, s, NULL, s, NULL, s, 0, 32, 8, 8192,
                                              128, NULL, 0.088f, NULL, 1024, NULL), GQA_OK);
  printf("%s\n", failures ? "FAILED" : "ALL OK");
  return failures ? 1 : 0;
}
