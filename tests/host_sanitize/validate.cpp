// validate.cpp -- drives the argument validation of every entry point in
// include/bcq.h on the host, for a build of the library whose host code is
// instrumented with AddressSanitizer and UndefinedBehaviorSanitizer.  Every
// call below must be rejected before any HIP call, so no GPU is needed.
// Prints one line per failed expectation and exits with the failure count.
#include <stdint.h>
#include <stdio.h>

#include "bcq.h"

static int failures = 0;

static void expect(const char *what, long got, long want) {
  if (got != want) {
    printf("FAIL %s: got %ld, want %ld\n", what, got, want);
    ++failures;
  }
}

// aligned, never dereferenced: validation rejects each call before a launch
static void *const FAKE = (void *)(uintptr_t)0x100000;

static bcq_store store(int32_t M, int32_t K, int32_t planes, bcq_dtype dt) {
  bcq_store s = {};
  s.M = M;
  s.K = K;
  s.group_size = 128;
  s.planes = planes;
  s.bits = (const uint32_t *)FAKE;
  s.scale_dtype = dt;
  for (int p = 1; p <= BCQ_MAX_PLANES; ++p) {
    s.alpha[p] = FAKE;
    s.zero[p] = FAKE;
  }
  return s;
}

int main() {
  const char *c = (const char *)FAKE;
  bcq_store s = store(64, 256, 4, BCQ_F16);

  // sizes and status strings
  expect("packed_bytes ok", (long)bcq_packed_bytes(4, 4096, 4096), 4L * 4096 * 512);
  expect("packed_bytes P=0", (long)bcq_packed_bytes(0, 16, 128), 0);
  expect("packed_bytes K=96", (long)bcq_packed_bytes(1, 16, 96), 0);
  expect("packed_bytes M=-1", (long)bcq_packed_bytes(1, -1, 128), 0);
  for (int code = -7; code <= 2; ++code) {
    const char *str = bcq_status_string((bcq_status)code);
    expect("status string non-null", str != nullptr, 1);
  }
  expect("workspace null store", (long)bcq_workspace_bytes(nullptr, 4), 0);
  expect("workspace b=0", (long)bcq_workspace_bytes(&s, 0), 0);

  // pack / unpack
  expect("pack null", bcq_pack_planes(nullptr, 4, 64, 256, (uint32_t *)FAKE, nullptr),
         BCQ_ERR_INVALID_ARG);
  expect("pack misaligned", bcq_pack_planes((const uint32_t *)FAKE, 4, 64, 256,
                                            (uint32_t *)(c + 4), nullptr),
         BCQ_ERR_ALIGNMENT);
  expect("unpack bad K", bcq_unpack_planes((const uint32_t *)FAKE, 4, 64, 100, (uint32_t *)FAKE,
                                           nullptr),
         BCQ_ERR_INVALID_ARG);

  // batch 1
  expect("gemv null store", bcq_gemv(nullptr, 2, FAKE, BCQ_F16, FAKE, BCQ_F16, nullptr),
         BCQ_ERR_INVALID_ARG);
  expect("gemv p=5", bcq_gemv(&s, 5, FAKE, BCQ_F16, FAKE, BCQ_F16, nullptr), BCQ_ERR_INVALID_ARG);
  expect("gemv dtype", bcq_gemv(&s, 2, FAKE, BCQ_F32, FAKE, BCQ_F16, nullptr), BCQ_ERR_UNSUPPORTED);
  expect("gemv x misaligned", bcq_gemv(&s, 2, c + 8, BCQ_F16, FAKE, BCQ_F16, nullptr),
         BCQ_ERR_ALIGNMENT);
  bcq_store g64 = s;
  g64.group_size = 64;
  expect("gemv group 64", bcq_gemv(&g64, 2, FAKE, BCQ_F16, FAKE, BCQ_F16, nullptr),
         BCQ_ERR_UNSUPPORTED);
  bcq_store notab = s;
  notab.alpha[3] = nullptr;
  expect("gemv missing table", bcq_gemv(&notab, 3, FAKE, BCQ_F16, FAKE, BCQ_F16, nullptr),
         BCQ_ERR_INVALID_ARG);
  bcq_store odd = store(24, 256, 4, BCQ_F16);
  expect("gate_up rows", bcq_gemv_gate_up(&odd, 2, FAKE, BCQ_F16, FAKE, BCQ_F16, nullptr),
         BCQ_ERR_INVALID_ARG);

  // batches
  const int32_t ps[4] = {2, 3, 4, 2};
  const int32_t bad_ps[3] = {2, 0, 4};
  expect("skinny b=0", bcq_gemm_skinny(&s, 2, FAKE, 0, 256, BCQ_F16, FAKE, 64, BCQ_F16, nullptr, 0,
                                       nullptr),
         BCQ_ERR_INVALID_ARG);
  expect("skinny ldx", bcq_gemm_skinny(&s, 2, FAKE, 4, 255, BCQ_F16, FAKE, 64, BCQ_F16, nullptr, 0,
                                       nullptr),
         BCQ_ERR_INVALID_ARG);
  bcq_store big = store(1024, 8192, 4, BCQ_F16);
  expect("skinny no workspace", bcq_gemm_skinny(&big, 2, FAKE, 16, 8192, BCQ_F16, FAKE, 1024,
                                                BCQ_F16, nullptr, 0, nullptr),
         BCQ_ERR_INVALID_ARG);
  bcq_store huge = store(36864, 65536, 4, BCQ_F16);
  expect("noalloc too large", bcq_gemm_skinny_noalloc(&huge, 4, FAKE, 64, 65536, BCQ_F16, FAKE,
                                                      36864, BCQ_F16, nullptr),
         BCQ_ERR_TOO_LARGE);
  expect("mixed bad p", bcq_gemv_mixed_p(&s, bad_ps, FAKE, 3, 256, BCQ_F16, FAKE, 64, BCQ_F16,
                                         nullptr, 0, nullptr),
         BCQ_ERR_INVALID_ARG);
  expect("mixed null p", bcq_gemv_mixed_p(&s, nullptr, FAKE, 3, 256, BCQ_F16, FAKE, 64, BCQ_F16,
                                          nullptr, 0, nullptr),
         BCQ_ERR_INVALID_ARG);
  expect("gate_up batch ldy", bcq_gemm_gate_up(&s, ps, FAKE, 4, 256, BCQ_F16, FAKE, 31, BCQ_F16,
                                               nullptr),
         BCQ_ERR_INVALID_ARG);

  // export, low-rank, quantizer
  expect("dequant ldw", bcq_dequantize(&s, 2, FAKE, 255, BCQ_F16, nullptr), BCQ_ERR_INVALID_ARG);
  expect("lowrank R=0", bcq_lowrank_correct((const uint32_t *)FAKE, (const uint32_t *)FAKE, FAKE, 0,
                                            64, 256, FAKE, FAKE, BCQ_F16, (float *)FAKE, nullptr),
         BCQ_ERR_INVALID_ARG);
  expect("lowrank z misaligned",
         bcq_lowrank_correct((const uint32_t *)FAKE, (const uint32_t *)FAKE, FAKE, 16, 64, 256, FAKE,
                             FAKE, BCQ_F16, (float *)(c + 2), nullptr),
         BCQ_ERR_ALIGNMENT);
  expect("gemv_lowrank R too big",
         bcq_gemv_lowrank(&s, 2, FAKE, BCQ_F16, (const uint32_t *)FAKE, (const uint32_t *)FAKE, FAKE,
                          BCQ_LOWRANK_MAX_RANK + 1, FAKE, BCQ_F16, (float *)FAKE, nullptr),
         BCQ_ERR_INVALID_ARG);
  expect("quantize P=5", bcq_quantize(FAKE, BCQ_F16, 64, 256, 256, 5, 2, 20, (uint32_t *)FAKE, FAKE,
                                      FAKE, BCQ_F16, nullptr),
         BCQ_ERR_INVALID_ARG);
  expect("quantize p_low > P", bcq_quantize(FAKE, BCQ_F16, 64, 256, 256, 2, 3, 20,
                                            (uint32_t *)FAKE, FAKE, FAKE, BCQ_F16, nullptr),
         BCQ_ERR_INVALID_ARG);

  printf("%d failures\n", failures);
  return failures;
}
