// bcq_api.hip -- the C ABI: argument validation on the host, then dispatch to
// the kernels.  Every check runs before any HIP call, so a rejected call
// enqueues nothing and touches no device state.
#include <stdint.h>

#include "bcq_internal.h"

namespace {

using bcq::kGroup;

constexpr int32_t kMaxM = 1 << 24;
constexpr int32_t kMaxK = 1 << 20;

size_t dtype_size(bcq_dtype d) { return d == BCQ_F16 ? 2 : 4; }
bool dtype_valid(bcq_dtype d) { return d == BCQ_F16 || d == BCQ_F32; }
bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bcq_status hip_status(hipError_t e) { return e == hipSuccess ? BCQ_OK : BCQ_ERR_HIP; }

bcq_status check_shape(int32_t P, int32_t M, int32_t K) {
  if (P < 1 || P > BCQ_MAX_PLANES) return BCQ_ERR_INVALID_ARG;
  if (M < 1 || M > kMaxM) return BCQ_ERR_INVALID_ARG;
  if (K < kGroup || K > kMaxK || K % kGroup != 0) return BCQ_ERR_INVALID_ARG;
  return BCQ_OK;
}

// Store-level checks shared by every product.
bcq_status check_store(const bcq_store *st) {
  if (st == nullptr || st->bits == nullptr) return BCQ_ERR_INVALID_ARG;
  if (st->group_size != kGroup) return BCQ_ERR_UNSUPPORTED;
  bcq_status s = check_shape(st->planes, st->M, st->K);
  if (s != BCQ_OK) return s;
  if (!dtype_valid(st->scale_dtype)) return BCQ_ERR_INVALID_ARG;
  if (!aligned(st->bits, 16)) return BCQ_ERR_ALIGNMENT;
  return BCQ_OK;
}

// The tables of precision p exist and are element aligned.
bcq_status check_precision(const bcq_store *st, int32_t p) {
  if (p < 1 || p > st->planes) return BCQ_ERR_INVALID_ARG;
  if (st->alpha[p] == nullptr || st->zero[p] == nullptr) return BCQ_ERR_INVALID_ARG;
  const size_t es = dtype_size(st->scale_dtype);
  if (!aligned(st->alpha[p], es) || !aligned(st->zero[p], es)) return BCQ_ERR_ALIGNMENT;
  return BCQ_OK;
}

bcq_status check_dtypes(const bcq_store *st, bcq_dtype x_dt, bcq_dtype y_dt) {
  if (!dtype_valid(x_dt) || !dtype_valid(y_dt)) return BCQ_ERR_INVALID_ARG;
  if (x_dt != st->scale_dtype || y_dt != st->scale_dtype) return BCQ_ERR_UNSUPPORTED;
  return BCQ_OK;
}

// Batched activations / outputs.
bcq_status check_batch(const bcq_store *st, const void *X, int32_t b, int32_t ldx, void *Y,
                       int32_t ldy) {
  if (X == nullptr || Y == nullptr) return BCQ_ERR_INVALID_ARG;
  if (b < 1 || b > BCQ_MAX_BATCH) return BCQ_ERR_INVALID_ARG;
  if (ldx < st->K || ldy < st->M) return BCQ_ERR_INVALID_ARG;
  const size_t es = dtype_size(st->scale_dtype);
  if (!aligned(X, 16) || ((size_t)ldx * es) % 16 != 0) return BCQ_ERR_ALIGNMENT;
  if (!aligned(Y, es)) return BCQ_ERR_ALIGNMENT;
  return BCQ_OK;
}

#define BCQ_TRY(expr)                 \
  do {                                \
    bcq_status s_ = (expr);           \
    if (s_ != BCQ_OK) return s_;      \
  } while (0)

// Requests [r0, r0+n) with their own precisions through the table kernel,
// up to kMaxReq per launch.
bcq_status run_table_batches(const bcq_store *st, const int32_t *p_of, const char *X, int32_t b,
                             int32_t ldx, char *Y, int32_t ldy, hipStream_t stream) {
  const size_t es = dtype_size(st->scale_dtype);
  for (int32_t r0 = 0; r0 < b; r0 += bcq::kMaxReq) {
    const int n = (b - r0) < bcq::kMaxReq ? (b - r0) : bcq::kMaxReq;
    bcq::ReqTables t{};
    int pmax = 0;
    for (int q = 0; q < n; ++q) {
      const int p = p_of[r0 + q];
      t.p[q] = p;
      t.alpha[q] = st->alpha[p];
      t.zero[q] = st->zero[p];
      pmax = p > pmax ? p : pmax;
    }
    for (int q = n; q < bcq::kMaxReq; ++q) {
      t.p[q] = 0;
      t.alpha[q] = st->alpha[p_of[r0]];
      t.zero[q] = st->zero[p_of[r0]];
    }
    const char *xr = X + (size_t)r0 * ldx * es;
    char *yr = Y + (size_t)r0 * ldy * es;
    hipError_t e;
    if (n == 1)
      e = bcq::launch_gemv_lut(st->bits, st->M, st->K, t.p[0], t.alpha[0], t.zero[0], xr, yr,
                               st->scale_dtype, stream);
    else
      e = bcq::launch_skinny_lut(st->bits, st->M, st->K, pmax, t, n, xr, ldx, yr, ldy,
                                 st->scale_dtype, stream);
    if (e != hipSuccess) return BCQ_ERR_HIP;
  }
  return BCQ_OK;
}

}  // namespace

extern "C" {

size_t bcq_packed_bytes(int32_t P, int32_t M, int32_t K) {
  if (check_shape(P, M, K) != BCQ_OK) return 0;
  return (size_t)P * bcq::row_tiles(M) * bcq::kTileRows * ((size_t)K / 8);
}

bcq_status bcq_pack_planes(const uint32_t *signs, int32_t P, int32_t M, int32_t K,
                           uint32_t *packed, hipStream_t stream) {
  if (signs == nullptr || packed == nullptr) return BCQ_ERR_INVALID_ARG;
  BCQ_TRY(check_shape(P, M, K));
  if (!aligned(signs, 4) || !aligned(packed, 16)) return BCQ_ERR_ALIGNMENT;
  return hip_status(bcq::launch_pack(signs, P, M, K, packed, stream));
}

bcq_status bcq_unpack_planes(const uint32_t *packed, int32_t P, int32_t M, int32_t K,
                             uint32_t *signs, hipStream_t stream) {
  if (signs == nullptr || packed == nullptr) return BCQ_ERR_INVALID_ARG;
  BCQ_TRY(check_shape(P, M, K));
  if (!aligned(signs, 4) || !aligned(packed, 16)) return BCQ_ERR_ALIGNMENT;
  return hip_status(bcq::launch_unpack(packed, P, M, K, signs, stream));
}

bcq_status bcq_gemv(const bcq_store *store, int32_t p, const void *x, bcq_dtype x_dtype, void *y,
                    bcq_dtype y_dtype, hipStream_t stream) {
  BCQ_TRY(check_store(store));
  BCQ_TRY(check_precision(store, p));
  BCQ_TRY(check_dtypes(store, x_dtype, y_dtype));
  if (x == nullptr || y == nullptr) return BCQ_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, dtype_size(y_dtype))) return BCQ_ERR_ALIGNMENT;
  return hip_status(bcq::launch_gemv_lut(store->bits, store->M, store->K, p, store->alpha[p],
                                         store->zero[p], x, y, store->scale_dtype, stream));
}

size_t bcq_workspace_bytes(const bcq_store *store, int32_t b) {
  if (check_store(store) != BCQ_OK || b < 1 || b > BCQ_MAX_BATCH) return 0;
  if (b < 16 || store->scale_dtype != BCQ_F16) return 0;
  return bcq::mfma_workspace_bytes(store->M, store->K, b);
}

bcq_status bcq_gemm_skinny(const bcq_store *store, int32_t p, const void *X, int32_t b,
                           int32_t ldx, bcq_dtype x_dtype, void *Y, int32_t ldy,
                           bcq_dtype y_dtype, void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  BCQ_TRY(check_store(store));
  BCQ_TRY(check_precision(store, p));
  BCQ_TRY(check_dtypes(store, x_dtype, y_dtype));
  BCQ_TRY(check_batch(store, X, b, ldx, Y, ldy));
  const size_t need = bcq_workspace_bytes(store, b);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return BCQ_ERR_INVALID_ARG;
  if (need > 0 && !aligned(workspace, 4)) return BCQ_ERR_ALIGNMENT;

  const size_t es = dtype_size(store->scale_dtype);
  const char *Xc = static_cast<const char *>(X);
  char *Yc = static_cast<char *>(Y);
  if (b >= 16 && store->scale_dtype == BCQ_F16) {
    for (int32_t r0 = 0; r0 < b; r0 += 64) {
      const int n = (b - r0) < 64 ? (b - r0) : 64;
      hipError_t e = bcq::launch_gemm_mfma(store->bits, store->M, store->K, p, store->alpha[p],
                                           store->zero[p], Xc + (size_t)r0 * ldx * es, ldx, n,
                                           Yc + (size_t)r0 * ldy * es, ldy, workspace, stream);
      if (e != hipSuccess) return BCQ_ERR_HIP;
    }
    return BCQ_OK;
  }
  int32_t ps[BCQ_MAX_BATCH];
  for (int32_t r = 0; r < b; ++r) ps[r] = p;
  return run_table_batches(store, ps, Xc, b, ldx, Yc, ldy, stream);
}

bcq_status bcq_gemv_mixed_p(const bcq_store *store, const int32_t *p_host, const void *X,
                            int32_t b, int32_t ldx, bcq_dtype x_dtype, void *Y, int32_t ldy,
                            bcq_dtype y_dtype, hipStream_t stream) {
  BCQ_TRY(check_store(store));
  BCQ_TRY(check_dtypes(store, x_dtype, y_dtype));
  BCQ_TRY(check_batch(store, X, b, ldx, Y, ldy));
  if (p_host == nullptr) return BCQ_ERR_INVALID_ARG;
  for (int32_t r = 0; r < b; ++r) BCQ_TRY(check_precision(store, p_host[r]));
  return run_table_batches(store, p_host, static_cast<const char *>(X), b, ldx,
                           static_cast<char *>(Y), ldy, stream);
}

const char *bcq_status_string(bcq_status status) {
  switch (status) {
    case BCQ_OK:
      return "BCQ_OK";
    case BCQ_ERR_INVALID_ARG:
      return "BCQ_ERR_INVALID_ARG: null pointer, bad shape, precision out of range or bad leading dimension";
    case BCQ_ERR_UNSUPPORTED:
      return "BCQ_ERR_UNSUPPORTED: dtype pairing or group size not implemented";
    case BCQ_ERR_ALIGNMENT:
      return "BCQ_ERR_ALIGNMENT: a pointer or leading dimension breaks the alignment rules";
    case BCQ_ERR_HIP:
      return "BCQ_ERR_HIP: the HIP runtime reported a launch error";
  }
  return "unknown bcq_status";
}

}  // extern "C"
