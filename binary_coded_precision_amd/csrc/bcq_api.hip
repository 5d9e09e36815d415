// bcq_api.hip -- the C ABI: argument validation on the host, then dispatch to
// the kernels.  Every check runs before any HIP call, so a rejected call
// enqueues nothing and touches no device state.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "bcq_internal.h"

// ---- scratch of the allocation-free entry point (bcq_gemm_skinny_noalloc)
//
// A fixed device array that stands in for the caller's workspace: the split-K
// partial sums of the matrix-core kernels.  Every GPU the library runs on
// holds its own copy from the first launch until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress, once per device, and only
// that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[BCQ_NOALLOC_SCRATCH_BYTES];

namespace {

using bcq::kGroup;

constexpr int32_t kMaxM = 1 << 24;
constexpr int32_t kMaxK = 1 << 20;
// Smallest fp16 batch always sent to the matrix cores.  From 3 requests the
// decoded tiles on the matrix cores beat the per-request table lookups at the
// layer shapes measured on gfx950 (1024..14336 rows, K 1024..14336, p = 3 and
// 4); only tiny products lose about 1 us to the tables (256x1024 at 4
// requests: 5.0 vs 4.0 us).  At 2 the matrix cores win where K stays within
// one workgroup and is past 2048 columns (4096x4096: 7.5 vs 8.3 us;
// 1024x4096: 5.9 vs 7.1 us); with K split, or K <= 2048, the table kernel is
// faster (4096x14336: 20.0 vs 22.6 us; 2048x2048: 5.2 vs 6.1 us).
constexpr int32_t kMfMinBatch = 3;

// Route switch for A/B measurement: BCQ_FORCE_PATH=lut sends every batched
// fp16 call (2 requests and more) to the vector-ALU table kernel, =mfma sends
// it to the matrix cores; unset or any other value keeps the rule below.
// Read at every call, so a process can compare both routes.  fp32 batches
// always use the tables (the matrix-core kernels take fp16 only) and batch 1
// always uses the batch-1 kernel.
enum class Route { kRule, kTables, kMatrixCores };

Route forced_route() {
  const char *v = getenv("BCQ_FORCE_PATH");
  if (v == nullptr) return Route::kRule;
  if (strcmp(v, "lut") == 0) return Route::kTables;
  if (strcmp(v, "mfma") == 0) return Route::kMatrixCores;
  return Route::kRule;
}

bool on_matrix_cores(const bcq_store *st, int32_t b) {
  if (st->scale_dtype != BCQ_F16 || b < 2) return false;
  switch (forced_route()) {
    case Route::kTables:
      return false;
    case Route::kMatrixCores:
      return true;
    case Route::kRule:
      break;
  }
  return b >= kMfMinBatch || (b == 2 && st->K > 2048 && bcq::mfma_whole_k(st->M, st->K, b));
}

// BCQ_LOG=1 prints each product call's route to stderr.
void log_route(const char *fn, const bcq_store *st, int32_t b, const char *route) {
  const char *v = getenv("BCQ_LOG");
  if (v == nullptr || strcmp(v, "1") != 0) return;
  fprintf(stderr, "[bcq] %s M=%d K=%d b=%d dtype=%s -> %s\n", fn, st->M, st->K, b,
          st->scale_dtype == BCQ_F16 ? "f16" : "f32", route);
}

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
  const size_t mg = (size_t)st->M * (st->K / kGroup) * es;  // bytes of one [M][G] plane
  for (int32_t r0 = 0; r0 < b; r0 += bcq::kMaxReq) {
    const int n = (b - r0) < bcq::kMaxReq ? (b - r0) : bcq::kMaxReq;
    int pmax = 0;
    for (int q = 0; q < n; ++q) pmax = p_of[r0 + q] > pmax ? p_of[r0 + q] : pmax;
    // one staged array per plane of each distinct precision, plus its offsets
    bcq::ReqTables t{};
    for (int p = 1; p <= BCQ_MAX_PLANES; ++p) {
      uint32_t mask = 0;
      for (int q = 0; q < n; ++q)
        if (p_of[r0 + q] == p) mask |= 1u << q;
      if (mask == 0) continue;
      for (int i = 0; i <= p; ++i) {
        const char *base = static_cast<const char *>(i < p ? st->alpha[p] : st->zero[p]);
        t.arr[t.n] = i < p ? base + i * mg : base;
        t.slot[t.n] = i < p ? i : bcq::sk_zero_slot(pmax);
        t.mask[t.n] = mask;
        ++t.n;
      }
    }
    for (int k = t.n; k < bcq::kMaxStage; ++k) t.arr[k] = t.arr[0];
    const char *xr = X + (size_t)r0 * ldx * es;
    char *yr = Y + (size_t)r0 * ldy * es;
    hipError_t e;
    if (n == 1)
      e = bcq::launch_gemv_lut(st->bits, st->M, st->K, pmax, st->alpha[pmax], st->zero[pmax], xr,
                               yr, st->scale_dtype, stream);
    else
      e = bcq::launch_skinny_lut(st->bits, st->M, st->K, pmax, t, n, xr, ldx, yr, ldy,
                                 st->scale_dtype, stream);
    if (e != hipSuccess) return BCQ_ERR_HIP;
  }
  return BCQ_OK;
}

// fp16 requests through the matrix-core kernel in launches of up to `chunk`
// requests.  The kernel decodes p planes with alpha[p] / zero[p]; p_of (host,
// b values, or nullptr for all p) gives each request's own precision, every
// one of which must read the same tables (checked by the caller).
bcq_status run_mfma_batches(const bcq_store *st, int32_t p, const int32_t *p_of, const char *X,
                            int32_t b, int32_t ldx, char *Y, int32_t ldy, void *ws, int chunk,
                            hipStream_t stream) {
  const size_t es = 2;
  for (int32_t r0 = 0; r0 < b; r0 += chunk) {
    const int n = (b - r0) < chunk ? (b - r0) : chunk;
    hipError_t e = bcq::launch_gemm_mfma(st->bits, st->M, st->K, p, st->alpha[p], st->zero[p],
                                         X + (size_t)r0 * ldx * es, ldx, n,
                                         Y + (size_t)r0 * ldy * es, ldy, ws,
                                         p_of != nullptr ? p_of + r0 : nullptr, stream);
    if (e != hipSuccess) return BCQ_ERR_HIP;
  }
  return BCQ_OK;
}

// Workspace checks shared by the batched products.
bcq_status check_workspace(const bcq_store *st, int32_t b, const void *ws, size_t ws_bytes) {
  const size_t need = bcq_workspace_bytes(st, b);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return BCQ_ERR_INVALID_ARG;
  if (need > 0 && !aligned(ws, 4)) return BCQ_ERR_ALIGNMENT;
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
  log_route("bcq_gemv", store, 1, "batch-1 tables");
  return hip_status(bcq::launch_gemv_lut(store->bits, store->M, store->K, p, store->alpha[p],
                                         store->zero[p], x, y, store->scale_dtype, stream));
}

bcq_status bcq_gemv_gate_up(const bcq_store *store, int32_t p, const void *x, bcq_dtype x_dtype,
                            void *y, bcq_dtype y_dtype, hipStream_t stream) {
  BCQ_TRY(check_store(store));
  BCQ_TRY(check_precision(store, p));
  BCQ_TRY(check_dtypes(store, x_dtype, y_dtype));
  if (store->M % bcq::kTileRows != 0) return BCQ_ERR_INVALID_ARG;
  if (x == nullptr || y == nullptr) return BCQ_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, dtype_size(y_dtype))) return BCQ_ERR_ALIGNMENT;
  return hip_status(bcq::launch_gemv_gate_up(store->bits, store->M, store->K, p,
                                             store->alpha[p], store->zero[p], x, y,
                                             store->scale_dtype, stream));
}

bcq_status bcq_gemm_gate_up(const bcq_store *store, const int32_t *p_host, const void *X,
                            int32_t b, int32_t ldx, bcq_dtype x_dtype, void *Y, int32_t ldy,
                            bcq_dtype y_dtype, hipStream_t stream) {
  BCQ_TRY(check_store(store));
  BCQ_TRY(check_dtypes(store, x_dtype, y_dtype));
  if (store->M % bcq::kTileRows != 0) return BCQ_ERR_INVALID_ARG;
  if (X == nullptr || Y == nullptr || p_host == nullptr) return BCQ_ERR_INVALID_ARG;
  if (b < 1 || b > BCQ_MAX_BATCH || ldx < store->K || ldy < store->M / 2)
    return BCQ_ERR_INVALID_ARG;
  const size_t es = dtype_size(store->scale_dtype);
  if (!aligned(X, 16) || ((size_t)ldx * es) % 16 != 0 || !aligned(Y, es)) return BCQ_ERR_ALIGNMENT;
  for (int32_t r = 0; r < b; ++r) BCQ_TRY(check_precision(store, p_host[r]));
  const char *Xc = static_cast<const char *>(X);
  char *Yc = static_cast<char *>(Y);
  int32_t pmax = 0;
  bool shared = true;
  for (int32_t r = 0; r < b; ++r) pmax = p_host[r] > pmax ? p_host[r] : pmax;
  for (int32_t r = 0; r < b; ++r)
    shared = shared && store->alpha[p_host[r]] == store->alpha[pmax] &&
             store->zero[p_host[r]] == store->zero[pmax];
  if (store->scale_dtype == BCQ_F16 && shared && b >= 2 && bcq::mfma_gate_up_ok(store->K, 16)) {
    // launches of up to 16 requests on the matrix cores, each at the largest
    // precision of its requests, every request summing its own planes
    log_route("bcq_gemm_gate_up", store, b, "matrix cores, whole K, silu(gate)*up epilogue");
    for (int32_t r0 = 0; r0 < b; r0 += 16) {
      const int n = (b - r0) < 16 ? (b - r0) : 16;
      int32_t pm = 0;
      for (int q = 0; q < n; ++q) pm = p_host[r0 + q] > pm ? p_host[r0 + q] : pm;
      hipError_t e = bcq::launch_gemm_gate_up(store->bits, store->M, store->K, pm,
                                              store->alpha[pm], store->zero[pm],
                                              Xc + (size_t)r0 * ldx * es, ldx, n,
                                              Yc + (size_t)r0 * ldy * es, ldy, p_host + r0, stream);
      if (e != hipSuccess) return BCQ_ERR_HIP;
    }
    return BCQ_OK;
  }
  // otherwise the batch-1 fused kernel, request by request, each with its own
  // precision's tables
  log_route("bcq_gemm_gate_up", store, b, "batch-1 fused kernel per request");
  for (int32_t r = 0; r < b; ++r) {
    const int32_t p = p_host[r];
    hipError_t e = bcq::launch_gemv_gate_up(store->bits, store->M, store->K, p, store->alpha[p],
                                            store->zero[p], Xc + (size_t)r * ldx * es,
                                            Yc + (size_t)r * ldy * es, store->scale_dtype, stream);
    if (e != hipSuccess) return BCQ_ERR_HIP;
  }
  return BCQ_OK;
}

bcq_status bcq_dequantize(const bcq_store *store, int32_t p, void *W, int32_t ldw,
                          bcq_dtype w_dtype, hipStream_t stream) {
  BCQ_TRY(check_store(store));
  BCQ_TRY(check_precision(store, p));
  if (w_dtype != BCQ_F16 && w_dtype != BCQ_F32) return BCQ_ERR_INVALID_ARG;
  if (w_dtype != store->scale_dtype) return BCQ_ERR_UNSUPPORTED;
  if (W == nullptr || ldw < store->K) return BCQ_ERR_INVALID_ARG;
  if (!aligned(W, 16) || ((size_t)ldw * dtype_size(w_dtype)) % 16 != 0) return BCQ_ERR_ALIGNMENT;
  return hip_status(bcq::launch_dequant(store->bits, store->M, store->K, p, store->alpha[p],
                                        store->zero[p], W, ldw, w_dtype, stream));
}

bcq_status bcq_lowrank_correct(const uint32_t *u_signs, const uint32_t *v_signs,
                               const void *alpha, int32_t R, int32_t M, int32_t K, const void *x,
                               void *y, bcq_dtype dtype, float *z, hipStream_t stream) {
  if (dtype != BCQ_F16 && dtype != BCQ_F32) return BCQ_ERR_INVALID_ARG;
  if (R < 1 || R > BCQ_LOWRANK_MAX_RANK || M < 1 || K < 32 || K % 32 != 0)
    return BCQ_ERR_INVALID_ARG;
  if (u_signs == nullptr || v_signs == nullptr || alpha == nullptr || x == nullptr ||
      y == nullptr || z == nullptr)
    return BCQ_ERR_INVALID_ARG;
  const size_t es = dtype_size(dtype);
  if (!aligned(u_signs, 4) || !aligned(v_signs, 4) || !aligned(z, 4) || !aligned(alpha, es) ||
      !aligned(x, 16) || !aligned(y, es))
    return BCQ_ERR_ALIGNMENT;
  return hip_status(bcq::launch_lowrank(u_signs, v_signs, alpha, R, M, K, x, y, dtype, z, stream));
}

bcq_status bcq_gemv_lowrank(const bcq_store *store, int32_t p, const void *x, bcq_dtype x_dtype,
                            const uint32_t *u_signs, const uint32_t *v_signs,
                            const void *lr_alpha, int32_t R, void *y, bcq_dtype y_dtype, float *z,
                            hipStream_t stream) {
  BCQ_TRY(check_store(store));
  BCQ_TRY(check_precision(store, p));
  BCQ_TRY(check_dtypes(store, x_dtype, y_dtype));
  if (R < 1 || R > BCQ_LOWRANK_MAX_RANK) return BCQ_ERR_INVALID_ARG;
  if (x == nullptr || y == nullptr || u_signs == nullptr || v_signs == nullptr ||
      lr_alpha == nullptr || z == nullptr)
    return BCQ_ERR_INVALID_ARG;
  const bcq_dtype dt = store->scale_dtype;
  if (!aligned(x, 16) || !aligned(y, dtype_size(y_dtype)) || !aligned(u_signs, 4) ||
      !aligned(v_signs, 4) || !aligned(z, 4) || !aligned(lr_alpha, dtype_size(dt)))
    return BCQ_ERR_ALIGNMENT;
  const bool fused = bcq::gemv_lowrank_fused_ok(store->K, R);
  log_route("bcq_gemv_lowrank", store, 1,
            fused ? "batch-1 tables, correction in the writeback" : "batch-1 tables, then correction");
  if (bcq::launch_lowrank_z(v_signs, lr_alpha, R, store->K, x, z, dt, stream) != hipSuccess)
    return BCQ_ERR_HIP;
  if (fused)
    return hip_status(bcq::launch_gemv_lowrank(store->bits, store->M, store->K, p,
                                               store->alpha[p], store->zero[p], x, y, u_signs, z,
                                               R, dt, stream));
  if (bcq::launch_gemv_lut(store->bits, store->M, store->K, p, store->alpha[p], store->zero[p], x,
                           y, dt, stream) != hipSuccess)
    return BCQ_ERR_HIP;
  return hip_status(bcq::launch_lowrank_expand(u_signs, R, store->M, z, y, dt, stream));
}

size_t bcq_workspace_bytes(const bcq_store *store, int32_t b) {
  if (check_store(store) != BCQ_OK || b < 1 || b > BCQ_MAX_BATCH) return 0;
  if (!on_matrix_cores(store, b)) return 0;
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
  BCQ_TRY(check_workspace(store, b, workspace, workspace_bytes));
  const char *Xc = static_cast<const char *>(X);
  char *Yc = static_cast<char *>(Y);
  if (on_matrix_cores(store, b)) {
    log_route("bcq_gemm_skinny", store, b,
              bcq::mfma_streamed(store->M, store->K, b)
                  ? "matrix cores, whole K, requests streamed"
                  : bcq::mfma_whole_k(store->M, store->K,
                                      b < bcq::kMfMaxBatch ? b : bcq::kMfMaxBatch)
                        ? "matrix cores, whole K"
                        : "matrix cores, split K");
    // the streamed whole-K kernel takes the whole batch in one launch
    const int chunk = bcq::mfma_streamed(store->M, store->K, b) ? BCQ_MAX_BATCH : bcq::kMfMaxBatch;
    return run_mfma_batches(store, p, nullptr, Xc, b, ldx, Yc, ldy, workspace, chunk, stream);
  }
  log_route("bcq_gemm_skinny", store, b, b == 1 ? "batch-1 tables" : "vector-ALU tables");
  int32_t ps[BCQ_MAX_BATCH];
  for (int32_t r = 0; r < b; ++r) ps[r] = p;
  return run_table_batches(store, ps, Xc, b, ldx, Yc, ldy, stream);
}

bcq_status bcq_gemv_mixed_p(const bcq_store *store, const int32_t *p_host, const void *X,
                            int32_t b, int32_t ldx, bcq_dtype x_dtype, void *Y, int32_t ldy,
                            bcq_dtype y_dtype, void *workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  BCQ_TRY(check_store(store));
  BCQ_TRY(check_dtypes(store, x_dtype, y_dtype));
  BCQ_TRY(check_batch(store, X, b, ldx, Y, ldy));
  if (p_host == nullptr) return BCQ_ERR_INVALID_ARG;
  for (int32_t r = 0; r < b; ++r) BCQ_TRY(check_precision(store, p_host[r]));
  BCQ_TRY(check_workspace(store, b, workspace, workspace_bytes));
  const char *Xc = static_cast<const char *>(X);
  char *Yc = static_cast<char *>(Y);
  // one decode of the largest precision serves every request when all of
  // them read the same tables (the shared-store layout: alpha[p] and zero[p]
  // alias those of the largest p); otherwise each request's tables are staged
  // separately by the table kernel
  int32_t pmax = 0;
  for (int32_t r = 0; r < b; ++r) pmax = p_host[r] > pmax ? p_host[r] : pmax;
  bool shared = true;
  for (int32_t r = 0; r < b; ++r)
    shared = shared && store->alpha[p_host[r]] == store->alpha[pmax] &&
             store->zero[p_host[r]] == store->zero[pmax];
  if (on_matrix_cores(store, b) && shared) {
    log_route("bcq_gemv_mixed_p", store, b, "matrix cores, per-plane accumulators");
    return run_mfma_batches(store, pmax, p_host, Xc, b, ldx, Yc, ldy, workspace,
                            bcq::kMfMaxMixed, stream);
  }
  log_route("bcq_gemv_mixed_p", store, b, "vector-ALU tables, per-request scale slots");
  return run_table_batches(store, p_host, Xc, b, ldx, Yc, ldy, stream);
}

bcq_status bcq_quantize(const void *W, bcq_dtype w_dtype, int32_t M, int32_t K, int32_t ldw,
                        int32_t P, int32_t p_low, int32_t iters, uint32_t *signs, void *alpha,
                        void *zero, bcq_dtype out_dtype, hipStream_t stream) {
  if (W == nullptr || signs == nullptr || alpha == nullptr || zero == nullptr)
    return BCQ_ERR_INVALID_ARG;
  if (w_dtype != BCQ_F16 && w_dtype != BCQ_F32) return BCQ_ERR_INVALID_ARG;
  if (out_dtype != BCQ_F16 && out_dtype != BCQ_F32 && out_dtype != BCQ_F64)
    return BCQ_ERR_INVALID_ARG;
  BCQ_TRY(check_shape(P, M, K));
  if (p_low < 1 || p_low > P || iters < 0 || iters > 1000 || ldw < K) return BCQ_ERR_INVALID_ARG;
  const size_t ws = w_dtype == BCQ_F16 ? 2 : 4;
  const size_t os = out_dtype == BCQ_F16 ? 2 : out_dtype == BCQ_F32 ? 4 : 8;
  if (!aligned(W, ws) || !aligned(signs, 4) || !aligned(alpha, os) || !aligned(zero, os))
    return BCQ_ERR_ALIGNMENT;
  return hip_status(bcq::launch_quantize(W, w_dtype, ldw, M, K, P, p_low, iters, signs, alpha,
                                         zero, out_dtype, stream));
}

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (the current device, which
// the stream must belong to), looked up once per device.  nullptr if HIP
// reports an error.
void *scratch_for_current_device(hipStream_t stream, bcq_status *err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = BCQ_ERR_HIP;
    return nullptr;
  }
  if (stream != nullptr) {
    int sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) {
      *err = BCQ_ERR_HIP;
      return nullptr;
    }
    if (sdev != dev) {
      *err = BCQ_ERR_INVALID_ARG;
      return nullptr;
    }
  }
  void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      *err = BCQ_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace

bcq_status bcq_gemm_skinny_noalloc(const bcq_store *store, int32_t p, const void *X, int32_t b,
                                   int32_t ldx, bcq_dtype x_dtype, void *Y, int32_t ldy,
                                   bcq_dtype y_dtype, hipStream_t stream) {
  BCQ_TRY(check_store(store));
  BCQ_TRY(check_precision(store, p));
  BCQ_TRY(check_dtypes(store, x_dtype, y_dtype));
  BCQ_TRY(check_batch(store, X, b, ldx, Y, ldy));
  const size_t need = bcq_workspace_bytes(store, b);
  if (need > (size_t)BCQ_NOALLOC_SCRATCH_BYTES) return BCQ_ERR_TOO_LARGE;
  void *ws = nullptr;
  if (need > 0) {
    bcq_status err = BCQ_OK;
    ws = scratch_for_current_device(stream, &err);
    if (ws == nullptr) return err;
  }
  return bcq_gemm_skinny(store, p, X, b, ldx, x_dtype, Y, ldy, y_dtype, ws, need, stream);
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
    case BCQ_ERR_TOO_LARGE:
      return "BCQ_ERR_TOO_LARGE: the call needs more device scratch than the allocation-free "
             "entry point holds (BCQ_NOALLOC_SCRATCH_BYTES); use bcq_gemm_skinny with a workspace";
  }
  return "unknown bcq_status";
}

}  // extern "C"
