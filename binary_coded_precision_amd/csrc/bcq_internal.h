// bcq_internal.h -- declarations shared by the library's translation units
// (host-side launchers and the packed-layout arithmetic).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bcq.h"

namespace bcq {

// Packed layout (see bcq_packed_bytes in bcq.h): one uint4 holds the 128 sign
// bits of one (plane, row, group); uint4 index = ((i*MT + t)*G + j)*16 + r.
constexpr int kTileRows = BCQ_TILE_ROWS;
constexpr int kGroup = BCQ_GROUP;

inline int row_tiles(int M) { return (M + kTileRows - 1) / kTileRows; }

// Per-request description used by the batched kernels: each request has its
// own precision and its own scale/offset tables (AnyBCQ per-request precision).
constexpr int kMaxReq = 8;  // requests handled by one launch of a batched kernel
struct ReqTables {
  const void *alpha[kMaxReq];  // [p_r][M][G]
  const void *zero[kMaxReq];   // [M][G]
  int p[kMaxReq];              // precision of each request (0 for padding slots)
};

// ---- launchers (return hipGetLastError() after the launch) ----
hipError_t launch_pack(const uint32_t *signs, int P, int M, int K, uint32_t *packed,
                       hipStream_t s);
hipError_t launch_unpack(const uint32_t *packed, int P, int M, int K, uint32_t *signs,
                         hipStream_t s);

// Batch-1 product: table-lookup kernel.
hipError_t launch_gemv_lut(const uint32_t *bits, int M, int K, int p, const void *alpha,
                           const void *zero, const void *x, void *y, bcq_dtype dt,
                           hipStream_t s);

// Batched products with 2..8 requests per launch (vector ALUs, shared tables).
// x rows at x + r*ldx, y rows at y + r*ldy, r < nreq; p_max = max of t.p[].
hipError_t launch_skinny_lut(const uint32_t *bits, int M, int K, int p_max, const ReqTables &t,
                             int nreq, const void *x, int ldx, void *y, int ldy, bcq_dtype dt,
                             hipStream_t s);

// Batched products with >= 16 requests at one precision: fp16 dequantised
// tiles on the matrix cores.
// fp16 only, b <= 64 per launch; ws holds mfma_workspace_bytes(M, K, b) bytes.
hipError_t launch_gemm_mfma(const uint32_t *bits, int M, int K, int p, const void *alpha,
                            const void *zero, const void *x, int ldx, int b, void *y, int ldy,
                            void *ws, hipStream_t s);
int mfma_slices(int M, int K);
size_t mfma_workspace_bytes(int M, int K, int b);

}  // namespace bcq
