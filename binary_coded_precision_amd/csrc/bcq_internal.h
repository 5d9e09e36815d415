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

// The gated-MLP epilogue of a gate/up store: silu(g) * u with
// silu(g) = g / (1 + exp(-g)), in fp32.
__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.f + expf(-g)) * u; }

// Scale description used by the batched table kernel.  Each request of a
// launch has its own precision and reads the scale/offset tables of that
// precision (AnyBCQ per-request precision).  The host lists every distinct
// [M][G] array the launch needs -- one per plane of each distinct alpha[p],
// plus zero[p] -- with the slot it fills and the requests that read it; the
// kernel stages each array once per window and fans it out to those requests.
constexpr int kMaxReq = 8;     // requests handled by one launch of the batched kernel
constexpr int kMaxStage = 16;  // distinct arrays per launch (at most 4+3+2+1 + 4 offsets)
struct ReqTables {
  const void *arr[kMaxStage];  // [M][G] array: one plane of some alpha[p], or zero[p]
  int slot[kMaxStage];         // 0..pmax-1: plane index; pmax: offsets
  uint32_t mask[kMaxStage];    // bit q set: request q of the launch reads this array
  int n;                       // arrays in use, 1..kMaxStage
};
// The batched kernel works on planes in pairs, so it reserves an even number
// of plane slots; the offsets go in the slot after them.
constexpr int sk_zero_slot(int pmax) { return 2 * ((pmax + 1) / 2); }

// ---- launchers (return hipGetLastError() after the launch) ----
hipError_t launch_pack(const uint32_t *signs, int P, int M, int K, uint32_t *packed,
                       hipStream_t s);
hipError_t launch_unpack(const uint32_t *packed, int P, int M, int K, uint32_t *signs,
                         hipStream_t s);

// Batch-1 product: table-lookup kernel.
hipError_t launch_gemv_lut(const uint32_t *bits, int M, int K, int p, const void *alpha,
                           const void *zero, const void *x, void *y, bcq_dtype dt,
                           hipStream_t s);
// Gate/up store (rows interleaved in 8-row halves of each tile): y[j] =
// silu(gate_j . x) * (up_j . x) for j < M / 2.
hipError_t launch_gemv_gate_up(const uint32_t *bits, int M, int K, int p, const void *alpha,
                           const void *zero, const void *x, void *y, bcq_dtype dt,
                           hipStream_t s);

// Dense reconstruction W[m][k] = z + sum_{i<p} alpha_i s_i (bcq_dequantize).
hipError_t launch_dequant(const uint32_t *bits, int M, int K, int p, const void *alpha,
                          const void *zero, void *W, int ldw, bcq_dtype dt, hipStream_t s);

// Binary low-rank correction (bcq_lowrank_correct): y += sum_r alpha_r u_r (v_r . x).
constexpr int kLrMaxRank = BCQ_LOWRANK_MAX_RANK;
hipError_t launch_lowrank(const uint32_t *u, const uint32_t *v, const void *alpha, int R, int M,
                          int K, const void *x, void *y, bcq_dtype dt, float *z, hipStream_t s);
// Its two steps: z_r = alpha_r (v_r . x) into z (fp32), then y += U z.
hipError_t launch_lowrank_z(const uint32_t *v, const void *alpha, int R, int K, const void *x,
                            float *z, bcq_dtype dt, hipStream_t s);
hipError_t launch_lowrank_expand(const uint32_t *u, int R, int M, const float *z, void *y,
                                 bcq_dtype dt, hipStream_t s);
// Batch-1 product with the correction U z (z from launch_lowrank_z) added
// before the output is rounded, one launch; only where
// gemv_lowrank_fused_ok(K, R) (K <= 4096, R <= 1024).
bool gemv_lowrank_fused_ok(int K, int R);
hipError_t launch_gemv_lowrank(const uint32_t *bits, int M, int K, int p, const void *alpha,
                               const void *zero, const void *x, void *y, const uint32_t *u,
                               const float *z, int R, bcq_dtype dt, hipStream_t s);

// Progressive-precision quantizer (bcq_quantize): W [M][ldw] of w_dt (fp16 or
// fp32) -> canonical signs [P][M][K/32] and the scale / offset tables of
// precisions p_low..P in out_dt (fp16, fp32 or fp64).
hipError_t launch_quantize(const void *W, bcq_dtype w_dt, int ldw, int M, int K, int P,
                           int p_low, int iters, uint32_t *signs, void *alpha, void *zero,
                           bcq_dtype out_dt, hipStream_t s);

// Batched products with 2..8 requests per launch (vector ALUs, shared tables).
// x rows at x + r*ldx, y rows at y + r*ldy, r < nreq; p_max = max of t.p[].
hipError_t launch_skinny_lut(const uint32_t *bits, int M, int K, int p_max, const ReqTables &t,
                             int nreq, const void *x, int ldx, void *y, int ldy, bcq_dtype dt,
                             hipStream_t s);

// Batched fp16 products on the matrix cores (weights decoded to fp16 tiles).
// p planes are decoded with the tables alpha ([p][M][G]) and zero; request q
// uses the first p_req[q] of them (p_req: host array of b values in 1..p, or
// nullptr for all p).  Per-request precisions need b <= kMfMaxMixed; otherwise
// b <= kMfMaxBatch per launch (a call with more runs several launches in
// order), or b <= BCQ_MAX_BATCH where mfma_streamed holds.  ws holds at least mfma_workspace_bytes(M, K, b) bytes for the call's
// whole batch b (nullptr when that is 0: launches that keep K within one
// workgroup need none).
constexpr int kMfMaxBatch = 64;
constexpr int kMfMaxMixed = 32;
hipError_t launch_gemm_mfma(const uint32_t *bits, int M, int K, int p, const void *alpha,
                            const void *zero, const void *x, int ldx, int b, void *y, int ldy,
                            void *ws, const int32_t *p_req, hipStream_t s);
size_t mfma_workspace_bytes(int M, int K, int b);

// Gate/up stores at batch b <= 16 with K <= 4096 (mfma_gate_up_ok), fp16:
// the whole-K matrix-core kernel with the silu(gate) * up epilogue; request
// q at precision p_req[q] (host, b values in 1..p; nullptr: all p), the tables
// alpha / zero of precision p serving every request.  Y is [b][ldy], M / 2
// outputs per request.
bool mfma_gate_up_ok(int K, int n);
hipError_t launch_gemm_gate_up(const uint32_t *bits, int M, int K, int p, const void *alpha,
                               const void *zero, const void *x, int ldx, int b, void *y, int ldy,
                               const int32_t *p_req, hipStream_t s);

// True when a launch of n fp16 requests on (M, K) keeps K within one
// workgroup (no workspace, no second kernel).
bool mfma_whole_k(int M, int K, int n);
// True when a uniform-precision launch of n fp16 requests on (M, K) runs the
// streamed whole-K kernel, which takes up to BCQ_MAX_BATCH requests in one
// launch (the weights decoded once for all of them).
bool mfma_streamed(int M, int K, int n);

}  // namespace bcq
