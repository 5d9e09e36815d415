/*
 * bcq.h -- C ABI of the MI355X (gfx950) binary-coded quantization (BCQ) library.
 *
 * The operation (AnyBCQ paper notes, "Method / key designs", and the AnyBCQ
 * abstract on the mlsanity page): a weight matrix W [M][K] is held as P binary
 * planes B_1..B_P with entries in {-1,+1}, a scale per plane and per
 * (row, group of g = 128 columns), and one offset z per (row, group)
 * (asymmetric, group-wise BCQ: AnyBCQ paper notes, "Training strategy").  A
 * product at precision p <= P uses only the first p planes:
 *
 *     y[m] = sum_j [ sum_{i<p} alpha_p[i][m][j] * (sum_{k in group j} s_i[m][k] x[k])
 *                    + zero_p[m][j] * (sum_{k in group j} x[k]) ]
 *
 * One stored set of planes serves every precision, and the precision may be
 * chosen per call or per request (AnyBCQ paper notes, "overall framework" and
 * "progressive precision expansion"; abstract: per-request precision).  Reading
 * the first p planes must not touch the others, so each plane is a separate
 * contiguous array in device memory.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the parameter name ends in _host.
 *    The caller allocates and owns all memory; the library allocates nothing
 *    and keeps no state between calls.
 *  - Calls that take a stream validate their arguments on the host first.  A
 *    failed check returns an error and enqueues nothing.  A passing call
 *    enqueues its kernels on `stream` and returns without synchronising.
 *    BCQ_ERR_HIP reports a launch failure (hipGetLastError after the launch).
 *  - Calls on different streams are independent.  Calls that share output
 *    buffers must be ordered by the caller.
 *  - Dtypes: scales, activations and outputs use one dtype per call
 *    (BCQ_F16 or BCQ_F32); other pairings return BCQ_ERR_UNSUPPORTED.
 *    Products accumulate in fp32 and round once (to nearest even) at writeback.
 *    Two fp16 routes also round an intermediate once to fp16, each adding at
 *    most 2^-11 of an output's term magnitude sum_k |w_k x_k| to its error:
 *    the summed decode of the matrix cores (see bcq_gemm_skinny), and the
 *    batch-1 tables for 4096 < K <= 28672 (and for 2048 < K <= 4096 when
 *    the call has 129 to 256 row tiles of 16 rows), whose entries (sums of
 *    four signed activations, formed in fp32) are held in fp16.
 *  - Shapes: K must be a positive multiple of 128 (group_size must be 128),
 *    M >= 1, 1 <= p <= planes <= 4.
 */
#ifndef BCQ_H_
#define BCQ_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BCQ_MAX_PLANES 4
#define BCQ_GROUP 128
/* Rows per tile of the packed device layout (see bcq_pack_planes). */
#define BCQ_TILE_ROWS 16
/* Largest batch accepted by bcq_gemm_skinny / bcq_gemv_mixed_p in one call. */
#define BCQ_MAX_BATCH 256
/* Largest rank accepted by bcq_lowrank_correct and bcq_gemv_lowrank. */
#define BCQ_LOWRANK_MAX_RANK 4096
/* bcq_gemv_lowrank adds the correction inside the product's own launch (one
 * rounding of y) for K <= 4096 and R up to this rank. */
#define BCQ_LOWRANK_FUSED_MAX_RANK 1024
/* Device scratch held by the library for bcq_gemm_skinny_noalloc, per GPU. */
#define BCQ_NOALLOC_SCRATCH_BYTES (16u << 20)

typedef enum {
  BCQ_OK = 0,
  BCQ_ERR_INVALID_ARG = -1, /* null pointer, bad shape, p out of range, bad leading dim */
  BCQ_ERR_UNSUPPORTED = -2, /* valid but not implemented: dtype pairing, group size != 128 */
  BCQ_ERR_ALIGNMENT = -3,   /* a pointer or leading dimension breaks the alignment rules */
  BCQ_ERR_HIP = -4,         /* the HIP runtime reported an error for a launch */
  BCQ_ERR_TOO_LARGE = -5    /* bcq_gemm_skinny_noalloc: the call needs more scratch than it holds */
} bcq_status;

/* BCQ_F64 is accepted only for bcq_quantize's scale and offset tables. */
typedef enum { BCQ_F16 = 1, BCQ_F32 = 2, BCQ_F64 = 3 } bcq_dtype;

/*
 * A packed store: the planes in device layout plus the scale tables.
 *
 * bits:  written by bcq_pack_planes for (planes, M, K); 16-byte aligned.
 * alpha[p], zero[p] for p = 1..planes: the tables used at precision p.
 *   alpha[p] -> [p][M][K/128] scales, zero[p] -> [M][K/128] offsets, dtype
 *   scale_dtype, row-major, element aligned.  AnyBCQ refits every scale when it
 *   adds a plane, so each precision may have its own tables; when one table is
 *   shared, alpha[p] for every p may point at the same [planes][M][K/128]
 *   buffer (its first p planes are the table for precision p) and all zero[p]
 *   may alias.  alpha[0] and zero[0] are ignored.  Only the entries for the
 *   precisions a call uses must be non-null.
 */
typedef struct {
  int32_t M;
  int32_t K;
  int32_t group_size; /* must be 128 */
  int32_t planes;     /* P stored planes, 1..4 */
  const uint32_t *bits;
  bcq_dtype scale_dtype;
  const void *alpha[BCQ_MAX_PLANES + 1];
  const void *zero[BCQ_MAX_PLANES + 1];
} bcq_store;

/*
 * Bytes of the packed device layout for (P, M, K), or 0 if the shape is
 * invalid.  Layout: plane-major; within a plane, rows in tiles of 16 (the last
 * tile padded with clear bits); within a tile, group-major; within a group, the
 * 16 rows' 128 bits (16 bytes each) are contiguous.  So word index =
 * (((i*MT + t)*G + j)*16 + r)*4 + q with MT = ceil(M/16), G = K/128,
 * row m = 16t + r, columns 128j + 32q .. 128j + 32q + 31; within that word,
 * bit b holds column 128j + 32q + 2b for b < 16 and 128j + 32q + 2(b-16) + 1
 * for b >= 16 (even columns in the low half, odd columns in the high half).
 * The first p planes are a contiguous prefix of p * (bytes / P) bytes.
 */
size_t bcq_packed_bytes(int32_t P, int32_t M, int32_t K);

/*
 * Pack canonical sign planes into the device layout.
 * Defined by: AnyBCQ paper notes, "Method / key designs" (direct bit-plane
 * kernel): the planes are consumed one at a time and a precision-p product
 * loads only the first p of them, so each plane is stored as its own
 * contiguous array and the first p planes form a prefix of the buffer.  The
 * planes hold -1/+1 entries ("Method / key designs", the weight as a sum of
 * scaled binary planes), one bit each.
 * signs:  [P][M][K/32] uint32; column k of plane i, row m is bit (k mod 32),
 *         least significant first, of word [i][m][k/32]; set = +1, clear = -1.
 *         4-byte aligned.
 * packed: bcq_packed_bytes(P, M, K) bytes, 16-byte aligned; fully overwritten.
 * The round trip through bcq_unpack_planes is bit-exact.
 */
bcq_status bcq_pack_planes(const uint32_t *signs, int32_t P, int32_t M, int32_t K,
                           uint32_t *packed, hipStream_t stream);

/*
 * Inverse of bcq_pack_planes (for tests and inspection): the canonical
 * [P][M][K/32] sign words back from the device layout, bit-exact.  Same
 * source as bcq_pack_planes (AnyBCQ paper notes, "Method / key designs": one
 * bit per -1/+1 plane entry).  signs is fully overwritten; alignment and
 * validation as in bcq_pack_planes.
 */
bcq_status bcq_unpack_planes(const uint32_t *packed, int32_t P, int32_t M, int32_t K,
                             uint32_t *signs, hipStream_t stream);

/*
 * y = BCQ product at precision p for one activation vector (batch 1).
 * Defined by: AnyBCQ paper notes, "Method / key designs" (direct bit-plane
 * kernel): for each of the first p planes the product with x is additions and
 * subtractions of activations, scaled by that plane's factor and accumulated;
 * the output is written once the p-th plane is done, and a lower precision
 * reads fewer planes.  The group-wise offset term comes from "Training
 * strategy" (asymmetric BCQ, g = 128).  The mlsanity page's AnyBCQ abstract
 * states the same kernel goal: compute directly on the bit-planes and touch
 * only the planes of the precision a request asks for.
 * x: [K], 16-byte aligned.  y: [M], element aligned; every element written.
 * Rejected arguments (null pointers, p outside [1, planes], a missing table
 * for p, mixed dtypes, misalignment) return an error and enqueue nothing.
 */
bcq_status bcq_gemv(const bcq_store *store, int32_t p, const void *x, bcq_dtype x_dtype,
                    void *y, bcq_dtype y_dtype, hipStream_t stream);

/*
 * Gated-MLP epilogue fused into one product at batch 1: y[j] = silu(g_j) * u_j
 * with g_j and u_j the BCQ products (precision p) of gate row j and up row j,
 * and silu(g) = g / (1 + exp(-g)), evaluated in fp32 on the fp32 sums and
 * rounded once.  This is the consumer of the gate and up projections of the
 * MLP-shaped workload (two products of the same x); one launch serves both,
 * sharing the activation tables.
 * store: 2 * Mo rows, Mo a multiple of 8 (store->M a multiple of 16), packed
 *   so that rows 0..7 of every 16-row tile t are gate rows 8t..8t+7 and rows
 *   8..15 the up rows 8t..8t+7 (canonical row 16t + i holds gate row 8t + i,
 *   row 16t + 8 + i up row 8t + i, before bcq_pack_planes); the scale and
 *   offset tables follow the same row order.  Otherwise BCQ_ERR_INVALID_ARG.
 * x: [K], 16-byte aligned.  y: [Mo] = [store->M / 2], element aligned.
 * Dtypes, validation and stream behaviour as in bcq_gemv.
 */
bcq_status bcq_gemv_gate_up(const bcq_store *store, int32_t p, const void *x, bcq_dtype x_dtype,
                            void *y, bcq_dtype y_dtype, hipStream_t stream);

/*
 * The gated-MLP epilogue of bcq_gemv_gate_up for a batch of requests, each at
 * its own precision: Y[r][j] = silu(g_rj) * u_rj for j < M/2, where g_rj and
 * u_rj are the BCQ products at precision p_host[r] of gate row j and up row j
 * with X[r] (AnyBCQ paper notes, "Method / key designs" for the products and
 * "overall framework" for per-request precision), silu(g) = g / (1 +
 * exp(-g)) in fp32 on the fp32 sums, rounded once.  The store is laid out as
 * for bcq_gemv_gate_up (M a multiple of 16; rows 0..7 of each 16-row tile the
 * gate rows, 8..15 the matching up rows).
 * Routes: fp16 batches of 2 and more whose precisions read one shared scale
 * table (alpha[p], zero[p] aliasing those of the largest requested p) and
 * K <= 4096 run on the matrix cores in launches of up to 16 requests (the
 * whole-K kernel of bcq_gemm_skinny, each plane an exact fp16 operand, the
 * epilogue on the summed partial products); all other calls run the batch-1
 * fused kernel once per request.  No workspace.
 * p_host: [b] in HOST memory, every entry in [1, planes] with its tables
 *   present; X: [b][ldx] (ldx >= K, 16-byte aligned, ldx*size a multiple of
 *   16 bytes); Y: [b][ldy], ldy >= M/2, element aligned.  1 <= b <=
 *   BCQ_MAX_BATCH.  Dtypes, validation and stream behaviour as in bcq_gemv.
 */
bcq_status bcq_gemm_gate_up(const bcq_store *store, const int32_t *p_host, const void *X,
                            int32_t b, int32_t ldx, bcq_dtype x_dtype, void *Y, int32_t ldy,
                            bcq_dtype y_dtype, hipStream_t stream);

/*
 * Y[r] = BCQ product at precision p for each of b activation rows X[r].
 * Defined by: the product of bcq_gemv (AnyBCQ paper notes, "Method / key
 * designs") applied to every row of a decode batch; one read of the first p
 * planes serves all b requests.  The BiLoCo summary ("results: speed") notes
 * that add/subtract work grows with the batch while the weight read does not,
 * which is why larger batches decode weights for the matrix cores.
 * X: [b][ldx] (row r starts at X + r*ldx elements), 16-byte aligned, so ldx*size
 * must be a multiple of 16 bytes; ldx >= K.  Y: [b][ldy], ldy >= M, element
 * aligned.  1 <= b <= BCQ_MAX_BATCH.
 * Batch 1 runs the batch-1 kernel.  fp32 batches, and fp16 batches of 2 unless
 * K is past 2048 and stays within one workgroup (below), run on the vector
 * ALUs with sign-combination tables shared by up to 8 requests per launch
 * (exact fp32 sums of the stored values).  Other fp16 batches of 2, and those
 * of 3 and more,
 * decode tiles of W to fp16 once per launch of up to 64 requests (of the whole
 * batch, up to BCQ_MAX_BATCH, in the calls at one precision with
 * 2048 < K <= 4096 on 2049 to 4096 rows) and contract them with X on the
 * matrix cores (fp32 accumulation; in launches of up to 16
 * requests, and in per-request-precision launches of up to 32, each plane's
 * +-alpha is an exact fp16 operand; in larger launches at one precision the
 * decoded weight z + sum +-alpha is rounded to fp16).  Launches of up to 16 requests with
 * K <= 4096 keep K within one workgroup, except K <= 2048 on more than 256
 * tiles of 16 rows (M > 4096); so do calls of 17 to BCQ_MAX_BATCH requests
 * with 2048 < K <= 4096 on 2049 to 4096 rows.  Other launches split K over
 * workgroups and use bcq_workspace_bytes(store, b) bytes of device workspace
 * (4-byte aligned) for the K slices' partial sums: contents need no
 * initialisation and are clobbered by the call, so calls that may run at the
 * same time need separate workspaces.  That size depends on (M, K, b) only,
 * so it also covers the 17..256-request shapes just named, whose
 * per-request-precision calls split K; calls at one precision there leave the
 * workspace untouched.  workspace may be NULL when that size is 0; a smaller
 * workspace gives BCQ_ERR_INVALID_ARG.
 * Accuracy of the summed decode (fp16, launches of more than 16 requests at
 * one precision): every decoded weight z + sum +-alpha is rounded to fp16
 * (relative error up to 2^-11 of the weight) before the contraction, so an
 * output whose terms nearly cancel carries an absolute error of about
 * 2^-11 * sum_k |w_k x_k| rather than a small fraction of its own size; the
 * other routes use exact fp16 operands or fp32 tables.
 */
bcq_status bcq_gemm_skinny(const bcq_store *store, int32_t p, const void *X, int32_t b,
                           int32_t ldx, bcq_dtype x_dtype, void *Y, int32_t ldy,
                           bcq_dtype y_dtype, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Device workspace bcq_gemm_skinny and bcq_gemv_mixed_p need for a batch of b
 * (0 when none), or 0 for an invalid store.
 */
size_t bcq_workspace_bytes(const bcq_store *store, int32_t b);

/*
 * bcq_gemm_skinny without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same product, kernels, validation and
 * results as bcq_gemm_skinny (bit for bit); where that call would need a
 * workspace (bcq_workspace_bytes(store, b) > 0) this one uses a device array
 * the library holds, BCQ_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, kept from
 * the first use on that GPU until the process ends.  The call allocates
 * nothing (no hipMalloc or allocating library routine, on any path).
 * Limits and errors:
 *  - a call needing more than BCQ_NOALLOC_SCRATCH_BYTES returns
 *    BCQ_ERR_TOO_LARGE and enqueues nothing (every LLaMA-3.1-8B layer shape
 *    needs at most 8 MiB at any batch);
 *  - the stream must belong to the current device (BCQ_ERR_INVALID_ARG);
 *  - all calls on one GPU share its one array: calls that may run at the same
 *    time on that GPU (on different streams, or from different threads) race
 *    on it and must be ordered by the caller.  Nothing in it needs clearing:
 *    each call writes every partial sum before reading it.
 */
bcq_status bcq_gemm_skinny_noalloc(const bcq_store *store, int32_t p, const void *X, int32_t b,
                                   int32_t ldx, bcq_dtype x_dtype, void *Y, int32_t ldy,
                                   bcq_dtype y_dtype, hipStream_t stream);

/*
 * Per-request precision: Y[r] = BCQ product of X[r] at precision p_host[r],
 * using alpha[p_host[r]] and zero[p_host[r]].
 * Defined by: AnyBCQ paper notes, "overall framework" (online inference loads
 * the bit-planes a request needs and lets each request pick its precision)
 * and "key designs" (per-precision scales refitted over shared planes); the
 * mlsanity page's AnyBCQ abstract names per-request precision selection with
 * negligible switching overhead.  Every plane up to the largest
 * requested precision is read once per launch for all its requests, so mixing
 * precisions costs no extra plane traffic.  When every requested precision's
 * tables alias those of the largest one (one shared [P][M][G] scale array and
 * one offset array, as a shared store lays them out), fp16 batches that
 * bcq_gemm_skinny would send to the matrix cores (3 and more, or 2 where K is
 * past 2048 and stays within one workgroup) run there in launches of up to 32:
 * each plane has its own accumulator and request r sums its first p_host[r]
 * planes.  Otherwise the
 * table kernel runs launches of up to 8, giving each request zero scales for
 * planes past its precision.
 * p_host: [b] in HOST memory; every entry must lie in [1, planes], otherwise
 * BCQ_ERR_INVALID_ARG and nothing is enqueued.  1 <= b <= BCQ_MAX_BATCH.
 * X, Y, ldx, ldy, workspace and workspace_bytes as in bcq_gemm_skinny (the
 * workspace size is bcq_workspace_bytes(store, b) here too).
 */
bcq_status bcq_gemv_mixed_p(const bcq_store *store, const int32_t *p_host, const void *X,
                            int32_t b, int32_t ldx, bcq_dtype x_dtype, void *Y, int32_t ldy,
                            bcq_dtype y_dtype, void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * Dense reconstruction of the weights at precision p (AnyBCQ paper notes,
 * "Method / key designs": a weight is the offset plus each plane's sign times
 * its scale), for large batches that go through a dense matrix product:
 *     W[m][k] = zero_p[m][k/128] + sum_{i<p} alpha_p[i][m][k/128] * s_i[m][k]
 * formed in fp32 as zero, then + or - each alpha in plane order, and rounded
 * once (to nearest even) to w_dtype.
 * W: [M][ldw] (row m starts at W + m*ldw elements), ldw >= K, 16-byte aligned
 *   with ldw*size a multiple of 16 bytes; columns past K are not written.
 * w_dtype must equal store->scale_dtype.  Validation and stream behaviour as
 * in bcq_gemv.
 */
bcq_status bcq_dequantize(const bcq_store *store, int32_t p, void *W, int32_t ldw,
                          bcq_dtype w_dtype, hipStream_t stream);

/*
 * Binary low-rank correction, added in place to a product's output:
 *     y[m] += sum_{r<R} alpha[r] * u[m][r] * (v[r] . x)
 * with u and v in {-1,+1} (BiLoCo summary, "core idea": every rank-one term
 * is a scale times two sign vectors, so v . x takes only additions and
 * subtractions).  z_r = alpha_r (v_r . x) is formed in fp32; y is read, the
 * correction added in fp32 and the sum rounded once (to nearest even).
 * u_signs: [M][ceil(R/32)] uint32, bit r mod 32 of word [m][r/32] set = +1
 *   (bits past R ignored), 4-byte aligned.
 * v_signs: [R][K/32] uint32, bit k mod 32 of word [r][k/32] set = +1, 4-byte
 *   aligned.  K must be a positive multiple of 32.
 * alpha: [R], x: [K], y: [M] (read and written), all of one dtype (BCQ_F16 or
 *   BCQ_F32); x 16-byte aligned, alpha and y element aligned.
 * z: device workspace of R floats, 4-byte aligned, clobbered (calls that may
 *   run at the same time need separate ones).
 * 1 <= R <= BCQ_LOWRANK_MAX_RANK, M >= 1.  Validation and stream behaviour as
 * in bcq_gemv: a rejected call enqueues nothing.
 */
bcq_status bcq_lowrank_correct(const uint32_t *u_signs, const uint32_t *v_signs,
                               const void *alpha, int32_t R, int32_t M, int32_t K, const void *x,
                               void *y, bcq_dtype dtype, float *z, hipStream_t stream);

/*
 * Batch-1 product with a binary low-rank correction, written (not added):
 *     y[m] = (W_hat_p x)[m] + sum_{r<R} lr_alpha[r] * u[m][r] * (v[r] . x)
 * with W_hat_p the store's reconstruction at precision p (as bcq_gemv) and
 * u, v, lr_alpha the terms of bcq_lowrank_correct.  Defined by: AnyBCQ paper
 * notes, "Method / key designs" (the product) and the BiLoCo summary, "core
 * idea" and its fused-operator section (the correction, computed as
 * z = lr_alpha * (V x) first and expanded by u into the product's output
 * before it is written back).
 * Two launches on `stream`: z_r = lr_alpha[r] (v_r . x) into z, then the
 * product.  When K <= 4096 and R <= BCQ_LOWRANK_FUSED_MAX_RANK the product's
 * kernel adds sum_r u[m][r] z_r to its fp32 row sums and rounds y once;
 * otherwise the product is written and a third launch adds the correction to
 * it (y rounded twice).
 * store, p, x, x_dtype, y, y_dtype: as in bcq_gemv.
 * u_signs [M][ceil(R/32)], v_signs [R][K/32], z (R floats, clobbered): as in
 * bcq_lowrank_correct; lr_alpha [R] in the store's scale dtype, element
 * aligned.  1 <= R <= BCQ_LOWRANK_MAX_RANK.  Validation and stream behaviour
 * as in bcq_gemv: a rejected call enqueues nothing.
 */
bcq_status bcq_gemv_lowrank(const bcq_store *store, int32_t p, const void *x, bcq_dtype x_dtype,
                            const uint32_t *u_signs, const uint32_t *v_signs,
                            const void *lr_alpha, int32_t R, void *y, bcq_dtype y_dtype, float *z,
                            hipStream_t stream);

/*
 * Offline quantizer: a weight matrix W [M][K] becomes P shared sign planes and
 * one scale and offset table per precision p = p_low..P, by AnyBCQ's
 * progressive precision expansion (AnyBCQ paper notes, "Method / key
 * designs": greedy start and alternating refinement -- a least-squares scale
 * fit, then a search for each weight's best code -- at the base precision;
 * then, per added plane, the earlier planes frozen, the new plane the sign of
 * the residual and every scale refit by least squares; "Training strategy":
 * asymmetric group-wise BCQ with g = 128).  Per (row, group of 128):
 *  1. greedy start: offset = group mean; for each of the p_low planes,
 *     plane = sign(residual) (sign(0) = +1), scale = mean |residual|, and the
 *     scaled plane leaves the residual;
 *  2. `iters` rounds of: least-squares fit of the p_low scales and the
 *     offset, then every weight takes the code (one sign per plane) whose
 *     level z + sum +-alpha_i is nearest (first code on a tie, code c giving
 *     plane i the sign +1 when bit i of c is set); then a last fit;
 *  3. for p = p_low..P-1: plane p+1 = sign(W - W_hat_p), earlier planes
 *     unchanged, then a least-squares fit of all p+1 scales and the offset.
 * Least squares solves the normal equations over the columns [planes, ones];
 * a plane linearly dependent on the ones column and the earlier kept planes
 * gets scale 0.  Sums over a group are pairwise (halving) sums in fp64 and
 * no multiply-add is fused, so every decision is taken on fully specified
 * values; the results are deterministic.
 * W: [M][ldw] (row m at W + m*ldw), ldw >= K, w_dtype BCQ_F16 or BCQ_F32,
 *   element aligned.  M >= 1, K a positive multiple of 128, 1 <= p_low <= P
 *   <= 4, 0 <= iters <= 1000.
 * signs: [P][M][K/32] uint32 in bcq_pack_planes' canonical input format
 *   (4-byte aligned); fully overwritten.
 * alpha: the tables of p = p_low..P one after another, table p being
 *   [p][M][K/128] and starting (p(p-1)/2 - p_low(p_low-1)/2) * M * (K/128)
 *   elements into the buffer; zero: [P - p_low + 1][M][K/128], the offsets of
 *   precision p at table p - p_low.  out_dtype BCQ_F16, BCQ_F32 or BCQ_F64,
 *   each value rounded once to nearest even from fp64; element aligned.
 * Validation and stream behaviour as in bcq_gemv: a rejected call enqueues
 * nothing.
 */
bcq_status bcq_quantize(const void *W, bcq_dtype w_dtype, int32_t M, int32_t K, int32_t ldw,
                        int32_t P, int32_t p_low, int32_t iters, uint32_t *signs, void *alpha,
                        void *zero, bcq_dtype out_dtype, hipStream_t stream);

/* Static text for a status code (never null). */
const char *bcq_status_string(bcq_status status);

#ifdef __cplusplus
}
#endif

#endif /* BCQ_H_ */
