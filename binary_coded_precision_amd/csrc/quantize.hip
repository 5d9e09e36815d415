// quantize.hip -- AnyBCQ's offline progressive-precision quantizer on gfx950:
// a weight matrix W [M][K] becomes P shared sign planes plus one scale and
// offset table per precision p = p_low..P.
//
// Method (AnyBCQ paper notes, "Method / key designs", progressive precision
// expansion; "Training strategy": asymmetric BCQ, groups of 128, alternating
// refinement at initialisation), per (row, group) of 128 weights:
//  1. Greedy start at the base precision p_low: the offset is the group mean;
//     each plane is the sign of the residual (sign(0) = +1) and its scale the
//     mean absolute residual, which then leaves the residual.
//  2. `iters` rounds of alternating refinement: a least-squares fit of every
//     scale and the offset for the current planes, then the sign update --
//     every weight takes the code (one sign per plane) of its nearest level,
//     the first code on a tie (code c: plane i is +1 when bit i of c is set).
//     A last least-squares fit makes the base scales optimal for the planes.
//  3. Expansion to p + 1: earlier planes stay frozen, the new plane is the
//     sign of the residual, and all scales of precision p + 1 and its offset
//     are refit by least squares.
// Least squares solves the normal equations over the columns [planes,
// ones]; a plane that is linearly dependent on the ones column and the
// earlier kept planes (exact integer test on the Gram matrix) gets scale 0.
// The kept system is solved by Gaussian elimination without pivoting in
// index order (it is symmetric positive definite).
//
// Design for CDNA4.  One wavefront per (row, group): lane l holds columns l
// and l + 64 in fp64.  A plane is two 64-bit ballots (wave-uniform), so the
// Gram matrix of the columns is exact integer arithmetic on popcounts.  Every
// sum over the group is a pairwise sum -- the lane adds its two columns, then
// xor-butterfly shuffles over 32, 16, .., 1 lanes -- which gives every lane
// the same bits, so all lanes take identical decisions without a broadcast,
// and the decisions match any implementation that sums in the same pairwise
// order.  All floating-point arithmetic is fp64 with no contraction of a
// multiply and an add into one rounding (pragma below), so each sign update
// sees exactly rounded values.  The work is offline: a 4096x4096 matrix is
// 131072 independent wavefronts.
#pragma clang fp contract(off)

#include "bcq_internal.h"

namespace bcq {
namespace {

constexpr int kQWaves = 4;  // groups (wavefronts) per workgroup
constexpr int kQMax = BCQ_MAX_PLANES;

// Pairwise sum over the group: a = this lane's column l, b = its column l+64.
__device__ __forceinline__ double group_sum(double a, double b) {
  double v = a + b;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ double pm(bool pos, double a) { return pos ? a : -a; }

// Exact determinant test by fraction-free (Bareiss) elimination of an N x N
// integer matrix whose leading N-1 columns are linearly independent, so no
// pivot before the last is zero.  Entries are minors of a Gram matrix of
// +-1 vectors of length 128 (at most 128^4 before the last step), so every
// product fits int64.
template <int N>
__device__ __forceinline__ long long bareiss_last(long long (&A)[kQMax + 1][kQMax + 1]) {
  long long prev = 1;
#pragma unroll
  for (int k = 0; k < N - 1; ++k) {
#pragma unroll
    for (int i = k + 1; i < N; ++i)
#pragma unroll
      for (int j = k + 1; j < N; ++j) A[i][j] = (A[i][j] * A[k][k] - A[i][k] * A[k][j]) / prev;
    prev = A[k][k];
  }
  return A[N - 1][N - 1];
}

// Planes of one group: sign bits of columns 0..63 (lo) and 64..127 (hi).
struct Planes {
  uint64_t lo[kQMax], hi[kQMax];
};

// <b_a, b_b> for planes a, b: 128 - 2 * (number of columns where they differ).
__device__ __forceinline__ long long dot_planes(const Planes &B, int a, int b) {
  return 128 - 2 * (long long)(__popcll(B.lo[a] ^ B.lo[b]) + __popcll(B.hi[a] ^ B.hi[b]));
}
// <b_a, ones>.
__device__ __forceinline__ long long dot_ones(const Planes &B, int a) {
  return 2 * (long long)(__popcll(B.lo[a]) + __popcll(B.hi[a])) - 128;
}

// Least-squares scales alpha[0..NP-1] and offset z for the first NP planes.
// s0[i], s1[i]: this lane's sign of plane i at columns l and l+64.
template <int NP>
__device__ __forceinline__ void ls_fit(const Planes &B, const bool (&s0)[kQMax],
                                       const bool (&s1)[kQMax], double w0, double w1,
                                       double wsum, double (&alpha)[kQMax], double &z) {
  constexpr int n = NP + 1;  // columns: planes 0..NP-1, then ones
  long long Gi[n][n];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
#pragma unroll
    for (int j = 0; j < NP; ++j) Gi[i][j] = dot_planes(B, i, j);
    Gi[i][NP] = Gi[NP][i] = dot_ones(B, i);
  }
  Gi[NP][NP] = 128;
  // kept columns: the ones column, then each plane that is independent of the
  // ones column and the planes kept before it
  bool keep[n];
  keep[NP] = true;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    // matrix on [ones, plane 0..i], planes not kept replaced by identity
    // rows and columns (which leave the determinant unchanged)
    long long A[kQMax + 1][kQMax + 1];
#pragma unroll
    for (int r = 0; r < i + 2; ++r)
#pragma unroll
      for (int c = 0; c < i + 2; ++c) {
        const int cr = r == 0 ? NP : r - 1, cc = c == 0 ? NP : c - 1;
        const bool ar = r == 0 || r == i + 1 || keep[r - 1];
        const bool ac = c == 0 || c == i + 1 || keep[c - 1];
        A[r][c] = (ar && ac) ? Gi[cr][cc] : (r == c ? 1 : 0);
      }
    long long det;
    switch (i) {
      case 0: det = bareiss_last<2>(A); break;
      case 1: det = bareiss_last<3>(A); break;
      case 2: det = bareiss_last<4>(A); break;
      default: det = bareiss_last<5>(A); break;
    }
    keep[i] = det != 0;
  }
  // normal equations in fp64; dropped columns: identity row and column, zero
  // right-hand side
  double G[n][n], c[n];
#pragma unroll
  for (int i = 0; i < n; ++i) {
#pragma unroll
    for (int j = 0; j < n; ++j)
      G[i][j] = (keep[i] && keep[j]) ? (double)Gi[i][j] : (i == j ? 1.0 : 0.0);
  }
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const double ci = group_sum(pm(s0[i], w0), pm(s1[i], w1));
    c[i] = keep[i] ? ci : 0.0;
  }
  c[NP] = wsum;
#pragma unroll
  for (int k = 0; k < n; ++k) {
#pragma unroll
    for (int i = k + 1; i < n; ++i) {
      const double f = G[i][k] / G[k][k];
#pragma unroll
      for (int j = k; j < n; ++j) G[i][j] = G[i][j] - f * G[k][j];
      c[i] = c[i] - f * c[k];
    }
  }
  double th[n];
#pragma unroll
  for (int k = n - 1; k >= 0; --k) {
    double s = c[k];
#pragma unroll
    for (int j = k + 1; j < n; ++j) s = s - G[k][j] * th[j];
    th[k] = s / G[k][k];
  }
#pragma unroll
  for (int i = 0; i < kQMax; ++i) alpha[i] = i < NP ? th[i] : 0.0;
  z = th[NP];
}

__device__ __forceinline__ void ls_fit_p(int p, const Planes &B, const bool (&s0)[kQMax],
                                         const bool (&s1)[kQMax], double w0, double w1,
                                         double wsum, double (&alpha)[kQMax], double &z) {
  switch (p) {
    case 1: ls_fit<1>(B, s0, s1, w0, w1, wsum, alpha, z); break;
    case 2: ls_fit<2>(B, s0, s1, w0, w1, wsum, alpha, z); break;
    case 3: ls_fit<3>(B, s0, s1, w0, w1, wsum, alpha, z); break;
    default: ls_fit<4>(B, s0, s1, w0, w1, wsum, alpha, z); break;
  }
}

// Level of a code: z + (+-alpha_0) + (+-alpha_1) + ... in plane order.
__device__ __forceinline__ double level(int p, const bool (&s)[kQMax], const double (&alpha)[kQMax],
                                        double z) {
  double lv = z;
#pragma unroll
  for (int i = 0; i < kQMax; ++i)
    if (i < p) lv = lv + pm(s[i], alpha[i]);
  return lv;
}

// Nearest of the 2^p levels to w; ties to the first code.  Writes its signs.
__device__ __forceinline__ void nearest(int p, double w, const double (&alpha)[kQMax], double z,
                                        bool (&s)[kQMax]) {
  double best = __builtin_huge_val();
  int best_code = 0;
  for (int code = 0; code < (1 << p); ++code) {
    double lv = z;
#pragma unroll
    for (int i = 0; i < kQMax; ++i)
      if (i < p) lv = lv + pm((code >> i) & 1, alpha[i]);
    const double d = __builtin_fabs(w - lv);
    if (d < best) {
      best = d;
      best_code = code;
    }
  }
#pragma unroll
  for (int i = 0; i < kQMax; ++i)
    if (i < p) s[i] = (best_code >> i) & 1;
}

// fp64 -> fp16 bits, rounded once to nearest even (no detour through fp32,
// whose own rounding could move a value onto an fp16 halfway point).
__device__ __forceinline__ uint16_t f64_to_f16_bits(double d) {
  const uint64_t u = __builtin_bit_cast(uint64_t, d);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000u);
  const int ex = (int)((u >> 52) & 0x7FF);
  const uint64_t man = u & 0xFFFFFFFFFFFFFull;
  if (ex == 0x7FF) return sign | (man ? 0x7E00 : 0x7C00);
  uint64_t sig = ex ? (man | (1ull << 52)) : man;  // value = sig * 2^(e - 52)
  int e = ex ? ex - 1023 : -1022;
  if (e >= -14) {  // normal fp16 range (or overflow)
    uint64_t q = sig >> 42;
    const uint64_t rem = sig & ((1ull << 42) - 1), half = 1ull << 41;
    if (rem > half || (rem == half && (q & 1))) ++q;
    if (q == (1ull << 11)) {
      q >>= 1;
      ++e;
    }
    if (e > 15) return sign | 0x7C00;
    return sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q & 0x3FF);
  }
  // subnormal fp16: units of 2^-24; value = sig * 2^(e - 28) units
  const int sh = 28 - e;  // > 42
  if (sh > 53) return sign;  // below half a unit
  uint64_t q = sig >> sh;
  const uint64_t rem = sig & ((1ull << sh) - 1), half = 1ull << (sh - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  return sign | (uint16_t)q;  // q == 1024 is the smallest normal, encoded alike
}

template <typename T>
__device__ __forceinline__ double load_w(const T *p) {
  if constexpr (sizeof(T) == 2)
    return (double)(float)*reinterpret_cast<const _Float16 *>(p);
  else
    return (double)*p;
}

__device__ __forceinline__ void store_scale(void *out, size_t idx, double v, int out_dt) {
  if (out_dt == BCQ_F16)
    static_cast<uint16_t *>(out)[idx] = f64_to_f16_bits(v);
  else if (out_dt == BCQ_F32)
    static_cast<float *>(out)[idx] = (float)v;
  else
    static_cast<double *>(out)[idx] = v;
}

// Grid: ceil(M*G / kQWaves) workgroups of kQWaves wavefronts; wavefront q of
// workgroup x takes group (x*kQWaves + q) of the row-major [M][G] list.  A
// wavefront past the end returns as a whole (its index is wave-uniform).
template <typename T, int P>
__global__ __launch_bounds__(64 * kQWaves) void quantize_kernel(
    const T *__restrict__ W, int ldw, int M, int G, int p_low, int iters,
    uint32_t *__restrict__ signs, void *__restrict__ alpha_out, void *__restrict__ zero_out,
    int out_dt) {
  const int lane = threadIdx.x & 63;
  const long long prob = (long long)blockIdx.x * kQWaves + (threadIdx.x >> 6);
  if (prob >= (long long)M * G) return;
  const int m = (int)(prob / G), j = (int)(prob % G);
  const T *row = W + (size_t)m * ldw + (size_t)j * kGroup;
  const double w0 = load_w(row + lane), w1 = load_w(row + 64 + lane);
  const double wsum = group_sum(w0, w1);

  Planes B;
  bool s0[kQMax], s1[kQMax];
#pragma unroll
  for (int i = 0; i < kQMax; ++i) {
    B.lo[i] = B.hi[i] = 0;
    s0[i] = s1[i] = false;
  }
  double alpha[kQMax] = {0.0, 0.0, 0.0, 0.0};
  double z = wsum / 128.0;

  // 1. greedy start at p_low
  {
    double r0 = w0 - z, r1 = w1 - z;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      if (i < p_low) {
        s0[i] = r0 >= 0.0;
        s1[i] = r1 >= 0.0;
        const double a = group_sum(__builtin_fabs(r0), __builtin_fabs(r1)) / 128.0;
        r0 = r0 - pm(s0[i], a);
        r1 = r1 - pm(s1[i], a);
        alpha[i] = a;
      }
    }
  }
  auto ballots = [&](int p) {
#pragma unroll
    for (int i = 0; i < P; ++i)
      if (i < p) {
        B.lo[i] = __ballot(s0[i]);
        B.hi[i] = __ballot(s1[i]);
      }
  };
  ballots(p_low);

  // 2. alternating refinement at p_low, then the final fit
  for (int it = 0; it < iters; ++it) {
    ls_fit_p(p_low, B, s0, s1, w0, w1, wsum, alpha, z);
    nearest(p_low, w0, alpha, z, s0);
    nearest(p_low, w1, alpha, z, s1);
    ballots(p_low);
  }
  ls_fit_p(p_low, B, s0, s1, w0, w1, wsum, alpha, z);

  // per-precision tables: precision p's [p][M][G] scales start after those of
  // p_low..p-1; its [M][G] offsets are table p - p_low of zero_out
  const size_t MG = (size_t)M * G;
  auto emit = [&](int p) {
    if (lane < kQMax + 1) {
      const size_t base = (size_t)(p * (p - 1) / 2 - p_low * (p_low - 1) / 2) * MG;
      if (lane < p) {
        double a = 0.0;
#pragma unroll
        for (int i = 0; i < kQMax; ++i)
          if (i == lane) a = alpha[i];
        store_scale(alpha_out, base + (size_t)lane * MG + prob, a, out_dt);
      } else if (lane == kQMax) {
        store_scale(zero_out, (size_t)(p - p_low) * MG + prob, z, out_dt);
      }
    }
  };
  emit(p_low);

  // 3. expansion: freeze the planes, add sign(residual), refit every scale
#pragma unroll
  for (int p = 1; p < P; ++p) {
    if (p >= p_low) {
      const double r0 = w0 - level(p, s0, alpha, z), r1 = w1 - level(p, s1, alpha, z);
      s0[p] = r0 >= 0.0;
      s1[p] = r1 >= 0.0;
      B.lo[p] = __ballot(s0[p]);
      B.hi[p] = __ballot(s1[p]);
      ls_fit_p(p + 1, B, s0, s1, w0, w1, wsum, alpha, z);
      emit(p + 1);
    }
  }

  // canonical sign words: plane i, row m, words 4j..4j+3 = columns 0..31,
  // 32..63, 64..95, 96..127 of the group; lanes 0..3 write one word each
  if (lane < 4) {
    const size_t K32 = (size_t)G * 4;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const uint64_t v = lane < 2 ? B.lo[i] : B.hi[i];
      const uint32_t word = (uint32_t)(lane & 1 ? v >> 32 : v);
      signs[((size_t)i * M + m) * K32 + (size_t)j * 4 + lane] = word;
    }
  }
}

template <typename T>
hipError_t launch_q(const T *W, int ldw, int M, int K, int P, int p_low, int iters,
                    uint32_t *signs, void *alpha, void *zero, int out_dt, hipStream_t s) {
  const int G = K / kGroup;
  const long long n = (long long)M * G;
  const dim3 grid((unsigned)((n + kQWaves - 1) / kQWaves)), block(64 * kQWaves);
#define BCQ_Q(PV)                                                                                \
  hipLaunchKernelGGL((quantize_kernel<T, PV>), grid, block, 0, s, W, ldw, M, G, p_low, iters, \
                     signs, alpha, zero, out_dt)
  switch (P) {
    case 1: BCQ_Q(1); break;
    case 2: BCQ_Q(2); break;
    case 3: BCQ_Q(3); break;
    default: BCQ_Q(4); break;
  }
#undef BCQ_Q
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const void *W, bcq_dtype w_dt, int ldw, int M, int K, int P,
                           int p_low, int iters, uint32_t *signs, void *alpha, void *zero,
                           bcq_dtype out_dt, hipStream_t s) {
  if (w_dt == BCQ_F16)
    return launch_q(static_cast<const _Float16 *>(W), ldw, M, K, P, p_low, iters, signs, alpha,
                    zero, (int)out_dt, s);
  return launch_q(static_cast<const float *>(W), ldw, M, K, P, p_low, iters, signs, alpha, zero,
                  (int)out_dt, s);
}

}  // namespace bcq
