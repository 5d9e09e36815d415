// gemm_mfma.hip -- BCQ product for 16 or more requests at one precision:
// weights are dequantised tile by tile to fp16 and contracted on the matrix
// cores (v_mfma_f32_16x16x32_f16, fp32 accumulation).
//
// Why this path: past a few requests the sign-sum tables cost one add per
// request per table read, while a dequantised tile is built once and reused by
// every request; at that point the product is a dense contraction.  (The
// BiLoCo write-up's speed results make the same point for its +-1 correction:
// the add/subtract work grows with batch while the weight read stays flat, so
// larger batches belong on the tensor cores.)
//
// Tile and lane mapping.  A workgroup is 4 wavefronts; wavefront v owns the 16
// rows of packed tile 4*blockIdx.x + v.  blockIdx.y selects a slice of the
// K groups (split K, so that enough workgroups exist and each reads only its
// slice of X).  Per group the workgroup stages the requests' 128 activations in
// LDS (row stride padded to 272 B so the 16 rows read by one MFMA operand load
// hit distinct banks), each lane dequantises 8 weights of one row per 32-column
// step, and every 16-request tile reuses that operand.
//
// Dequantisation w = z + sum_i alpha_i * s_i is done in packed fp16: a 16-entry
// LDS table maps a nibble of sign bits to four +-1.0 values, and v_pk_fma_f16
// accumulates alpha_i * (+-1) from the smallest-scale plane to the largest, then
// adds z.  The operand is fp16 rather than bf16 because both MFMA operands
// must share one type and bf16 activations would lose the fp16 inputs' bits.
#include "bcq_internal.h"

namespace bcq {
namespace {

using half_t = _Float16;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kMfThreads = 256;
constexpr int kMfWaves = kMfThreads / 64;
constexpr int kXStride = kGroup * 2 + 16;  // bytes per staged request row

__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
__device__ __forceinline__ uint32_t as_u(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// Operands of one K group, double-buffered across the group loop.
template <int NT, int P>
struct MfOperands {
  uint4 x[NT];         // this thread's share of the staged activations
  uint4 bits[P];       // this lane's row: 128 sign bits per plane
  uint32_t alpha2[P];  // (alpha, alpha) as packed fp16
  uint32_t zero2;      // (z, z)
};

// P (the precision) is a template argument and the load phase has no branches:
// request rows past b, rows past M and tiles past MT read clamped in-range
// addresses whose values are never stored.
template <int NT, int P>
__global__ __launch_bounds__(kMfThreads) void gemm_mfma_kernel(
    const uint4 *__restrict__ bits, const half_t *__restrict__ alpha,
    const half_t *__restrict__ zero, const half_t *__restrict__ X, int ldx, int b,
    half_t *__restrict__ Y, int ldy, float *__restrict__ ws, int M, int G, int MT,
    int groups_per_slice) {
  using Ops = MfOperands<NT, P>;
  __shared__ __attribute__((aligned(16))) char xt[2][NT * 16 * kXStride];
  __shared__ __attribute__((aligned(16))) uint2 pm1[16];  // +-1.0 for the 4 bits of a nibble

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int kb = lane >> 4;
  const int t = blockIdx.x * kMfWaves + wave;
  const int t_safe = min(t, MT - 1);
  const int m_safe = min(t * kTileRows + r, M - 1);
  const int s = blockIdx.y;
  const int j0 = s * groups_per_slice;
  const int j1 = min(G, j0 + groups_per_slice);
  const size_t plane_stride = (size_t)MT * G * kTileRows;
  const uint4 *tbits = bits + (size_t)t_safe * G * kTileRows + r;
  const size_t MG = (size_t)M * G;

  if (tid < 16) {
    unsigned short h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = ((tid >> q) & 1) ? 0x3C00u : 0xBC00u;  // +1.0 / -1.0
    pm1[tid] = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
  }

  floatx4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto fetch = [&](int j_in, Ops &o) {
    const int j = min(j_in, j1 - 1);
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int c = tid + q * kMfThreads;  // 16-byte chunk: request c/16, columns 8*(c%16)..
      const int n = min(c >> 4, b - 1);
      o.x[q] = *reinterpret_cast<const uint4 *>(X + (size_t)n * ldx + (size_t)j * kGroup +
                                                (c & 15) * 8);
    }
#pragma unroll
    for (int i = 0; i < P; ++i) {
      o.bits[i] = tbits[i * plane_stride + (size_t)j * kTileRows];
      const uint32_t a =
          *reinterpret_cast<const unsigned short *>(alpha + i * MG + (size_t)m_safe * G + j);
      o.alpha2[i] = a | (a << 16);
    }
    const uint32_t zz = *reinterpret_cast<const unsigned short *>(zero + (size_t)m_safe * G + j);
    o.zero2 = zz | (zz << 16);
  };

  auto consume = [&](int buf, const Ops &o) {
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int c = tid + q * kMfThreads;
      *reinterpret_cast<uint4 *>(xt[buf] + (c >> 4) * kXStride + (c & 15) * 16) = o.x[q];
    }
    __syncthreads();
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      // dequantise 8 weights: row r, columns 128j + 32*s4 + 8*kb .. +7
      half2v w2[4] = {as_h2(0u), as_h2(0u), as_h2(0u), as_h2(0u)};
#pragma unroll
      for (int i = P - 1; i >= 0; --i) {
        const uint32_t word =
            s4 == 0 ? o.bits[i].x : (s4 == 1 ? o.bits[i].y : (s4 == 2 ? o.bits[i].z : o.bits[i].w));
        const uint32_t byte = (word >> (8 * kb)) & 0xFFu;
        const uint2 lo = pm1[byte & 15u];
        const uint2 hi = pm1[byte >> 4];
        const half2v a2 = as_h2(o.alpha2[i]);
        w2[0] = __builtin_elementwise_fma(a2, as_h2(lo.x), w2[0]);
        w2[1] = __builtin_elementwise_fma(a2, as_h2(lo.y), w2[1]);
        w2[2] = __builtin_elementwise_fma(a2, as_h2(hi.x), w2[2]);
        w2[3] = __builtin_elementwise_fma(a2, as_h2(hi.y), w2[3]);
      }
      const half2v zz = as_h2(o.zero2);
      half8 a;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const half2v v = w2[q] + zz;
        a[2 * q] = v[0];
        a[2 * q + 1] = v[1];
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const half8 bop = *reinterpret_cast<const half8 *>(
            xt[buf] + (nt * 16 + r) * kXStride + (32 * s4 + 8 * kb) * 2);
        acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bop, acc[nt], 0, 0, 0);
      }
    }
  };

  // ping-pong: group j+1 loads while group j computes; the staged x tile is
  // double-buffered in LDS, so one barrier per group suffices
  if (j0 < j1) {
    Ops A, B;
    fetch(j0, A);
    for (int j = j0; j < j1; j += 2) {
      fetch(j + 1, B);
      consume(0, A);
      if (j + 1 >= j1) break;  // uniform
      fetch(j + 2, A);
      consume(1, B);
    }
  }

  // D layout: lane holds rows 4*kb .. 4*kb+3 of the tile for request column r
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = nt * 16 + r;
    if (n >= b) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mm = t * kTileRows + 4 * kb + v;
      if (mm >= M) continue;
      if (ws == nullptr)
        Y[(size_t)n * ldy + mm] = (half_t)acc[nt][v];
      else
        ws[((size_t)s * b + n) * M + mm] = acc[nt][v];
    }
  }
}

// Sums the split-K partials in slice order and rounds once.
__global__ __launch_bounds__(256) void splitk_finalize_kernel(const float *__restrict__ ws,
                                                              int slices, int b, int M,
                                                              half_t *__restrict__ Y, int ldy) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)b * M) return;
  const int n = (int)(idx / M);
  const int mm = (int)(idx % M);
  float s = 0.f;
  for (int q = 0; q < slices; ++q) s += ws[((size_t)q * b + n) * M + mm];
  Y[(size_t)n * ldy + mm] = (half_t)s;
}

}  // namespace

// Number of K slices for a (M, K) problem: enough workgroups to cover the chip,
// with at least 4 groups per slice.
int mfma_slices(int M, int K) {
  const int G = K / kGroup;
  const int wgs = (row_tiles(M) + kMfWaves - 1) / kMfWaves;
  int s = (256 + wgs - 1) / wgs;
  s = s < 1 ? 1 : s;
  const int smax = G / 4 > 0 ? G / 4 : 1;
  return s > smax ? smax : s;
}

size_t mfma_workspace_bytes(int M, int K, int b) {
  const int s = mfma_slices(M, K);
  if (s <= 1) return 0;
  const int bb = b < 64 ? b : 64;
  return (size_t)s * bb * M * sizeof(float);
}

hipError_t launch_gemm_mfma(const uint32_t *bits, int M, int K, int p, const void *alpha,
                            const void *zero, const void *x, int ldx, int b, void *y, int ldy,
                            void *ws, hipStream_t s) {
  const int G = K / kGroup;
  const int MT = row_tiles(M);
  const int S = mfma_slices(M, K);
  const int gps = (G + S - 1) / S;
  const uint4 *b4 = reinterpret_cast<const uint4 *>(bits);
  const half_t *a = static_cast<const half_t *>(alpha);
  const half_t *z = static_cast<const half_t *>(zero);
  const half_t *X = static_cast<const half_t *>(x);
  half_t *Y = static_cast<half_t *>(y);
  float *w = S > 1 ? static_cast<float *>(ws) : nullptr;
  dim3 grid((MT + kMfWaves - 1) / kMfWaves, S), block(kMfThreads);
  const int NT = (b + 15) / 16;
#define BCQ_MF(NTV, PV)                                                                    \
  hipLaunchKernelGGL((gemm_mfma_kernel<NTV, PV>), grid, block, 0, s, b4, a, z, X, ldx, b, Y, \
                     ldy, w, M, G, MT, gps)
#define BCQ_MF_NT(NTV)              \
  switch (p) {                      \
    case 1: BCQ_MF(NTV, 1); break;  \
    case 2: BCQ_MF(NTV, 2); break;  \
    case 3: BCQ_MF(NTV, 3); break;  \
    default: BCQ_MF(NTV, 4); break; \
  }
  switch (NT) {
    case 1: BCQ_MF_NT(1) break;
    case 2: BCQ_MF_NT(2) break;
    case 3: BCQ_MF_NT(3) break;
    default: BCQ_MF_NT(4) break;
  }
#undef BCQ_MF_NT
#undef BCQ_MF
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S <= 1) return e;
  const size_t n = (size_t)b * M;
  hipLaunchKernelGGL(splitk_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     w, S, b, M, Y, ldy);
  return hipGetLastError();
}

}  // namespace bcq
