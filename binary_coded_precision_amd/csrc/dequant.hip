// dequant.hip -- dense reconstruction W[m][k] = z + sum_{i<p} alpha_i s_i of a
// packed store (AnyBCQ paper notes, "Method / key designs": a weight is the
// offset plus each plane's sign times its scale), for large batches that go
// through a dense matrix product instead.
//
// One workgroup per (16-row tile, 128-column group).  The packed layout keeps
// that block's plane words together (16 rows x 16 bytes per plane), so the
// workgroup reads them once and no other workgroup -- on another XCD, with
// its own L2 -- touches them.  A thread owns one 16-byte chunk of one row
// (8 fp16 or 4 fp32 columns): it loads the chunk's plane word, scales and
// offset, forms each weight in fp32 as z, then + or - alpha_i plane by plane,
// rounds once and stores the chunk with a streaming (non-temporal) store, so
// a wavefront writes whole 256-byte row segments.  The + or - is made without
// a compare: bit 31 of the plane word shifted left by (31 - b), complemented
// and flipped by alpha's sign, becomes the sign of |alpha| (one v_bfi_b32).
// Within a packed word bit b holds column 2b for b < 16 and column
// 2(b - 16) + 1 for b >= 16 (pack.hip).
#include "bcq_internal.h"

namespace bcq {
namespace {

constexpr int kDqThreads = 256;

template <typename T>
struct Vec16;  // 16 bytes of T
template <>
struct Vec16<_Float16> {
  typedef _Float16 type __attribute__((ext_vector_type(8)));
  static constexpr int n = 8;
};
template <>
struct Vec16<float> {
  typedef float type __attribute__((ext_vector_type(4)));
  static constexpr int n = 4;
};

// bit 31 from s, bits 0..30 from m (an ALU instruction, no memory operand)
__device__ __forceinline__ uint32_t sign_insert(uint32_t s, uint32_t m) {
  uint32_t r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "s"(0x80000000u), "v"(s), "v"(m));
  return r;
}

template <typename T, int P>
__global__ __launch_bounds__(kDqThreads) void dequant_kernel(const uint32_t *__restrict__ bits,
                                                             const T *__restrict__ alpha,
                                                             const T *__restrict__ zero, int M,
                                                             int G, int MT, T *__restrict__ W,
                                                             int ldw) {
  typedef typename Vec16<T>::type V;
  constexpr int N = Vec16<T>::n;
  constexpr int CPG = kGroup / N;        // 16-byte chunks in a row of one group
  constexpr int RPP = kDqThreads / CPG;  // rows per pass: 16 (fp16) or 8 (fp32)
  // workgroup -> (tile t, group j), groups fastest
  const int j = (int)(blockIdx.x % (unsigned)G);
  const int t = (int)(blockIdx.x / (unsigned)G);
  const int cc = threadIdx.x % CPG;
  const int q = cc * N / 32, o = (cc * N) & 31;  // word of the group, first column in it
  const size_t plane_words = (size_t)MT * G * kTileRows * 4;
  const size_t MG = (size_t)M * G;
#pragma unroll
  for (int pass = 0; pass < kTileRows / RPP; ++pass) {
    const int r = pass * RPP + threadIdx.x / CPG;
    const int m = t * kTileRows + r;
    if (m >= M) break;
    const size_t widx = ((size_t)(t * G + j) * kTileRows + r) * 4 + q;
    uint32_t wx[P], am[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const uint32_t w = bits[i * plane_words + widx];
      const uint32_t ab = __float_as_uint((float)alpha[i * MG + (size_t)m * G + j]);
      // bit 31 of (wx << (31 - b)) is the sign the term of bit b takes
      wx[i] = ~w ^ (uint32_t)((int32_t)ab >> 31);
      am[i] = ab & 0x7fffffffu;
    }
    const float z = (float)zero[(size_t)m * G + j];
    V out;
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const int c = o + e;
      const int b = (c & 1) ? 16 + (c >> 1) : (c >> 1);
      float v = z;
#pragma unroll
      for (int i = 0; i < P; ++i) v += __uint_as_float(sign_insert(wx[i] << (31 - b), am[i]));
      out[e] = (T)v;
    }
    __builtin_nontemporal_store(out, reinterpret_cast<V *>(W + (size_t)m * ldw + j * kGroup + cc * N));
  }
}

template <typename T>
hipError_t dequant_launch(const uint32_t *bits, int M, int K, int p, const void *alpha,
                          const void *zero, void *W, int ldw, hipStream_t s) {
  const int G = K / kGroup;
  const int MT = row_tiles(M);
  const dim3 grid((unsigned)((size_t)MT * G)), block(kDqThreads);
  const T *a = static_cast<const T *>(alpha);
  const T *z = static_cast<const T *>(zero);
  T *w = static_cast<T *>(W);
  switch (p) {
    case 1: hipLaunchKernelGGL((dequant_kernel<T, 1>), grid, block, 0, s, bits, a, z, M, G, MT, w, ldw); break;
    case 2: hipLaunchKernelGGL((dequant_kernel<T, 2>), grid, block, 0, s, bits, a, z, M, G, MT, w, ldw); break;
    case 3: hipLaunchKernelGGL((dequant_kernel<T, 3>), grid, block, 0, s, bits, a, z, M, G, MT, w, ldw); break;
    default: hipLaunchKernelGGL((dequant_kernel<T, 4>), grid, block, 0, s, bits, a, z, M, G, MT, w, ldw); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const uint32_t *bits, int M, int K, int p, const void *alpha,
                          const void *zero, void *W, int ldw, bcq_dtype dt, hipStream_t s) {
  if (dt == BCQ_F16) return dequant_launch<_Float16>(bits, M, K, p, alpha, zero, W, ldw, s);
  return dequant_launch<float>(bits, M, K, p, alpha, zero, W, ldw, s);
}

}  // namespace bcq
