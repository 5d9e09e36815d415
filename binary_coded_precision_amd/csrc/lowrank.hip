// lowrank.hip -- binary low-rank correction y += sum_r alpha_r u_r (v_r . x).
//
// Each rank-one term is a scale times two {-1,+1} vectors, so v . x takes only
// additions and subtractions (BiLoCo summary, "core idea").  Two launches:
//  * z_r = alpha_r (v_r . x): one workgroup per rank; each thread adds or
//    subtracts whole 32-column words of x in fp32 by the sign bits (the word's
//    activations loaded 16 bytes at a time), and the workgroup sums the
//    threads in a fixed order (lane moves within a wavefront, LDS across
//    wavefronts).
//  * y_m += sum_r u_mr z_r: z is turned into 16-entry tables of sign
//    combinations over 4 consecutive ranks in LDS (the same primitive as the
//    batch-1 product's activation tables), and each row looks up the nibbles
//    of its u bits.  Four lanes share a row, taking every fourth chunk of
//    ranks; their sums meet by lane moves.  y is read, added to in fp32 and
//    rounded once.
#include "bcq_internal.h"

namespace bcq {
namespace {

constexpr int kLrThreads = 256;        // rank workgroups
constexpr int kLrExpandThreads = 64;   // row workgroups: 16 rows, 4 lanes each
constexpr int kLrRowsPerBlock = kLrExpandThreads / 4;

template <typename T>
__device__ __forceinline__ float lr_load(const T *p, int i) {
  return (float)p[i];
}

// 32 consecutive elements of x as fp32, loaded as 16-byte pieces (x is 16-byte
// aligned, so every 32-element word of it is)
template <typename T>
__device__ __forceinline__ void lr_load32(const T *p, float (&f)[32]);
template <>
__device__ __forceinline__ void lr_load32<_Float16>(const _Float16 *p, float (&f)[32]) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const h8 *q = reinterpret_cast<const h8 *>(p);
  h8 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = q[i];
#pragma unroll
  for (int i = 0; i < 32; ++i) f[i] = (float)v[i / 8][i % 8];
}
template <>
__device__ __forceinline__ void lr_load32<float>(const float *p, float (&f)[32]) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 *q = reinterpret_cast<const f4 *>(p);
  f4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = q[i];
#pragma unroll
  for (int i = 0; i < 32; ++i) f[i] = v[i / 4][i % 4];
}

// one workgroup per rank: thread t takes the 32-column words t, t + 256, ...
// of v_r (one sign word and 32 activations, all requested before use)
template <typename T>
__global__ __launch_bounds__(kLrThreads) void lowrank_z_kernel(const uint32_t *__restrict__ v,
                                                               int K, const T *__restrict__ x,
                                                               const T *__restrict__ alpha,
                                                               float *__restrict__ z) {
  __shared__ float wsum[kLrThreads / 64];
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int nw = K / 32;
  const uint32_t *vr = v + (size_t)r * nw;
  float s = 0.f;
  for (int w = tid; w < nw; w += kLrThreads) {
    const uint32_t bits = vr[w];
    float f[32];
    lr_load32(x + (size_t)w * 32, f);
#pragma unroll
    for (int j = 0; j < 32; ++j) s += (bits >> j) & 1u ? f[j] : -f[j];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kLrThreads / 64; ++w) t += wsum[w];
    z[r] = lr_load(alpha, r) * t;
  }
}

template <typename T>
__global__ __launch_bounds__(kLrExpandThreads) void lowrank_expand_kernel(
    const uint32_t *__restrict__ u, int R, int M, const float *__restrict__ z, T *__restrict__ y) {
  // tables T_c[e] = sum_{t<4} (bit t of e ? +z : -z)_{4c+t}, ranks past R as 0;
  // ceil(R/4) x 16 floats of dynamic LDS
  extern __shared__ float tab_mem[];
  float(*tab)[16] = reinterpret_cast<float(*)[16]>(tab_mem);
  const int tid = threadIdx.x;
  const int nc = (R + 3) / 4;
  for (int c = tid; c < nc; c += kLrExpandThreads) {
    float f[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) f[t] = 4 * c + t < R ? z[4 * c + t] : 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) s += (e >> t) & 1 ? f[t] : -f[t];
      tab[c][e] = s;
    }
  }
  __syncthreads();
  const int q = tid & 3;
  const int m = min((int)blockIdx.x * kLrRowsPerBlock + (tid >> 2), M - 1);
  const int wu = (R + 31) / 32;
  const uint32_t *um = u + (size_t)m * wu;
  float s = 0.f;
  for (int c = q; c < nc; c += 4) s += tab[c][(um[c >> 3] >> (4 * (c & 7))) & 15u];
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  const int row = (int)blockIdx.x * kLrRowsPerBlock + (tid >> 2);
  if (q == 0 && row < M) y[row] = (T)((float)y[row] + s);
}

template <typename T>
hipError_t lowrank_z_launch(const uint32_t *v, const void *alpha, int R, int K, const void *x,
                            float *z, hipStream_t s) {
  hipLaunchKernelGGL(lowrank_z_kernel<T>, dim3(R), dim3(kLrThreads), 0, s, v, K,
                     static_cast<const T *>(x), static_cast<const T *>(alpha), z);
  return hipGetLastError();
}

template <typename T>
hipError_t lowrank_expand_launch(const uint32_t *u, int R, int M, const float *z, void *y,
                                 hipStream_t s) {
  const size_t lds = (size_t)((R + 3) / 4) * 16 * sizeof(float);  // <= 64 KB
  hipLaunchKernelGGL(lowrank_expand_kernel<T>, dim3((M + kLrRowsPerBlock - 1) / kLrRowsPerBlock),
                     dim3(kLrExpandThreads), lds, s, u, R, M, z, static_cast<T *>(y));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lowrank_z(const uint32_t *v, const void *alpha, int R, int K, const void *x,
                            float *z, bcq_dtype dt, hipStream_t s) {
  if (dt == BCQ_F16) return lowrank_z_launch<_Float16>(v, alpha, R, K, x, z, s);
  return lowrank_z_launch<float>(v, alpha, R, K, x, z, s);
}

hipError_t launch_lowrank_expand(const uint32_t *u, int R, int M, const float *z, void *y,
                                 bcq_dtype dt, hipStream_t s) {
  if (dt == BCQ_F16) return lowrank_expand_launch<_Float16>(u, R, M, z, y, s);
  return lowrank_expand_launch<float>(u, R, M, z, y, s);
}

hipError_t launch_lowrank(const uint32_t *u, const uint32_t *v, const void *alpha, int R, int M,
                          int K, const void *x, void *y, bcq_dtype dt, float *z, hipStream_t s) {
  hipError_t e = launch_lowrank_z(v, alpha, R, K, x, z, dt, s);
  if (e != hipSuccess) return e;
  return launch_lowrank_expand(u, R, M, z, y, dt, s);
}

}  // namespace bcq
