// pack.hip -- canonical sign planes <-> packed device layout.
//
// Each plane stays one contiguous array so that precision p reads a prefix of
// the store (AnyBCQ paper notes, "key designs": a 3-bit product loads three
// planes, not four with one discarded).  Within a plane the 128 sign bits of
// one (row, group) are 16 contiguous bytes, and the 16 rows of a tile are
// adjacent for each group, so a wavefront that covers 16 rows x 4 groups
// reads 1 KiB of contiguous memory per load instruction.
//
// Within each 32-column word the bits are stored even columns first: packed
// bit b holds column 2b for b < 16 and column 2(b - 16) + 1 for b >= 16.  So
// bits b and b + 16 are the adjacent columns (2b, 2b + 1): one shift moves
// both to the two fp16 sign positions of a register, next to the natural fp16
// pair of activations they multiply (gemm_mfma.hip decodes weights this way).
#include "bcq_internal.h"

namespace bcq {
namespace {

constexpr int kPackThreads = 256;

__device__ __forceinline__ int packed_column(int b) { return b < 16 ? 2 * b : 2 * (b - 16) + 1; }

// canonical word (bit k = column k) -> packed word, and back
__device__ __forceinline__ uint32_t to_packed(uint32_t w) {
  uint32_t o = 0u;
#pragma unroll
  for (int b = 0; b < 32; ++b) o |= ((w >> packed_column(b)) & 1u) << b;
  return o;
}
__device__ __forceinline__ uint32_t from_packed(uint32_t w) {
  uint32_t o = 0u;
#pragma unroll
  for (int b = 0; b < 32; ++b) o |= ((w >> b) & 1u) << packed_column(b);
  return o;
}

__global__ __launch_bounds__(kPackThreads) void pack_kernel(const uint32_t *__restrict__ signs,
                                                            int P, int M, int K, int MT,
                                                            uint4 *__restrict__ packed) {
  const int G = K / kGroup;
  const size_t total = (size_t)P * MT * G * kTileRows;
  const size_t o = (size_t)blockIdx.x * kPackThreads + threadIdx.x;
  if (o >= total) return;
  const int r = (int)(o % kTileRows);
  const int j = (int)((o / kTileRows) % G);
  const int t = (int)((o / ((size_t)kTileRows * G)) % MT);
  const int i = (int)(o / ((size_t)kTileRows * G * MT));
  const int m = t * kTileRows + r;
  uint4 v = make_uint4(0u, 0u, 0u, 0u);  // padding rows hold clear bits
  if (m < M) {
    const uint32_t *src = signs + ((size_t)i * M + m) * (size_t)(K / 32) + (size_t)j * 4;
    v.x = to_packed(src[0]);
    v.y = to_packed(src[1]);
    v.z = to_packed(src[2]);
    v.w = to_packed(src[3]);
  }
  packed[o] = v;
}

__global__ __launch_bounds__(kPackThreads) void unpack_kernel(const uint4 *__restrict__ packed,
                                                              int P, int M, int K, int MT,
                                                              uint32_t *__restrict__ signs) {
  const int G = K / kGroup;
  const size_t total = (size_t)P * MT * G * kTileRows;
  const size_t o = (size_t)blockIdx.x * kPackThreads + threadIdx.x;
  if (o >= total) return;
  const int r = (int)(o % kTileRows);
  const int j = (int)((o / kTileRows) % G);
  const int t = (int)((o / ((size_t)kTileRows * G)) % MT);
  const int i = (int)(o / ((size_t)kTileRows * G * MT));
  const int m = t * kTileRows + r;
  if (m >= M) return;
  const uint4 v = packed[o];
  uint32_t *dst = signs + ((size_t)i * M + m) * (size_t)(K / 32) + (size_t)j * 4;
  dst[0] = from_packed(v.x);
  dst[1] = from_packed(v.y);
  dst[2] = from_packed(v.z);
  dst[3] = from_packed(v.w);
}

unsigned blocks_for(int P, int M, int K) {
  const size_t total = (size_t)P * row_tiles(M) * (K / kGroup) * kTileRows;
  return (unsigned)((total + kPackThreads - 1) / kPackThreads);
}

}  // namespace

hipError_t launch_pack(const uint32_t *signs, int P, int M, int K, uint32_t *packed,
                       hipStream_t s) {
  hipLaunchKernelGGL(pack_kernel, dim3(blocks_for(P, M, K)), dim3(kPackThreads), 0, s, signs,
                     P, M, K, row_tiles(M), reinterpret_cast<uint4 *>(packed));
  return hipGetLastError();
}

hipError_t launch_unpack(const uint32_t *packed, int P, int M, int K, uint32_t *signs,
                         hipStream_t s) {
  hipLaunchKernelGGL(unpack_kernel, dim3(blocks_for(P, M, K)), dim3(kPackThreads), 0, s,
                     reinterpret_cast<const uint4 *>(packed), P, M, K, row_tiles(M), signs);
  return hipGetLastError();
}

}  // namespace bcq
