// probe.hip -- measurement kernels for the benchmark's floor row, built into
// libbcq_probe.so (not part of the BCQ library or its ABI): an empty launch,
// and a plain streaming read of n 16-byte blocks with every lane keeping
// several loads in flight.  They give the launch overhead and the cold-read
// time of one launch over a given byte count, the floor any single-launch
// kernel that must read those bytes sits on.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

namespace {

__global__ void empty_kernel() {}

// Each thread reads U blocks, tid + k * 256 (k < U) of its workgroup's span of
// 256 * U blocks, issuing every load before using any (coalesced: 4 KB per
// wavefront-instruction set), and folds them into one word; lane 0 of each
// workgroup writes its word only when it is a value no input makes, so the
// loads cannot be removed and the store never happens in practice.
template <int U>
__global__ __launch_bounds__(256) void read_kernel(const u32x4 *__restrict__ src, size_t n,
                                                   uint32_t *__restrict__ sink) {
  const size_t base = (size_t)blockIdx.x * 256 * U + threadIdx.x;
  u32x4 v[U];
#pragma unroll
  for (int k = 0; k < U; ++k) {
    const size_t i = base + (size_t)k * 256;
    v[k] = i < n ? src[i] : u32x4{0, 0, 0, 0};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int k = 0; k < U; ++k) acc += v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  if (acc == 0x9E3779B9u && threadIdx.x == 0) sink[blockIdx.x] = acc;
}

}  // namespace

extern "C" {

// Launch an empty kernel (one workgroup of 64 lanes) on stream.
int bcq_probe_empty(hipStream_t stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

// Read nbytes (a multiple of 16) from the 16-byte aligned device buffer src,
// each lane loading `per_lane` (1, 2, 4, 8 or 16) blocks of 16 bytes at once;
// sink holds one word per workgroup (ceil(nbytes / (4096 * per_lane))),
// written only in the never-taken case above.
int bcq_probe_read(const void *src, size_t nbytes, int per_lane, uint32_t *sink,
                   hipStream_t stream) {
  if (src == nullptr || sink == nullptr || nbytes % 16 != 0 || ((uintptr_t)src % 16) != 0)
    return -1;
  const size_t n = nbytes / 16;
  const u32x4 *s4 = static_cast<const u32x4 *>(src);
  const size_t span = (size_t)256 * per_lane;
  const dim3 grid((unsigned)((n + span - 1) / span)), block(256);
  switch (per_lane) {
    case 1: hipLaunchKernelGGL(read_kernel<1>, grid, block, 0, stream, s4, n, sink); break;
    case 2: hipLaunchKernelGGL(read_kernel<2>, grid, block, 0, stream, s4, n, sink); break;
    case 4: hipLaunchKernelGGL(read_kernel<4>, grid, block, 0, stream, s4, n, sink); break;
    case 8: hipLaunchKernelGGL(read_kernel<8>, grid, block, 0, stream, s4, n, sink); break;
    case 16: hipLaunchKernelGGL(read_kernel<16>, grid, block, 0, stream, s4, n, sink); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
