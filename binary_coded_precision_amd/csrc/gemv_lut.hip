// gemv_lut.hip -- BCQ products for batch 1 and for small batches (2..8 requests
// per launch) on the vector ALUs, with sign-combination tables in LDS.
//
// Method (AnyBCQ paper notes, "Method / key designs", direct bit-plane kernel):
// each plane is consumed on its own; because plane entries are -1 or +1 the
// plane product is additions and subtractions of activations; common partial
// results are cached LUT-GEMM style; each plane's partial sum is scaled by its
// factor and accumulated, and the output is written after the p-th plane.
//
// Design for CDNA4 (gfx950):
//  * Tables.  For every 4-column chunk c of x the workgroup builds the 16 sums
//    T_c[e] = sum_t (bit t of e ? +x_{4c+t} : -x_{4c+t}) in fp32 in LDS.  One
//    table read then replaces four signed adds: the 4 sign bits of one row in
//    one plane are the table index.  (A 16-entry table per 4 columns keeps the
//    build at 4 entries per column, cheap enough to repeat in every
//    workgroup; 256-entry byte tables would cost 32 entries per column.)
//  * Scales fuse at the group boundary: acc += alpha_i * P_i after the 32
//    lookups of a group, and acc += z * S_j with S_j the group's activation sum
//    (asymmetric BCQ offset, AnyBCQ paper notes, "Training strategy").
//  * Lane mapping.  A workgroup owns a tile of 16 rows and all of K.  Lane
//    (r, ks) of the 256 handles row r and one group per window of 16 groups, so
//    a wavefront (16 rows x 4 groups) loads 1 KiB of contiguous packed bits per
//    plane and per window (see pack.hip).  Every load of the workgroup is
//    issued before the first table is built, so a workgroup keeps up to
//    p * 16 B * windows per lane in flight.
//  * LDS banks.  Table c sits at 80-byte stride (16 entries + 16 B pad) so that
//    the 16-byte writes of 16 consecutive chunks cover distinct banks, and
//    groups sit at a stride that rotates the bank set by 16 so the four groups
//    read by one wavefront use disjoint banks.
//  * The reduction over the 16 K-sub lanes of a row is a fixed-order shuffle
//    + LDS sum, so results are deterministic.
#include "bcq_internal.h"

namespace bcq {
namespace {

using half_t = _Float16;

constexpr int kChunksPerGroup = kGroup / 4;  // 32 four-column chunks per group
constexpr int kEntries = 16;                 // table entries per chunk

// ---------------------------------------------------------------- activations

template <typename T>
struct Act;

template <>
struct Act<float> {
  using raw = float4;  // the 4 activations of one chunk
  static __device__ __forceinline__ raw load(const float *p) {
    return *reinterpret_cast<const float4 *>(p);
  }
  static __device__ __forceinline__ raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  static __device__ __forceinline__ void cvt(const raw &v, float (&f)[4]) {
    f[0] = v.x;
    f[1] = v.y;
    f[2] = v.z;
    f[3] = v.w;
  }
};

template <>
struct Act<half_t> {
  using raw = uint2;
  static __device__ __forceinline__ raw load(const half_t *p) {
    return *reinterpret_cast<const uint2 *>(p);
  }
  static __device__ __forceinline__ raw zero() { return make_uint2(0u, 0u); }
  static __device__ __forceinline__ void cvt(const raw &v, float (&f)[4]) {
    f[0] = (float)__builtin_bit_cast(half_t, (unsigned short)(v.x & 0xFFFFu));
    f[1] = (float)__builtin_bit_cast(half_t, (unsigned short)(v.x >> 16));
    f[2] = (float)__builtin_bit_cast(half_t, (unsigned short)(v.y & 0xFFFFu));
    f[3] = (float)__builtin_bit_cast(half_t, (unsigned short)(v.y >> 16));
  }
};

// The 16 signed sums of one chunk, entry e at float index e (bit t of e selects
// +x_t).  lo(e & 3) is -A, D, -D, A and hi(e >> 2) is -C, E, -E, C.
__device__ __forceinline__ void chunk_entries(const float (&f)[4], float4 (&v)[4]) {
  const float A = f[0] + f[1], D = f[0] - f[1];
  const float C = f[2] + f[3], E = f[2] - f[3];
  v[0] = make_float4(-A - C, D - C, -D - C, A - C);
  v[1] = make_float4(-A + E, D + E, -D + E, A + E);
  v[2] = make_float4(-A - E, D - E, -D - E, A - E);
  v[3] = make_float4(-A + C, D + C, -D + C, A + C);
}

__device__ __forceinline__ float comp(const float4 &v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// LDS addressing.  Table addresses are 32-bit LDS byte offsets: a lane's table
// base plus a byte offset that already sits in one byte of a register.  The
// add uses an SDWA byte select (one VALU op per lookup); without it the
// compiler emits shift + mask + add.  The chunk's constant offset goes into
// the ds_read immediate.
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) const float lds_float;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) const f32x2 lds_float2;
typedef __attribute__((address_space(3))) const f32x4 lds_float4;

__device__ __forceinline__ uint32_t lds_addr(const char *p) {
  return (uint32_t)(size_t)(lds_char *)p;
}

template <int B>
__device__ __forceinline__ uint32_t add_byte(uint32_t base, uint32_t v);
#define BCQ_ADD_BYTE(B)                                                                   \
  template <>                                                                             \
  __device__ __forceinline__ uint32_t add_byte<B>(uint32_t base, uint32_t v) {            \
    uint32_t r;                                                                           \
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD "   \
        "src1_sel:BYTE_" #B                                                               \
        : "=v"(r)                                                                         \
        : "v"(base), "v"(v));                                                             \
    return r;                                                                             \
  }
BCQ_ADD_BYTE(0)
BCQ_ADD_BYTE(1)
BCQ_ADD_BYTE(2)
BCQ_ADD_BYTE(3)
#undef BCQ_ADD_BYTE

template <int B>
__device__ __forceinline__ lds_float *lds_at(uint32_t base, uint32_t v) {
  return (lds_float *)(size_t)add_byte<B>(base, v);
}

// ---------------------------------------------------------------- batch 1

constexpr int kG1Threads = 256;
constexpr int kG1Ksub = 16;                                   // groups per window
constexpr int kG1ChunkStride = 80;                            // bytes
constexpr int kG1GroupStride = kChunksPerGroup * kG1ChunkStride + 64;  // 2624
constexpr int kG1WindowBytes = kG1Ksub * kG1GroupStride;      // 41984
constexpr int kG1WindowChunks = kG1Ksub * kChunksPerGroup;    // 512

// Sum over the 32 chunks of one group of T_c[nibble c of the row's 128 bits].
// base is the LDS byte offset of the group's first table.
__device__ __forceinline__ float g1_plane_sum(const uint4 bw, uint32_t base) {
  constexpr int S = kG1ChunkStride / 4;  // chunk stride in floats
  const uint32_t wd[4] = {bw.x, bw.y, bw.z, bw.w};
  float s[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    // nibble n times 4 (the entry's byte offset), one per byte: even n, then odd n
    const uint32_t ev = (wd[q] << 2) & 0x3C3C3C3Cu;
    const uint32_t od = (wd[q] >> 2) & 0x3C3C3C3Cu;
    const int c = q * 8;
    const float t0 = lds_at<0>(base, ev)[(c + 0) * S] + lds_at<0>(base, od)[(c + 1) * S];
    const float t1 = lds_at<1>(base, ev)[(c + 2) * S] + lds_at<1>(base, od)[(c + 3) * S];
    const float t2 = lds_at<2>(base, ev)[(c + 4) * S] + lds_at<2>(base, od)[(c + 5) * S];
    const float t3 = lds_at<3>(base, ev)[(c + 6) * S] + lds_at<3>(base, od)[(c + 7) * S];
    if (q == 0) {
      s[0] = t0;
      s[1] = t1;
      s[2] = t2;
      s[3] = t3;
    } else {
      s[0] += t0;
      s[1] += t1;
      s[2] += t2;
      s[3] += t3;
    }
  }
  return (s[0] + s[1]) + (s[2] + s[3]);
}

template <typename T, int WMAX>
__global__ __launch_bounds__(kG1Threads) void gemv_lut_kernel(
    const uint4 *__restrict__ bits, const T *__restrict__ alpha, const T *__restrict__ zero,
    const T *__restrict__ x, T *__restrict__ y, int M, int G, int MT, int p) {
  __shared__ __attribute__((aligned(16))) char lut[kG1WindowBytes];
  __shared__ float gsum[kG1Ksub];
  __shared__ float part[kG1Threads / 64][kTileRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int ks = wave * 4 + (lane >> 4);
  const int tile = blockIdx.x;
  const int m = tile * kTileRows + r;
  const bool row_ok = m < M;
  const int nwin = (G + kG1Ksub - 1) / kG1Ksub;
  const size_t plane_stride = (size_t)MT * G * kTileRows;  // in uint4
  const uint4 *tbits = bits + (size_t)tile * G * kTileRows + r;
  const size_t MG = (size_t)M * G;

  float acc = 0.f;

  for (int w0 = 0; w0 < nwin; w0 += WMAX) {
    // ---- issue every load of this batch of windows: x for the tables first,
    // then per window the sign words, scales and offsets
    typename Act<T>::raw xr[WMAX][2];
    uint4 bw[WMAX][BCQ_MAX_PLANES];
    T al[WMAX][BCQ_MAX_PLANES];
    T zz[WMAX];
#pragma unroll
    for (int u = 0; u < WMAX; ++u) {
      const int w = w0 + u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = tid + h * kG1Threads;
        const int j = w * kG1Ksub + c / kChunksPerGroup;
        xr[u][h] = (w < nwin && j < G)
                       ? Act<T>::load(x + ((size_t)w * kG1WindowChunks + c) * 4)
                       : Act<T>::zero();
      }
    }
#pragma unroll
    for (int u = 0; u < WMAX; ++u) {
      const int w = w0 + u;
      const int j = w * kG1Ksub + ks;
      const bool ok = (w < nwin) && (j < G);
#pragma unroll
      for (int i = 0; i < BCQ_MAX_PLANES; ++i) {
        bw[u][i] = (ok && i < p) ? tbits[i * plane_stride + (size_t)j * kTileRows]
                                 : make_uint4(0u, 0u, 0u, 0u);
        al[u][i] = (ok && row_ok && i < p) ? alpha[i * MG + (size_t)m * G + j] : T(0);
      }
      zz[u] = (ok && row_ok) ? zero[(size_t)m * G + j] : T(0);
    }

#pragma unroll
    for (int u = 0; u < WMAX; ++u) {
      const int w = w0 + u;
      if (w >= nwin) break;  // uniform over the workgroup
      __syncthreads();       // the previous window's lookups are done with lut[]
      // ---- build the window's tables (chunk c = tid and tid + 256)
      float cs[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = tid + h * kG1Threads;
        float f[4];
        Act<T>::cvt(xr[u][h], f);
        float4 v[4];
        chunk_entries(f, v);
        float4 *dst = reinterpret_cast<float4 *>(lut + (c / kChunksPerGroup) * kG1GroupStride +
                                                 (c % kChunksPerGroup) * kG1ChunkStride);
        dst[0] = v[0];
        dst[1] = v[1];
        dst[2] = v[2];
        dst[3] = v[3];
        cs[h] = (f[0] + f[1]) + (f[2] + f[3]);
      }
      // group sums: the 32 chunks of a group are 32 consecutive lanes
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) {
        cs[0] += __shfl_xor(cs[0], off);
        cs[1] += __shfl_xor(cs[1], off);
      }
      if ((tid & 31) == 0) {
        gsum[tid / 32] = cs[0];
        gsum[tid / 32 + 8] = cs[1];
      }
      __syncthreads();
      // ---- lookups for this lane's group
      const int j = w * kG1Ksub + ks;
      if (j < G) {
        const uint32_t base = lds_addr(lut + ks * kG1GroupStride);
#pragma unroll
        for (int i = 0; i < BCQ_MAX_PLANES; ++i) {
          if (i < p) acc = fmaf((float)al[u][i], g1_plane_sum(bw[u][i], base), acc);
        }
        acc = fmaf((float)zz[u], gsum[ks], acc);
      }
    }
  }

  // ---- reduce the 16 K-sub partials of each row in a fixed order
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if (lane < 16) part[wave][lane] = acc;
  __syncthreads();
  if (tid < kTileRows) {
    const float s = (part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid]);
    const int mm = tile * kTileRows + tid;
    if (mm < M) y[mm] = (T)s;
  }
}

template <typename T>
hipError_t gemv_dispatch(const uint32_t *bits, int M, int K, int p, const void *alpha,
                         const void *zero, const void *x, void *y, hipStream_t s) {
  const int G = K / kGroup;
  const int MT = row_tiles(M);
  const int nwin = (G + kG1Ksub - 1) / kG1Ksub;
  const uint4 *b4 = reinterpret_cast<const uint4 *>(bits);
  const T *a = static_cast<const T *>(alpha);
  const T *z = static_cast<const T *>(zero);
  const T *xx = static_cast<const T *>(x);
  T *yy = static_cast<T *>(y);
  dim3 grid(MT), block(kG1Threads);
  if (nwin <= 1)
    hipLaunchKernelGGL((gemv_lut_kernel<T, 1>), grid, block, 0, s, b4, a, z, xx, yy, M, G, MT, p);
  else if (nwin <= 2)
    hipLaunchKernelGGL((gemv_lut_kernel<T, 2>), grid, block, 0, s, b4, a, z, xx, yy, M, G, MT, p);
  else if (nwin <= 4)
    hipLaunchKernelGGL((gemv_lut_kernel<T, 4>), grid, block, 0, s, b4, a, z, xx, yy, M, G, MT, p);
  else
    hipLaunchKernelGGL((gemv_lut_kernel<T, 8>), grid, block, 0, s, b4, a, z, xx, yy, M, G, MT, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- batches of 2..8
//
// One wavefront per workgroup: 16 rows x 4 groups per window.  Table entries
// hold NB fp32 values (one per request) side by side, so one address serves NB
// requests.  Requests carry their own precision and scale tables, which is
// how per-request precision costs nothing extra: planes up to the largest
// precision are read once, and a request simply stops accumulating after its
// own p (AnyBCQ paper notes, per-request precision; abstract: negligible
// overhead for per-request selection).

constexpr int kSkThreads = 64;
constexpr int kSkKsub = 4;  // groups per window

// Table geometry for NB requests.  An entry holds up to 4 requests' fp32 sums
// side by side (16 B); with 8 requests a chunk holds two such 16-entry halves,
// so the byte offset of an entry is always nibble * entry_bytes and fits the
// byte-select add.  Chunks sit at a stride of (halves * 16 entries + 1) x 16 B
// so 16-byte writes by consecutive chunks spread over the banks.
template <int NB>
struct SkGeom {
  static constexpr int lanes = NB < 4 ? NB : 4;                      // requests per entry
  static constexpr int halves = NB / lanes;                          // 1 or 2
  static constexpr int entry_bytes = lanes * 4;                      // 8 or 16
  static constexpr int half_bytes = kEntries * entry_bytes;          // 128 or 256
  static constexpr int chunk_stride = halves * half_bytes + 16;
  static constexpr int group_stride = kChunksPerGroup * chunk_stride;
  static constexpr int window_bytes = kSkKsub * group_stride;
  static constexpr int window_chunks = kSkKsub * kChunksPerGroup;    // 128
};

// Per-request plane sums over one group: s[q] += T_c[nibble c] for request q.
template <int NB>
__device__ __forceinline__ void sk_plane_sums(const uint4 bw, uint32_t base, float (&s)[NB]) {
  using Gm = SkGeom<NB>;
#pragma unroll
  for (int q = 0; q < NB; ++q) s[q] = 0.f;
  const uint32_t wd[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t ev, od;  // nibble * entry_bytes, one per byte (even nibbles, odd nibbles)
    if constexpr (Gm::entry_bytes == 8) {
      ev = (wd[q] << 3) & 0x78787878u;
      od = (wd[q] >> 1) & 0x78787878u;
    } else {
      ev = (wd[q] << 4) & 0xF0F0F0F0u;
      od = wd[q] & 0xF0F0F0F0u;
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = q * 8 + 2 * b + e;
        uint32_t a;
        if (b == 0) a = add_byte<0>(base, e ? od : ev);
        else if (b == 1) a = add_byte<1>(base, e ? od : ev);
        else if (b == 2) a = add_byte<2>(base, e ? od : ev);
        else a = add_byte<3>(base, e ? od : ev);
        const uint32_t off = c * Gm::chunk_stride;
        if constexpr (Gm::lanes == 2) {
          const f32x2 v = *(lds_float2 *)(size_t)(a + off);
          s[0] += v.x;
          s[1] += v.y;
        } else {
#pragma unroll
          for (int h = 0; h < Gm::halves; ++h) {
            const f32x4 v = *(lds_float4 *)(size_t)(a + off + h * Gm::half_bytes);
            s[4 * h + 0] += v.x;
            s[4 * h + 1] += v.y;
            s[4 * h + 2] += v.z;
            s[4 * h + 3] += v.w;
          }
        }
      }
    }
  }
}

template <typename T, int NB>
__global__ __launch_bounds__(kSkThreads) void skinny_lut_kernel(
    const uint4 *__restrict__ bits, ReqTables tabs, int nreq, int p_max,
    const T *__restrict__ x, int ldx, T *__restrict__ y, int ldy, int M, int G, int MT) {
  using Gm = SkGeom<NB>;
  __shared__ __attribute__((aligned(16))) char lut[Gm::window_bytes];
  __shared__ float gsum[kSkKsub][NB];

  const int lane = threadIdx.x;
  const int r = lane & 15;
  const int ks = lane >> 4;
  const int tile = blockIdx.x;
  const int m = tile * kTileRows + r;
  const bool row_ok = m < M;
  const int nwin = (G + kSkKsub - 1) / kSkKsub;
  const size_t plane_stride = (size_t)MT * G * kTileRows;
  const uint4 *tbits = bits + (size_t)tile * G * kTileRows + r;
  const size_t MG = (size_t)M * G;

  float acc[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) acc[q] = 0.f;

  // registers for the window being consumed; the next window is prefetched
  uint4 bw[BCQ_MAX_PLANES];
  typename Act<T>::raw xr[2][NB];

  auto load_window = [&](int w, uint4 (&b)[BCQ_MAX_PLANES], typename Act<T>::raw (&xv)[2][NB]) {
    const int j = w * kSkKsub + ks;
#pragma unroll
    for (int i = 0; i < BCQ_MAX_PLANES; ++i)
      b[i] = (w < nwin && j < G && i < p_max) ? tbits[i * plane_stride + (size_t)j * kTileRows]
                                               : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = lane + h * kSkThreads;
      const int jc = w * kSkKsub + c / kChunksPerGroup;
#pragma unroll
      for (int q = 0; q < NB; ++q)
        xv[h][q] = (w < nwin && jc < G && q < nreq)
                       ? Act<T>::load(x + (size_t)q * ldx + ((size_t)w * Gm::window_chunks + c) * 4)
                       : Act<T>::zero();
    }
  };

  load_window(0, bw, xr);
  for (int w = 0; w < nwin; ++w) {
    const int j = w * kSkKsub + ks;
    const bool gok = j < G && row_ok;
    // this window's scales and offsets: issued now, consumed after the lookups
    T al[NB][BCQ_MAX_PLANES];
    T zz[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
#pragma unroll
      for (int i = 0; i < BCQ_MAX_PLANES; ++i)
        al[q][i] = (gok && i < tabs.p[q])
                       ? static_cast<const T *>(tabs.alpha[q])[i * MG + (size_t)m * G + j]
                       : T(0);
      zz[q] = (gok && tabs.p[q] > 0) ? static_cast<const T *>(tabs.zero[q])[(size_t)m * G + j]
                                     : T(0);
    }
    uint4 nbw[BCQ_MAX_PLANES];
    typename Act<T>::raw nxr[2][NB];
    load_window(w + 1, nbw, nxr);  // prefetch (all-zero past the end)

    __syncthreads();  // the previous window's lookups are done with lut[]
    // ---- build tables for the 128 chunks of the window, NB requests each
    float cs[2][NB];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = lane + h * kSkThreads;
      char *dst = lut + (c / kChunksPerGroup) * Gm::group_stride +
                  (c % kChunksPerGroup) * Gm::chunk_stride;
#pragma unroll
      for (int hf = 0; hf < Gm::halves; ++hf) {
        constexpr int L = Gm::lanes;
        float4 v[L][4];
#pragma unroll
        for (int q = 0; q < L; ++q) {
          float f[4];
          Act<T>::cvt(xr[h][hf * L + q], f);
          chunk_entries(f, v[q]);
          cs[h][hf * L + q] = (f[0] + f[1]) + (f[2] + f[3]);
        }
        char *hd = dst + hf * Gm::half_bytes;
#pragma unroll
        for (int e = 0; e < kEntries; ++e) {
          char *ed = hd + e * Gm::entry_bytes;
          if constexpr (L == 2) {
            *reinterpret_cast<float2 *>(ed) =
                make_float2(comp(v[0][e >> 2], e & 3), comp(v[1][e >> 2], e & 3));
          } else {
            *reinterpret_cast<float4 *>(ed) =
                make_float4(comp(v[0][e >> 2], e & 3), comp(v[1][e >> 2], e & 3),
                            comp(v[2][e >> 2], e & 3), comp(v[3][e >> 2], e & 3));
          }
        }
      }
    }
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1)
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        cs[0][q] += __shfl_xor(cs[0][q], off);
        cs[1][q] += __shfl_xor(cs[1][q], off);
      }
    if ((lane & 31) == 0) {
#pragma unroll
      for (int q = 0; q < NB; ++q) {
        gsum[lane / 32][q] = cs[0][q];
        gsum[lane / 32 + 2][q] = cs[1][q];
      }
    }
    __syncthreads();

    // ---- lookups, then per-request scale and offset
    if (gok) {
      const uint32_t base = lds_addr(lut + ks * Gm::group_stride);
#pragma unroll
      for (int i = 0; i < BCQ_MAX_PLANES; ++i) {
        if (i < p_max) {
          float ps[NB];
          sk_plane_sums<NB>(bw[i], base, ps);
#pragma unroll
          for (int q = 0; q < NB; ++q) acc[q] = fmaf((float)al[q][i], ps[q], acc[q]);
        }
      }
#pragma unroll
      for (int q = 0; q < NB; ++q) acc[q] = fmaf((float)zz[q], gsum[ks][q], acc[q]);
    }
#pragma unroll
    for (int i = 0; i < BCQ_MAX_PLANES; ++i) bw[i] = nbw[i];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < NB; ++q) xr[h][q] = nxr[h][q];
  }

  // ---- reduce the 4 K-sub partials of each row (lanes r, r+16, r+32, r+48)
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    acc[q] += __shfl_xor(acc[q], 16);
    acc[q] += __shfl_xor(acc[q], 32);
  }
  if (ks == 0 && row_ok) {
#pragma unroll
    for (int q = 0; q < NB; ++q)
      if (q < nreq) y[(size_t)q * ldy + m] = (T)acc[q];
  }
}

template <typename T>
hipError_t skinny_dispatch(const uint32_t *bits, int M, int K, int p_max, const ReqTables &t,
                           int nreq, const void *x, int ldx, void *y, int ldy, hipStream_t s) {
  const int G = K / kGroup;
  const int MT = row_tiles(M);
  const uint4 *b4 = reinterpret_cast<const uint4 *>(bits);
  const T *xx = static_cast<const T *>(x);
  T *yy = static_cast<T *>(y);
  dim3 grid(MT), block(kSkThreads);
  if (nreq <= 2)
    hipLaunchKernelGGL((skinny_lut_kernel<T, 2>), grid, block, 0, s, b4, t, nreq, p_max, xx, ldx,
                       yy, ldy, M, G, MT);
  else if (nreq <= 4)
    hipLaunchKernelGGL((skinny_lut_kernel<T, 4>), grid, block, 0, s, b4, t, nreq, p_max, xx, ldx,
                       yy, ldy, M, G, MT);
  else
    hipLaunchKernelGGL((skinny_lut_kernel<T, 8>), grid, block, 0, s, b4, t, nreq, p_max, xx, ldx,
                       yy, ldy, M, G, MT);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_lut(const uint32_t *bits, int M, int K, int p, const void *alpha,
                           const void *zero, const void *x, void *y, bcq_dtype dt,
                           hipStream_t s) {
  if (dt == BCQ_F16) return gemv_dispatch<half_t>(bits, M, K, p, alpha, zero, x, y, s);
  return gemv_dispatch<float>(bits, M, K, p, alpha, zero, x, y, s);
}

hipError_t launch_skinny_lut(const uint32_t *bits, int M, int K, int p_max, const ReqTables &t,
                             int nreq, const void *x, int ldx, void *y, int ldy, bcq_dtype dt,
                             hipStream_t s) {
  if (dt == BCQ_F16) return skinny_dispatch<half_t>(bits, M, K, p_max, t, nreq, x, ldx, y, ldy, s);
  return skinny_dispatch<float>(bits, M, K, p_max, t, nreq, x, ldx, y, ldy, s);
}

}  // namespace bcq
