// gemm_mfma.hip -- BCQ product for 16 or more fp16 requests at one precision:
// weights decoded to fp16 on the vector ALUs and contracted on the matrix
// cores (v_mfma_f32_16x16x32_f16, fp32 accumulation).
//
// Why this path: past a few requests the product is a dense contraction of
// the decoded weights with the requests' activations, so it belongs on the
// matrix cores; the BiLoCo summary's speed results make the same point for
// its +-1 correction, whose add/subtract work grows with batch while the
// weight read stays flat.  The decode (decode.h) is the same as the batched
// vector kernel's: per plane and fp16 pair one shift, one bit-field insert and
// one packed add, so a weight is decoded once per launch whatever the batch.
//
// Operand layout.  A wavefront owns one 16-row tile.  For each group, lane
// (r, h) decodes row r's h-th 32-column word into 16 fp16 pairs; pairs
// 4n..4n+3 (columns 32h + 8n .. 8n+7) are that lane's A operand of MFMA n,
// i.e. lane (r, h) supplies row r and k-block h of a 32-wide k slice made of
// columns 8n..8n+7 of each of the group's four words.  The B operand of lane
// (c, h) is then request c's activations at the same 8 columns: one 16-byte
// LDS read of x in its natural order.  Four MFMAs cover a group for 16
// requests; NT tiles of 16 requests reuse each decoded pair.
//
// Staging.  The four wavefronts (64 rows) share each window's activations,
// staged in LDS as [group][word][8-column block][request] 16-byte blocks;
// every word's region is padded by 128 bytes so the two words read by one
// half-wavefront fall 32 banks apart.  The next window is loaded into
// registers while the current one computes and written to the other LDS
// buffer before the barrier, so one barrier per window suffices.
//
// Split K.  blockIdx.y takes a contiguous run of windows; with more than one
// run the partial products go to an fp32 workspace and a finalize kernel sums
// them in a fixed order, so results are deterministic.
#include "decode.h"

namespace bcq {
namespace {

using half_t = _Float16;
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
// 16-byte blocks as a native vector (HIP's uint4 struct is copied with memcpy,
// which keeps the staging registers from being promoted out of memory)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfWaves = 4;  // 16-row tiles per workgroup, one per wavefront
constexpr int kMfThreads = 64 * kMfWaves;
constexpr int kMfGroups = 4;           // groups per window
constexpr int kMfWords = kGroup / 32;  // 32-column words per group
constexpr int kMfBlocks = 4;           // 8-column blocks per word

template <int NB>
struct MfStage {
  static constexpr int kWordStride = kMfBlocks * NB + 8;  // 16-byte blocks
  static constexpr int kGroupStride = kMfWords * kWordStride;
  static constexpr int kBufBlocks = kMfGroups * kGroupStride;
  static constexpr int kTasks = kMfGroups * kMfWords * kMfBlocks * NB / kMfThreads;  // NB / 4
};

// This thread's share of one window's activations (16-byte blocks).
template <int NB>
struct MfX {
  u32x4 v[MfStage<NB>::kTasks];
};

// Operands of one window for one lane: sign words, scales and offsets of its
// row in each of the window's groups.
template <int P>
struct MfW {
  uint32_t bits[kMfGroups][P];
  uint32_t a[kMfGroups][P];
  uint32_t z[kMfGroups];
};

// NT tiles of 16 requests, P planes.  The load phase has no branches: rows past
// M, tiles past MT, requests past b and groups past G read clamped in-range
// addresses whose values are never stored.
template <int NT, int P>
__global__ __launch_bounds__(kMfThreads) void gemm_mfma_kernel(
    const uint32_t *__restrict__ bits, const half_t *__restrict__ alpha,
    const half_t *__restrict__ zero, const half_t *__restrict__ X, int ldx, int b,
    half_t *__restrict__ Y, int ldy, float *__restrict__ ws, int M, int G, int MT, int wps) {
  constexpr int NB = 16 * NT;
  using St = MfStage<NB>;
  using OpsW = MfW<P>;
  using OpsX = MfX<NB>;
  __shared__ u32x4 xs[2][St::kBufBlocks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int h = lane >> 4;
  const int t = blockIdx.x * kMfWaves + wave;
  const int t_safe = min(t, MT - 1);
  const int m_safe = min(t_safe * kTileRows + r, M - 1);
  const int nwin = (G + kMfGroups - 1) / kMfGroups;
  const int s = blockIdx.y;
  const int w0 = s * wps;
  const int w1 = min(nwin, w0 + wps);  // the host leaves no slice empty
  const size_t plane_words = (size_t)MT * G * kTileRows * 4;
  const size_t MG = (size_t)M * G;
  const uint32_t *tb = bits + ((size_t)t_safe * G * kTileRows + r) * 4 + h;

  // staging: block u*256 + tid is (group, word, 8-column block, request), request fastest
  auto fetch_x = [&](int w, OpsX &o) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < St::kTasks; ++u) {
      const int id = u * kMfThreads + tid;
      const int q = min(id % NB, b - 1);
      const int blk = (id / NB) % kMfBlocks;
      const int wrd = (id / (NB * kMfBlocks)) % kMfWords;
      const int grp = id / (NB * kMfBlocks * kMfWords);
      const int j = min(w * kMfGroups + grp, G - 1);
      o.v[u] = *reinterpret_cast<const u32x4 *>(X + (size_t)q * ldx + (size_t)j * kGroup +
                                                 wrd * 32 + blk * 8);
    }
  };
  auto write_x = [&](const OpsX &o, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < St::kTasks; ++u) {
      const int id = u * kMfThreads + tid;
      const int q = id % NB;
      const int blk = (id / NB) % kMfBlocks;
      const int wrd = (id / (NB * kMfBlocks)) % kMfWords;
      const int grp = id / (NB * kMfBlocks * kMfWords);
      xs[buf][grp * St::kGroupStride + wrd * St::kWordStride + blk * NB + q] = o.v[u];
    }
  };
  auto fetch_w = [&](int w, OpsW &o) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < kMfGroups; ++g) {
      const int j = min(w * kMfGroups + g, G - 1);
#pragma unroll
      for (int i = 0; i < P; ++i) {
        o.bits[g][i] = tb[i * plane_words + (size_t)j * kTileRows * 4];
        o.a[g][i] = *reinterpret_cast<const unsigned short *>(alpha + i * MG +
                                                              (size_t)m_safe * G + j);
      }
      o.z[g] = *reinterpret_cast<const unsigned short *>(zero + (size_t)m_safe * G + j);
    }
  };

  // one accumulator per (request tile, 8-column block): the four MFMAs of a
  // group are independent, so they issue back to back instead of waiting for
  // each other's result; the blocks are summed once at the end
  floatx4 acc[NT][kMfBlocks];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int n = 0; n < kMfBlocks; ++n) acc[nt][n] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int w, const OpsW &o, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < kMfGroups; ++g) {
      if (w * kMfGroups + g >= G) break;  // uniform
      dq_half2 wv[kDqPairs];
      dq_init(wv, o.z[g]);
#pragma unroll
      for (int i = 0; i < P; ++i) dq_plane(wv, o.bits[g][i], o.a[g][i]);
      const u32x4 *xb = &xs[buf][g * St::kGroupStride + h * St::kWordStride + r];
#pragma unroll
      for (int n = 0; n < kMfBlocks; ++n) {
        half8 a;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a[2 * u] = wv[4 * n + u][0];
          a[2 * u + 1] = wv[4 * n + u][1];
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const half8 bop = __builtin_bit_cast(half8, xb[n * NB + nt * 16]);
          acc[nt][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bop, acc[nt][n], 0, 0, 0);
        }
      }
    }
  };

  // pipeline over the slice's windows: window w computes from one LDS buffer
  // and its sign words and scales (loaded two windows earlier); then window
  // w+1's activations (loaded a window earlier) go to the other buffer, and
  // the loads of window w+2 are issued last, so the loop header sees the same
  // loads in flight on every path and its waits stay partial
  OpsW wa, wb;
  OpsX xo;
  fetch_x(w0, xo);
  fetch_w(w0, wa);
  write_x(xo, 0);
  fetch_x(w0 + 1, xo);
  fetch_w(w0 + 1, wb);
  __syncthreads();
  for (int w = w0; w < w1; w += 2) {
    compute(w, wa, 0);
    write_x(xo, 1);
    fetch_x(w + 2, xo);
    fetch_w(w + 2, wa);
    __syncthreads();
    if (w + 1 >= w1) break;  // uniform
    compute(w + 1, wb, 1);
    write_x(xo, 0);
    fetch_x(w + 3, xo);
    fetch_w(w + 3, wb);
    __syncthreads();
  }

  // D layout: lane (r, h) holds rows 4h .. 4h+3 of the tile for request r of each tile
  if (t < MT) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const floatx4 d = (acc[nt][0] + acc[nt][1]) + (acc[nt][2] + acc[nt][3]);
      const int n = nt * 16 + r;
      if (n >= b) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int mm = t * kTileRows + 4 * h + v;
        if (mm >= M) continue;
        if (ws == nullptr)
          Y[(size_t)n * ldy + mm] = (half_t)d[v];
        else
          ws[((size_t)s * b + n) * M + mm] = d[v];
      }
    }
  }
}

// Y[n][m] = sum over slices of the partial products, in slice order.
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

// Windows per slice and slice count for (M, K): about 256 workgroups, at least
// two windows per slice (the pipeline's depth), and no empty slice.
void mfma_split(int M, int K, int *wps, int *slices) {
  const int G = K / kGroup;
  const int nwin = (G + kMfGroups - 1) / kMfGroups;
  const int wgs = (row_tiles(M) + kMfWaves - 1) / kMfWaves;
  int s = (256 + wgs - 1) / wgs;
  const int smax = nwin / 2 > 0 ? nwin / 2 : 1;
  s = s < 1 ? 1 : (s > smax ? smax : s);
  *wps = (nwin + s - 1) / s;
  *slices = (nwin + *wps - 1) / *wps;
}

}  // namespace

int mfma_slices(int M, int K) {
  int wps, s;
  mfma_split(M, K, &wps, &s);
  return s;
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
  int wps, S;
  mfma_split(M, K, &wps, &S);
  const half_t *a = static_cast<const half_t *>(alpha);
  const half_t *z = static_cast<const half_t *>(zero);
  const half_t *X = static_cast<const half_t *>(x);
  half_t *Y = static_cast<half_t *>(y);
  float *w = S > 1 ? static_cast<float *>(ws) : nullptr;
  dim3 grid((MT + kMfWaves - 1) / kMfWaves, S), block(kMfThreads);
  const int NT = (b + 15) / 16;
#define BCQ_MF(NTV, PV)                                                                     \
  hipLaunchKernelGGL((gemm_mfma_kernel<NTV, PV>), grid, block, 0, s, bits, a, z, X, ldx, b, Y, \
                     ldy, w, M, G, MT, wps)
#define BCQ_MF_NT(NTV)              \
  switch (p) {                      \
    case 1: BCQ_MF(NTV, 1); break;  \
    case 2: BCQ_MF(NTV, 2); break;  \
    case 3: BCQ_MF(NTV, 3); break;  \
    default: BCQ_MF(NTV, 4); break; \
  }
  if (NT <= 1)
    BCQ_MF_NT(1)
  else if (NT == 2)
    BCQ_MF_NT(2)
  else if (NT == 3)
    BCQ_MF_NT(3)
  else
    BCQ_MF_NT(4)
#undef BCQ_MF_NT
#undef BCQ_MF
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || w == nullptr) return e;
  const size_t n = (size_t)b * M;
  hipLaunchKernelGGL(splitk_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     w, S, b, M, Y, ldy);
  return hipGetLastError();
}

}  // namespace bcq
