// gemv_dq.hip -- BCQ products for small fp16 batches (2..16 requests per launch)
// on the vector ALUs: each weight is decoded once from its sign planes and
// reused by every request of the launch.
//
// Method (AnyBCQ paper notes, "Method / key designs"): the p-plane weight is
// w = z + sum_{i<p} alpha_i s_i with s_i = +-1 the plane's sign bit and
// (alpha_i, z) the scale and offset of the weight's (row, 128-column group);
// y = W x.  With several requests the decode of w is the shared part of the
// work (the pages' point that the +-1 work stays flat while the per-request
// work grows with batch), so it is done once per weight and each request then
// costs one fused multiply-add per weight.
//
// The decode itself is in decode.h: per plane and fp16 pair one shift, one
// bit-field insert and one packed add.  The pair then meets each request's
// natural activation pair (columns 2t, 2t+1) in v_dot2_f32_f16 (exact fp16
// products, fp32 accumulation).  The decoded weight carries fp16 rounding,
// which is why this path serves fp16 inputs only; fp32 batches use the exact
// table kernel.
//
// Lane mapping.  A workgroup owns a 16-row tile and walks K in windows of 4
// groups; NH windows are in flight per step, one per 256-lane quarter of the
// workgroup.  Wavefront v takes group v % 4 of its window, lane (r, h) row r
// and the h-th 32-column word of that group, i.e. one packed sign word per
// plane.  Activations of the step are staged in LDS
// ([window][group][request][word][pair]) by the whole workgroup, double
// buffered, so each step needs one barrier.  All 16 lanes of a word read the
// same 64 bytes of a request's pairs (broadcast), and the two words of a
// half-wavefront sit 64 bytes apart (distinct banks).
#include "decode.h"

namespace bcq {
namespace {

using half_t = _Float16;
using half2v = dq_half2;
// 16-byte blocks as a native vector: HIP's uint4 is a struct copied with
// memcpy, which keeps arrays of it out of registers (in scratch or LDS).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kDqGroups = 4;           // groups per window (one per wavefront)
constexpr int kDqWords = kGroup / 32;  // 32-column sign words per group

// Windows in flight per workgroup: 4 (16 wavefronts, at most 128 VGPRs each)
// while the requests' accumulators and activation reads fit that budget, 2
// (8 wavefronts, up to 256 VGPRs) for more requests.  Mixed precisions keep
// more values live (the dot products follow several planes), so they switch
// earlier, and they are launched with at most 8 requests.
template <int NB, bool MIXED>
constexpr int dq_concurrent() { return NB <= (MIXED ? 2 : 4) ? 4 : 2; }
constexpr int kDqMaxMixed = kDqMaxMixedReq;

// Operands of one step for one lane: the sign words, scales and offset of its
// (row, group, word) position, and this thread's share of the activations to
// stage for the step after.
template <int NB, int P>
struct DqW {
  uint32_t bits[P];
  uint32_t a[P];
  uint32_t z;
};
template <int NB>
struct DqX {
  static constexpr int kTasks = (NB + 3) / 4;  // 16-byte pair blocks this thread stages
  u32x4 v[kTasks];                             // columns 8b .. 8b+7 of a word: pairs 4b..4b+3
};

// P: planes decoded (the largest precision of the launch).  MIXED: requests
// differ in precision, so after each plane the requests at that precision
// take the weight; otherwise every request takes it after plane P.
template <int NB, int P, int NH, bool MIXED>
__global__ __launch_bounds__(256 * NH) __attribute__((amdgpu_waves_per_eu(NH, NH))) void skinny_dq_kernel(
    const uint32_t *__restrict__ bits, const half_t *__restrict__ alpha,
    const half_t *__restrict__ zero, DqRequests rq, const half_t *__restrict__ x, int ldx,
    half_t *__restrict__ y, int ldy, int M, int G, int MT) {
  using OpsW = DqW<NB, P>;
  using OpsX = DqX<NB>;
  constexpr int kWaves = 4 * NH;
  // staged activations: [buffer][window][group][request][word][pair block] of 4 pairs
  __shared__ u32x4 xs[2][NH][kDqGroups][NB][kDqWords][4];
  __shared__ float part[kWaves][kTileRows][NB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave / kDqGroups;  // window of the step
  const int wl = wave % kDqGroups;    // group of the window
  const int tl = tid % 256;
  const int r = lane & 15;
  const int h = lane >> 4;
  const int tile = blockIdx.x;
  const int m = min(tile * kTileRows + r, M - 1);
  const int nwin = (G + kDqGroups - 1) / kDqGroups;
  const int nstep = (nwin + NH - 1) / NH;
  const size_t plane_words = (size_t)MT * G * kTileRows * 4;
  const size_t MG = (size_t)M * G;
  const uint32_t *tb = bits + ((size_t)tile * G * kTileRows + r) * 4 + h;

  // staging role of this thread: pair block sb of word sh of group sg of its
  // window, for requests sq0 + 4u (wave-uniform, so the row pointers are too)
  const int sb = tl & 3;
  const int sh = (tl >> 2) & 3;
  const int sg = (tl >> 4) & 3;
  const int sq0 = tl >> 6;
  const half_t *xrow[OpsX::kTasks];
#pragma unroll
  for (int u = 0; u < OpsX::kTasks; ++u) {
    const int q = __builtin_amdgcn_readfirstlane(min(sq0 + 4 * u, rq.n - 1));
    xrow[u] = x + (size_t)rq.row[q] * ldx;
  }

  auto fetch_x = [&](int step, OpsX &o) {
    const int w = min(step * NH + half, nwin - 1);
    const int j = min(w * kDqGroups + sg, G - 1);
    const int col = j * kGroup + sh * 32 + sb * 8;
#pragma unroll
    for (int u = 0; u < OpsX::kTasks; ++u) o.v[u] = *reinterpret_cast<const u32x4 *>(xrow[u] + col);
  };
  auto write_x = [&](const OpsX &o, int buf) {
#pragma unroll
    for (int u = 0; u < OpsX::kTasks; ++u) {
      const int q = sq0 + 4 * u;
      if (q < NB) xs[buf][half][sg][q][sh][sb] = o.v[u];  // wave-uniform
    }
  };
  auto fetch_w = [&](int step, OpsW &o) {
    const int w = min(step * NH + half, nwin - 1);
    const int j = min(w * kDqGroups + wl, G - 1);
#pragma unroll
    for (int i = 0; i < P; ++i) {
      o.bits[i] = tb[i * plane_words + (size_t)j * kTileRows * 4];
      o.a[i] = *reinterpret_cast<const unsigned short *>(alpha + i * MG + (size_t)m * G + j);
    }
    o.z = *reinterpret_cast<const unsigned short *>(zero + (size_t)m * G + j);
  };

  float acc[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) acc[q] = 0.f;

  auto compute = [&](int step, const OpsW &o, int buf) {
    const int j = (step * NH + half) * kDqGroups + wl;
    if (j >= G) return;  // wave-uniform
    half2v w[kDqPairs];
    dq_init(w, o.z);
    // the dot products of the requests in mask sel (bit q: request q), one
    // block of 4 pairs at a time: the block's activation reads of every
    // selected request are issued together, then the dot products follow, so
    // NB reads are in flight and consecutive dot2 feed different accumulators
    const u32x4 *xq = &xs[buf][half][wl][0][h][0];  // request q at xq + q * kDqWords * 4
    auto dots = [&](uint32_t sel) {
#pragma unroll
      for (int b4 = 0; b4 < 4; ++b4) {
        u32x4 xv[NB];
#pragma unroll
        for (int q = 0; q < NB; ++q)
          if ((sel >> q) & 1u) xv[q] = xq[q * kDqWords * 4 + b4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int q = 0; q < NB; ++q)
            if ((sel >> q) & 1u) {
              const uint32_t xu = u == 0 ? xv[q].x : u == 1 ? xv[q].y : u == 2 ? xv[q].z : xv[q].w;
              acc[q] = __builtin_amdgcn_fdot2(w[4 * b4 + u], dq_as_h2(xu), acc[q], false);
            }
      }
    };
#pragma unroll
    for (int i = 0; i < P; ++i) {
      dq_plane(w, o.bits[i], o.a[i]);
      if constexpr (MIXED) {
        // requests at precision i + 1 take the weight as it stands now
        const uint32_t at = rq.at[i];
        if (at != 0u) dots(at);
      }
    }
    if constexpr (!MIXED) dots(0xFFFFFFFFu);
  };

  // pipeline: step s computes from one LDS buffer and its sign words and
  // scales (loaded two steps earlier); then the activations of step s+1
  // (loaded a step earlier) go to the other buffer, and the loads of step s+2
  // are issued last.  Issuing them at the end of the body, not its start,
  // leaves the loop header with the same loads in flight on every path, so
  // the waits there stay partial and the loads overlap a whole step.
  OpsX xo;
  OpsW wa, wb;
  fetch_x(0, xo);
  fetch_w(0, wa);
  write_x(xo, 0);
  fetch_x(1, xo);
  fetch_w(1, wb);
  __syncthreads();
  for (int s = 0; s < nstep; s += 2) {
    compute(s, wa, 0);
    write_x(xo, 1);
    fetch_x(s + 2, xo);
    fetch_w(s + 2, wa);
    __syncthreads();
    if (s + 1 >= nstep) break;  // uniform
    compute(s + 1, wb, 1);
    write_x(xo, 0);
    fetch_x(s + 3, xo);
    fetch_w(s + 3, wb);
    __syncthreads();
  }

  // ---- reduce: the 4 words of a row in the wavefront, then the wavefronts
  // (groups and windows) through LDS, in a fixed order
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    acc[q] += __shfl_xor(acc[q], 16);
    acc[q] += __shfl_xor(acc[q], 32);
  }
  if (lane < kTileRows) {
#pragma unroll
    for (int q = 0; q < NB; ++q) part[wave][lane][q] = acc[q];
  }
  __syncthreads();
  static_assert(kTileRows * NB <= 256 * NH, "one output per thread");
  if (tid < kTileRows * NB) {
    const int q = tid / kTileRows;
    const int rr = tid % kTileRows;
    const int mm = tile * kTileRows + rr;
    int yrow = 0;  // rq.row[q], selected with constant indices
#pragma unroll
    for (int k = 0; k < NB; ++k) yrow = (k == q) ? rq.row[k] : yrow;
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) sum += part[v][rr][q];
    if (q < rq.n && mm < M) y[(size_t)yrow * ldy + mm] = (half_t)sum;
  }
}

template <int NB, int NH, bool MIXED>
void dq_launch_p(dim3 grid, hipStream_t s, const uint32_t *b, const half_t *a, const half_t *z,
                 const DqRequests &rq, const half_t *xx, int ldx, half_t *yy, int ldy, int M,
                 int G, int MT, int P) {
  const dim3 block(256 * NH);
#define BCQ_DQ(PP)                                                                        \
  hipLaunchKernelGGL((skinny_dq_kernel<NB, PP, NH, MIXED>), grid, block, 0, s, b, a, z, rq, xx, \
                     ldx, yy, ldy, M, G, MT)
  switch (P) {
    case 1: BCQ_DQ(1); break;
    case 2: BCQ_DQ(2); break;
    case 3: BCQ_DQ(3); break;
    default: BCQ_DQ(4); break;
  }
#undef BCQ_DQ
}

template <int NB>
void dq_launch_nb(hipStream_t s, const uint32_t *b, const half_t *a, const half_t *z,
                  const DqRequests &rq, const half_t *xx, int ldx, half_t *yy, int ldy, int M,
                  int G, int MT) {
  int P = 0, kinds = 0;
  for (int i = 0; i < BCQ_MAX_PLANES; ++i)
    if (rq.at[i] != 0u) {
      P = i + 1;
      ++kinds;
    }
  if constexpr (NB <= kDqMaxMixed) {
    if (kinds > 1) {
      dq_launch_p<NB, dq_concurrent<NB, true>(), true>(dim3(MT), s, b, a, z, rq, xx, ldx, yy, ldy,
                                                       M, G, MT, P);
      return;
    }
  }
  dq_launch_p<NB, dq_concurrent<NB, false>(), false>(dim3(MT), s, b, a, z, rq, xx, ldx, yy, ldy, M,
                                                     G, MT, P);
}

}  // namespace

hipError_t launch_skinny_dq(const uint32_t *bits, int M, int K, const void *alpha,
                            const void *zero, const DqRequests &rq, const void *x, int ldx,
                            void *y, int ldy, hipStream_t s) {
  const int G = K / kGroup;
  const int MT = row_tiles(M);
  const half_t *a = static_cast<const half_t *>(alpha);
  const half_t *z = static_cast<const half_t *>(zero);
  const half_t *xx = static_cast<const half_t *>(x);
  half_t *yy = static_cast<half_t *>(y);
  if (rq.n <= 2)
    dq_launch_nb<2>(s, bits, a, z, rq, xx, ldx, yy, ldy, M, G, MT);
  else if (rq.n <= 4)
    dq_launch_nb<4>(s, bits, a, z, rq, xx, ldx, yy, ldy, M, G, MT);
  else if (rq.n <= 8)
    dq_launch_nb<8>(s, bits, a, z, rq, xx, ldx, yy, ldy, M, G, MT);
  else
    dq_launch_nb<16>(s, bits, a, z, rq, xx, ldx, yy, ldy, M, G, MT);
  return hipGetLastError();
}

}  // namespace bcq
