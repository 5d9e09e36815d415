// gemm_mfma.hip -- BCQ product for batches of fp16 requests (from 3, or 2
// where K stays within one workgroup): weights decoded to fp16 on the vector
// ALUs and contracted on the matrix cores (v_mfma_f32_16x16x32_f16, fp32
// accumulation).  Two kernels: one that splits K over workgroups (any batch
// up to 64 per launch, partials summed by a finalize kernel) and one that
// keeps K within a workgroup (up to 16 requests, K <= 4096), below.
//
// Why this path: past a few requests the product is a dense contraction of
// the decoded weights with the requests' activations, so it belongs on the
// matrix cores; the BiLoCo summary's speed results make the same point for
// its +-1 correction, whose add/subtract work grows with batch while the
// weight read stays flat.  A weight is decoded once per launch whatever the
// batch.
//
// Decode.  A BCQ weight is w = z + sum_{i<p} alpha_i s_i with s_i = +-1 the
// plane's sign bit (AnyBCQ paper notes, "Method / key designs").  Weights are
// formed as fp16 pairs (columns 2t, 2t+1) of one 32-column packed sign word,
// which holds even columns in its low half and odd columns in its high half
// (pack.hip), so the pair's sign bits are bits t and t+16 and one shift moves
// both to the fp16 sign positions (bits 15 and 31):
//   m     = word' << (15 - t)                      one shift
//   +-a   = (m & 0x80008000) | |alpha| in both     one bit-field insert
// where word' is the sign word inverted, or not when alpha < 0, so that a set
// bit yields +alpha.
//
// Operand layout.  A wavefront owns one 16-row tile and walks K in steps of
// four groups.  Lane (r, h) takes row r of group h of the step: one 16-byte
// load per plane brings its four sign words (128 columns), and the four lanes
// of a row read four consecutive 256-byte blocks of the packed plane, so each
// load instruction reads 1 KB contiguously.  MFMA n (n = 0..15) of a step
// contracts 8-column block n of every group: lane (r, h) supplies row r's
// weights at columns 8n..8n+7 of group h (fp16 pairs 4u..4u+3 of word n / 4,
// u = n % 4) as its A operand, and request r's activations at the same
// columns as its B operand.  The four k-blocks of one MFMA thus come from
// four different groups, which is why the scale has to live in the A operand.
//
// Two ways to apply the scales.
//  * Per plane (one tile of up to 16 requests, or up to 32 with per-request
//    precisions): A = the plane's +-alpha pair per column,
//    one bit-field insert per pair and plane (the shift is shared by two
//    planes, see below), and one MFMA per plane plus one with A = (z, z) for
//    the offset; the matrix cores do the sum over planes.  Each plane has its own
//    accumulator, so requests of one launch may use different precisions
//    (AnyBCQ notes, per-request precision): request r adds the accumulators of
//    its first p_r planes only, all planes having been read once.
//  * Summed (two or more request tiles at one precision): the weight
//    z + sum +-alpha is formed on the vector ALUs (a packed add per pair and
//    plane on top of the decode) and one MFMA per request tile contracts it,
//    since from two request tiles the per-plane MFMAs cost more than the VALU
//    work they save.
//
// Staging.  The eight wavefronts (128 rows) share each step's activations in
// LDS as [request][group][8-column block] 16-byte blocks, the block index
// XOR-swizzled by the request's low four bits: the 64 lanes writing one
// request's 1 KB of a step land in distinct banks, and the 16 requests read at
// one block land in 16 distinct 16-byte bank groups.  Activations of step s+1
// are loaded into registers while step s computes and written to the other LDS
// buffer before the barrier; sign words and scales are loaded two steps ahead.
//
// Split K.  blockIdx.y takes a contiguous run of steps (a slice); with more
// than one slice the partial products go to an fp32 workspace and a finalize
// kernel sums them in slice order, so results are deterministic.  (Summing
// them in the same launch -- the last workgroup of a row block to arrive adds
// the slices -- measured slower on gfx950: the hand-off across the XCDs' L2
// caches needs either an L2 write-back per workgroup or write-through stores
// and coherent reads, while the second launch of a captured graph costs
// little.)
#include "bcq_internal.h"

namespace bcq {
namespace {

using half_t = _Float16;
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ half2v as_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
// 16-byte blocks as a native vector (HIP's uint4 struct is copied with memcpy,
// which keeps staging arrays from being promoted to registers)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfGroups = 4;           // groups per step (lane (r, h) takes group h)
constexpr int kMfBlocks = kGroup / 8;  // 8-column blocks per group (MFMAs per step)

// Wavefronts (16-row tiles) per workgroup: 8, two per SIMD, so one's waits
// and issue stalls are filled by the other.  At 64 requests two wavefronts
// just fit a SIMD's registers (256 each, no spills); measured 5% faster than
// four wavefronts with one per SIMD.
constexpr int mf_waves(int) { return 8; }

template <int NB, int W>
struct MfStage {
  static constexpr int kThreads = 64 * W;
  static constexpr int kBlocks = NB * kMfGroups * kMfBlocks;  // 16-byte blocks per step
  static constexpr int kTasks = kBlocks / kThreads;           // NB / W per thread
};

// LDS block of request q, group h of the step, 8-column block n.
__device__ __forceinline__ int mf_slot(int q, int h, int n) {
  return ((q * kMfGroups + h) << 4) + (n ^ (q & 15));
}

// This thread's share of one step's activations, and a mask of the blocks
// that lie in a group past G (stored as zeros).
template <int NB, int W>
struct MfX {
  u32x4 v[MfStage<NB, W>::kTasks];
  uint32_t past;
};

// One lane's operands of one step: its four sign words per plane, the scales
// and offset of its (row, group) as raw fp16 bits.
template <int P>
struct MfW {
  u32x4 bits[P];
  uint32_t a[P];
  uint32_t z;
};

template <bool SUM, int P>
constexpr int mf_accs() { return SUM ? 1 : P + 1; }

// Precision of each request of a launch (1..P planes), passed by value.
struct MfPrec {
  uint8_t p[kMfMaxBatch];
};

// One lane's decode operands for a step: its sign words inverted unless alpha
// < 0 (a set bit then yields +|alpha|), and |alpha| in both fp16 halves.
template <int P>
__device__ __forceinline__ void mf_prep(const MfW<P> &o, uint32_t (&wp)[P][4],
                                        uint32_t (&mag)[P]) {
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const uint32_t a16 = o.a[i];
    const uint32_t neg = (uint32_t)((int32_t)(a16 << 16) >> 31);
    mag[i] = (a16 & 0x7FFFu) * 0x10001u;
#pragma unroll
    for (int q = 0; q < 4; ++q) wp[i][q] = ~(o.bits[i][q] ^ neg);
  }
}

// Summed decode of 8-column block n: the fp16 weights z + sum_i +-alpha_i of
// columns 8n..8n+7 of this lane's (row, group), planes added in order, each
// add rounded to fp16.  Planes i and i+1 share one 64-bit shift: the high
// word's bits shifted in from the low word land below bit 15, where the mask
// drops them.
template <int P>
__device__ __forceinline__ half8 mf_sum_block(const uint32_t (&wp)[P][4],
                                              const uint32_t (&mag)[P], uint32_t z2, int n) {
  const int q = n >> 2;
  const int u = n & 3;
  half2v w[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) w[v] = as_h2(z2);
#pragma unroll
  for (int i = 0; i < P; i += 2)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      int sh = 15 - (4 * u + v);
      if (i + 1 < P) {
        // opaque shift count: with it known, the compiler proves the spilled
        // bits masked and splits the shift back into two
        asm("" : "+s"(sh));
        const uint64_t w2 = ((uint64_t)wp[i + 1][q] << 32 | wp[i][q]) << sh;
        w[v] += as_h2(((uint32_t)w2 & 0x80008000u) | mag[i]);
        w[v] += as_h2(((uint32_t)(w2 >> 32) & 0x80008000u) | mag[i + 1]);
      } else {
        w[v] += as_h2(((wp[i][q] << sh) & 0x80008000u) | mag[i]);
      }
    }
  half8 a;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    a[2 * v] = w[v][0];
    a[2 * v + 1] = w[v][1];
  }
  return a;
}

// NT tiles of 16 requests, P planes.  Loads clamp rows past M, tiles past MT,
// requests past b and groups past G to in-range addresses; the activations of
// a group past G are staged as zeros, so it adds nothing (its clamped weights
// are finite), and rows or requests past the end are never stored.  Masks are
// applied to the staged activations, never to loaded values right after their
// load, so that no wait for a load is placed ahead of its use.
template <int NT, int P, bool SUM, int W>
__global__ __launch_bounds__(64 * W) void gemm_mfma_kernel(
    const u32x4 *__restrict__ bits, const half_t *__restrict__ alpha,
    const half_t *__restrict__ zero, const half_t *__restrict__ X, int ldx, int b,
    half_t *__restrict__ Y, int ldy, float *__restrict__ ws, int M, int G, int MT, int sps,
    const MfPrec prec) {
  constexpr int NB = 16 * NT;
  constexpr int NA = mf_accs<SUM, P>();
  using St = MfStage<NB, W>;
  using OpsW = MfW<P>;
  using OpsX = MfX<NB, W>;
  __shared__ u32x4 xs[2][St::kBlocks];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int h = lane >> 4;
  const int t = blockIdx.x * W + wave;
  const int t_safe = min(t, MT - 1);
  const int m_safe = min(t_safe * kTileRows + r, M - 1);
  const int nsteps = (G + kMfGroups - 1) / kMfGroups;
  const int sl = blockIdx.y;
  const int s0 = sl * sps;
  const int s1 = min(nsteps, s0 + sps);  // the host leaves no slice empty
  const size_t plane_blocks = (size_t)MT * G * kTileRows;
  const size_t MG = (size_t)M * G;
  const u32x4 *tb = bits + (size_t)t_safe * G * kTileRows + r;

  // block u*256 + tid of a step: 8-column block n fastest, then group, then
  // request, so a wavefront reads 1 KB of one request's row
  auto fetch_x = [&](int s, OpsX &o) __attribute__((always_inline)) {
    const int g = (tid >> 4) & 3;  // the same group for every task of this thread
    o.past = s * kMfGroups + g >= G ? ~0u : 0u;
    const int j = min(s * kMfGroups + g, G - 1);
#pragma unroll
    for (int u = 0; u < St::kTasks; ++u) {
      const int id = u * St::kThreads + tid;
      const int q = min(id >> 6, b - 1);
      o.v[u] = *reinterpret_cast<const u32x4 *>(X + (size_t)q * ldx + (size_t)j * kGroup +
                                                 (id & 15) * 8);
    }
  };
  auto write_x = [&](const OpsX &o, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < St::kTasks; ++u) {
      const int id = u * St::kThreads + tid;
      xs[buf][mf_slot(id >> 6, (id >> 4) & 3, id & 15)] = o.v[u] & ~o.past;
    }
  };
  auto fetch_w = [&](int s, OpsW &o) __attribute__((always_inline)) {
    const int j = min(s * kMfGroups + h, G - 1);
#pragma unroll
    for (int i = 0; i < P; ++i) {
      o.bits[i] = tb[i * plane_blocks + (size_t)j * kTileRows];
      o.a[i] = *reinterpret_cast<const unsigned short *>(alpha + i * MG + (size_t)m_safe * G + j);
    }
    o.z = *reinterpret_cast<const unsigned short *>(zero + (size_t)m_safe * G + j);
  };

  floatx4 acc[NT][NA];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int k = 0; k < NA; ++k) acc[nt][k] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const OpsW &o, int buf) __attribute__((always_inline)) {
    uint32_t wp[P][4], mag[P];
    mf_prep<P>(o, wp, mag);
    const uint32_t z2 = o.z * 0x10001u;
    const u32x4 *xb = xs[buf];
    auto read_b = [&](int n, half8 (&bo)[NT]) __attribute__((always_inline)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        bo[nt] = __builtin_bit_cast(half8, xb[mf_slot(nt * 16 + r, h, n)]);
    };
    if constexpr (SUM) {
      // weights of block n: z + sum +-alpha per column (mf_sum_block)
      auto decode = [&](int n) __attribute__((always_inline)) -> half8 {
        return mf_sum_block<P>(wp, mag, z2, n);
      };
      // software pipeline: block n+1's activations are read and its weights
      // decoded before block n's products are issued, so the LDS latency and
      // the matrix-core work overlap the decode (the compiler otherwise reads
      // each operand just before its product and waits for it there)
      half8 bc[NT], bn[NT];
      read_b(0, bc);
      half8 ac = decode(0);
#pragma unroll
      for (int n = 0; n < kMfBlocks; ++n) {
        half8 an;
        if (n + 1 < kMfBlocks) {
          read_b(n + 1, bn);
          an = decode(n + 1);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ac, bc[nt], acc[nt][0], 0, 0, 0);
        if (n + 1 < kMfBlocks) {
          ac = an;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) bc[nt] = bn[nt];
        }
      }
    } else {
#pragma unroll
      for (int n = 0; n < kMfBlocks; ++n) {
        const int q = n >> 2;
        const int u = n & 3;
        half8 bop[NT];
        read_b(n, bop);
#pragma unroll
        for (int i = 0; i < P; i += 2) {
          // planes i and i+1 share one 64-bit shift: the high word's bits
          // shifted in from the low word land below bit 15, where the mask
          // drops them
          u32x4 av, bv;
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            int sh = 15 - (4 * u + v);
            if (i + 1 < P) {
              // opaque shift count: with it known, the compiler proves the
              // spilled bits masked and splits the shift back into two
              asm("" : "+s"(sh));
              const uint64_t w2 = ((uint64_t)wp[i + 1][q] << 32 | wp[i][q]) << sh;
              av[v] = ((uint32_t)w2 & 0x80008000u) | mag[i];
              bv[v] = ((uint32_t)(w2 >> 32) & 0x80008000u) | mag[i + 1];
            } else {
              av[v] = ((wp[i][q] << sh) & 0x80008000u) | mag[i];
            }
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[nt][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av),
                                                                bop[nt], acc[nt][i], 0, 0, 0);
          if (i + 1 < P) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              acc[nt][i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  __builtin_bit_cast(half8, bv), bop[nt], acc[nt][i + 1], 0, 0, 0);
          }
        }
        const half8 az = __builtin_bit_cast(half8, u32x4{z2, z2, z2, z2});
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt][P] = __builtin_amdgcn_mfma_f32_16x16x32_f16(az, bop[nt], acc[nt][P], 0, 0, 0);
      }
    }
  };

  // pipeline over the slice's steps, two per iteration: step s computes from
  // one LDS buffer and its sign words and scales (loaded two steps earlier).
  // Every path issues the same loads (a fetch past the slice's last step
  // re-reads that step, lines already in flight) and the loop has no exit but
  // its header, so the waits stay partial; no instruction crosses a
  // sched_barrier, since the scheduler would otherwise start a step's scale
  // arithmetic, or the staging of the next step's activations, early and wait
  // there for loads issued just before.  An odd last step runs after the loop,
  // from buffer 0.
  //  * Small staging share (up to 32 requests): the activations of step s+2
  //    are requested as step s starts and staged to LDS after step s+1
  //    computes, two compute phases later (register sets xa, xb alternate).
  //  * Large share (48, 64 requests): one register set, requested after step
  //    s computes and staged after step s+1 -- a second set would not fit the
  //    registers.
  constexpr bool kDeepX = St::kTasks <= 4;
  const int s_last = s1 - 1;
  OpsW wa, wb;
  OpsX xa, xb;
  fetch_x(s0, xb);
  fetch_w(s0, wa);
  write_x(xb, 0);
  fetch_x(min(s0 + 1, s_last), xa);
  fetch_w(min(s0 + 1, s_last), wb);
  __syncthreads();
  int s = s0;
  if constexpr (kDeepX) {
    for (; s + 1 < s1; s += 2) {
      fetch_x(min(s + 2, s_last), xb);
      __builtin_amdgcn_sched_barrier(0);
      compute(wa, 0);
      __builtin_amdgcn_sched_barrier(0);
      write_x(xa, 1);
      fetch_w(min(s + 2, s_last), wa);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      fetch_x(min(s + 3, s_last), xa);
      __builtin_amdgcn_sched_barrier(0);
      compute(wb, 1);
      __builtin_amdgcn_sched_barrier(0);
      write_x(xb, 0);
      fetch_w(min(s + 3, s_last), wb);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    for (; s + 1 < s1; s += 2) {
      compute(wa, 0);
      __builtin_amdgcn_sched_barrier(0);
      write_x(xa, 1);
      fetch_x(min(s + 2, s_last), xa);
      fetch_w(min(s + 2, s_last), wa);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      compute(wb, 1);
      __builtin_amdgcn_sched_barrier(0);
      write_x(xa, 0);
      fetch_x(min(s + 3, s_last), xa);
      fetch_w(min(s + 3, s_last), wb);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (s < s1) compute(wa, 0);

  // D layout: lane (r, h) holds rows 4h .. 4h+3 of the tile for request r of each tile
  const bool vec_ws = (M & 3) == 0 && (reinterpret_cast<uintptr_t>(ws) & 15) == 0;
  const bool vec_y = (M & 3) == 0 && (ldy & 3) == 0 && (reinterpret_cast<uintptr_t>(Y) & 7) == 0;
  if (t < MT) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = nt * 16 + r;
      if (n >= b) continue;
      floatx4 d;
      if constexpr (SUM) {  // one precision per launch
        d = acc[nt][0];
      } else {  // the offset, then the planes this request uses
        const int pn = prec.p[n];
        d = acc[nt][P];
#pragma unroll
        for (int i = 0; i < P; ++i)
          if (i < pn) d += acc[nt][i];
      }
      // the four rows are consecutive: one 16-byte (partials) or 8-byte
      // (outputs) store where the row length and the buffer allow it
      const int mm0 = t * kTileRows + 4 * h;
      if (ws != nullptr && vec_ws && mm0 < M) {
        *reinterpret_cast<floatx4 *>(ws + ((size_t)sl * b + n) * M + mm0) = d;
      } else if (ws == nullptr && vec_y && mm0 < M) {
        *reinterpret_cast<half4v *>(Y + (size_t)n * ldy + mm0) =
            half4v{(half_t)d[0], (half_t)d[1], (half_t)d[2], (half_t)d[3]};
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int mm = mm0 + v;
          if (mm >= M) continue;
          if (ws == nullptr)
            Y[(size_t)n * ldy + mm] = (half_t)d[v];
          else
            ws[((size_t)sl * b + n) * M + mm] = d[v];
        }
      }
    }
  }
}

// Y[n][m] = sum over slices of the partial products, in slice order.  The
// partials of one output are loaded eight at a time so their latencies overlap.
// VEC (M a multiple of 4, workspace 16-byte aligned): each thread sums four
// consecutive outputs of one request with 16-byte loads, and stores them as
// one 8-byte store when Y's rows allow (vec_y).
template <bool VEC>
__global__ __launch_bounds__(256) void splitk_finalize_kernel(const float *__restrict__ ws,
                                                              int slices, int b, int M,
                                                              half_t *__restrict__ Y, int ldy,
                                                              int vec_y) {
  constexpr int E = VEC ? 4 : 1;  // outputs per thread
  const size_t e0 = ((size_t)blockIdx.x * 256 + threadIdx.x) * E;
  if (e0 >= (size_t)b * M) return;
  const int n = (int)(e0 / M);
  const int mm = (int)(e0 % M);
  const size_t stride = (size_t)b * M;
  const float *pp = ws + e0;
  float s[E];
#pragma unroll
  for (int c = 0; c < E; ++c) s[c] = 0.f;
  for (int q0 = 0; q0 < slices; q0 += 8) {
    float v[8][E];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (VEC) {
        const floatx4 f = q0 + k < slices
                              ? *reinterpret_cast<const floatx4 *>(pp + (size_t)(q0 + k) * stride)
                              : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < E; ++c) v[k][c] = f[c];
      } else {
        v[k][0] = q0 + k < slices ? pp[(size_t)(q0 + k) * stride] : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int c = 0; c < E; ++c) s[c] += v[k][c];
  }
  half_t *dst = Y + (size_t)n * ldy + mm;
  if constexpr (VEC) {
    if (vec_y) {
      *reinterpret_cast<half4v *>(dst) = half4v{(half_t)s[0], (half_t)s[1], (half_t)s[2], (half_t)s[3]};
      return;
    }
  }
#pragma unroll
  for (int c = 0; c < E; ++c) dst[c] = (half_t)s[c];
}

// ---------------------------------------------------------------- whole K
//
// Up to 16 requests and K <= 4096 (at most 32 groups): a workgroup owns whole
// 16-row tiles and needs no second pass.  Its eight wavefronts split K, four
// groups each, so wavefront w and lane (r, h) take group 4w + h: one step of
// the split kernel above, with the same decode and per-plane MFMAs.  Every
// request's activations for all of K (at most 16 x 4096 fp16, 128 KB) are
// staged once per workgroup in LDS with coalesced loads, laid out and
// swizzled like the split kernel's stage, and serve every tile the workgroup
// walks (tiles blockIdx.x + k * gridDim.x, grid = min(tiles, CUs)).  The
// eight wavefronts' partial products of each tile meet in LDS and are summed
// in wavefront order (deterministic), two tiles per pair of barriers (one pair
// per tile measured 2-5% slower at 3-4 tiles per workgroup: 14336x4096, b = 4,
// 15.0 -> 14.6 us).  The next tile's sign words and scales are requested while
// the current one computes.
constexpr int kWkWaves = 8;
// compute units of an MI355X (fixed, not queried: workspace sizes follow from it)
constexpr int kMfSlots = 256;
constexpr int kWkMaxGroups = kWkWaves * kMfGroups;  // 32 groups: K <= 4096

__device__ __forceinline__ int wk_slot(int q, int g, int n) {
  return ((q * kWkMaxGroups + g) << 4) + (n ^ (q & 15));
}

// One step of lane (r, h): its group's four sign words per plane against the
// staged activations of group slot gs (the four lanes h of a row take four
// groups), per-plane MFMAs plus the offset MFMA into acc.  rq is the staged
// request row this lane reads as its B operand.
template <int P>
__device__ __forceinline__ void wk_step(floatx4 (&acc)[P + 1], const MfW<P> &o, const u32x4 *xs,
                                        int rq, int gs) {
  uint32_t wp[P][4], mag[P];
  mf_prep<P>(o, wp, mag);
  const uint32_t z2 = o.z * 0x10001u;
  const half8 az = __builtin_bit_cast(half8, u32x4{z2, z2, z2, z2});
#pragma unroll
  for (int n = 0; n < kMfBlocks; ++n) {
    const int q = n >> 2;
    const int u = n & 3;
    const half8 bop = __builtin_bit_cast(half8, xs[wk_slot(rq, gs, n)]);
#pragma unroll
    for (int i = 0; i < P; i += 2) {
      u32x4 av, bv;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        int sh = 15 - (4 * u + v);
        if (i + 1 < P) {
          asm("" : "+s"(sh));
          const uint64_t w2 = ((uint64_t)wp[i + 1][q] << 32 | wp[i][q]) << sh;
          av[v] = ((uint32_t)w2 & 0x80008000u) | mag[i];
          bv[v] = ((uint32_t)(w2 >> 32) & 0x80008000u) | mag[i + 1];
        } else {
          av[v] = ((wp[i][q] << sh) & 0x80008000u) | mag[i];
        }
      }
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, av), bop, acc[i],
                                                      0, 0, 0);
      if (i + 1 < P)
        acc[i + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, bv), bop,
                                                            acc[i + 1], 0, 0, 0);
    }
    acc[P] = __builtin_amdgcn_mfma_f32_16x16x32_f16(az, bop, acc[P], 0, 0, 0);
  }
}

// The offset, then the planes request r uses (all P unless precisions differ).
template <int P, bool MIXED>
__device__ __forceinline__ floatx4 wk_sum(const floatx4 (&acc)[P + 1], const MfPrec &prec,
                                          int r) {
  floatx4 d = acc[P];
  if constexpr (MIXED) {
    const int pn = prec.p[r];
#pragma unroll
    for (int i = 0; i < P; ++i)
      if (i < pn) d += acc[i];
  } else {
#pragma unroll
    for (int i = 0; i < P; ++i) d += acc[i];
  }
  return d;
}

// GU: a gate/up store (rows 0..7 of each 16-row tile are gate rows, 8..15 the
// matching up rows, as bcq_gemv_gate_up lays them out); each tile's eight
// outputs per request are silu(gate) * up, evaluated in fp32 on the summed
// partial products and rounded once.
template <int P, bool MIXED, bool GU = false>
__global__ __launch_bounds__(64 * kWkWaves) void gemm_wk_kernel(
    const u32x4 *__restrict__ bits, const half_t *__restrict__ alpha,
    const half_t *__restrict__ zero, const half_t *__restrict__ X, int ldx, int b,
    half_t *__restrict__ Y, int ldy, int M, int G, int MT, const MfPrec prec) {
  constexpr int kReq = 16;
  __shared__ u32x4 xs[kReq * kWkMaxGroups * kMfBlocks];  // 128 KB
  __shared__ floatx4 red[2][kWkWaves][64];  // partial products of two tiles
  using OpsW = MfW<P>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int h = lane >> 4;
  const int g = wave * kMfGroups + h;  // this lane's group of K
  const int gc = min(g, G - 1);
  const int nt = (MT - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;  // my tiles
  const size_t plane_blocks = (size_t)MT * G * kTileRows;
  const size_t MG = (size_t)M * G;

  // ---- stage the activations: thread tid holds block (group tid / 16,
  // 8-column block tid % 16) of every request.  Groups past G are stored as
  // zeros (their lanes' clamped weights then add nothing).  Requests past b
  // are left unwritten: B-operand column c only reaches output column c, and
  // columns past b are never stored.
  {
    const int sg = tid >> 4;
    const int sn = tid & 15;
    if (sg < G) {
      const half_t *src = X + (size_t)sg * kGroup + sn * 8;
      u32x4 v[kReq];
#pragma unroll
      for (int q = 0; q < kReq; ++q)
        if (q < b) v[q] = *reinterpret_cast<const u32x4 *>(src + (size_t)q * ldx);
#pragma unroll
      for (int q = 0; q < kReq; ++q)
        if (q < b) xs[wk_slot(q, sg, sn)] = v[q];
    } else {
#pragma unroll
      for (int q = 0; q < kReq; ++q) xs[wk_slot(q, sg, sn)] = u32x4{0, 0, 0, 0};
    }
  }

  auto fetch_w = [&](int k, OpsW &o) __attribute__((always_inline)) {
    const int t = (int)blockIdx.x + min(k, nt - 1) * (int)gridDim.x;
    const int m = min(t * kTileRows + r, M - 1);
    const u32x4 *tb = bits + ((size_t)t * G + gc) * kTileRows + r;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      o.bits[i] = tb[i * plane_blocks];
      o.a[i] = *reinterpret_cast<const unsigned short *>(alpha + i * MG + (size_t)m * G + gc);
    }
    o.z = *reinterpret_cast<const unsigned short *>(zero + (size_t)m * G + gc);
  };

  OpsW wa, wb;
  fetch_w(0, wa);
  __syncthreads();

  auto tile = [&](int k, const OpsW &o) __attribute__((always_inline)) {
    floatx4 acc[P + 1];
#pragma unroll
    for (int i = 0; i <= P; ++i) acc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
    wk_step<P>(acc, o, xs, r, g);
    // D layout: lane (c, h) holds rows 4h .. 4h+3 for request c
    red[k & 1][wave][lane] = wk_sum<P, MIXED>(acc, prec, r);
  };
  // sum the eight wavefronts' partials of tiles k0 .. k0+n-1 (n = 1 or 2, k0
  // even) in wavefront order and store them: one pair of barriers per two tiles
  auto flush = [&](int k0, int n) __attribute__((always_inline)) {
    __syncthreads();
    if constexpr (GU) {
      // gate row i (lane l < 32, element v: row 4 * (l >> 4) + v) meets up row
      // i + 8 in lane l + 32, element v; output row t * 8 + i
      if (tid < 32 * 4 * n) {
        const int kk = tid >> 7;
        const int l = (tid >> 2) & 31, v = tid & 3;
        const int c = l & 15;
        const int t = (int)blockIdx.x + (k0 + kk) * (int)gridDim.x;
        const int jo = t * (kTileRows / 2) + 4 * (l >> 4) + v;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int w = 0; w < kWkWaves; ++w) {
          gs += red[kk][w][l][v];
          us += red[kk][w][l + 32][v];
        }
        if (c < b && jo < M / 2) Y[(size_t)c * ldy + jo] = (half_t)silu_mul(gs, us);
      }
    } else if (tid < 64 * 4 * n) {
      const int kk = tid >> 8;
      const int l = (tid >> 2) & 63, v = tid & 3;
      const int c = l & 15;
      const int t = (int)blockIdx.x + (k0 + kk) * (int)gridDim.x;
      const int mm = t * kTileRows + 4 * (l >> 4) + v;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kWkWaves; ++w) sum += red[kk][w][l][v];
      if (c < b && mm < M) Y[(size_t)c * ldy + mm] = (half_t)sum;
    }
    __syncthreads();
  };

  // two tiles per iteration, alternating register sets; a fetch past my last
  // tile re-reads it (lines already in flight), and the loop exits only at its
  // header, so the waits stay partial
  int k = 0;
  for (; k + 1 < nt; k += 2) {
    fetch_w(k + 1, wb);
    __builtin_amdgcn_sched_barrier(0);
    tile(k, wa);
    __builtin_amdgcn_sched_barrier(0);
    fetch_w(k + 2, wa);
    __builtin_amdgcn_sched_barrier(0);
    tile(k + 1, wb);
    __builtin_amdgcn_sched_barrier(0);
    flush(k, 2);
  }
  if (k < nt) {
    tile(k, wa);
    flush(k, 1);
  }
}

// ---------------------------------------------------------------- whole K, requests streamed
//
// 17 to 256 requests at one precision in one launch, 2048 < K <= 4096, one row
// tile per workgroup: its eight wavefronts split K as in the whole-K kernel
// (lane (r, h) of wavefront w takes group 4w + h).  Each lane decodes its 16
// blocks once into the summed fp16 weights z + sum +-alpha (mf_sum_block, 64
// registers), and the requests' activations pass through one 128 KB LDS
// stage, 16 requests at a time, in the whole-K stage's layout.  The
// activations go straight from memory to LDS (global_load_lds_dwordx4, no
// registers), so the decoded weights fit beside everything else without
// spilling.  Up to 64 requests (NT request tiles) the tiles' partials stay in
// registers and the eight wavefronts' partials meet once, in the stage, after
// the last tile; past 64 (NT = 0) the request tiles run in a loop, and after
// each tile's products its partials meet in a small LDS array and are summed
// while the next tile's activations load (one launch for the whole call: the
// weights are decoded once).  Either way the partials are summed in wavefront
// order.  No partial sums leave the compute unit and there is no
// second launch; in exchange every compute unit reads all of the activations
// (b x K fp16) from L2, where the split kernel reads one K slice per 128 rows
// but writes fp32 partials that a finalize reads back.  Wavefront w's groups
// are step w of the split kernel and the wavefront sums run in slice order,
// so the outputs equal the split kernel's bit for bit wherever it takes one
// step per slice (K = 4096, and every 2048 < K < 4096 measured).  Staging two
// 8-request halves in two buffers, so that one half loads while the other is
// contracted, measured slower (4096x4096, b = 64: 13.50 -> 16.26 us): half of
// each product's columns went unused and the barriers doubled.
template <int P, int NT>
__global__ __launch_bounds__(64 * kWkWaves) void gemm_wkx_kernel(
    const u32x4 *__restrict__ bits, const half_t *__restrict__ alpha,
    const half_t *__restrict__ zero, const half_t *__restrict__ X, int ldx, int b,
    half_t *__restrict__ Y, int ldy, int M, int G, int MT) {
  constexpr int kReq = 16;
  constexpr int kStage = kReq * kWkMaxGroups * kMfBlocks;  // 16-byte blocks, 128 KB
  constexpr int kLoads = kStage / (64 * kWkWaves);          // per lane and request tile
  static_assert(kLoads == kReq, "one stage load per request");
  static_assert(kWkWaves * NT * 64 <= kStage, "partials fit the stage");
  __shared__ u32x4 xs[kStage];
  __shared__ floatx4 red[kWkWaves][64];  // one request tile's wavefront partials

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int h = lane >> 4;
  const int g = wave * kMfGroups + h;  // this lane's group of K
  const int gc = min(g, G - 1);
  const int t = blockIdx.x;  // one row tile per workgroup (grid = MT)
  const int m = min(t * kTileRows + r, M - 1);
  const size_t plane_blocks = (size_t)MT * G * kTileRows;
  const size_t MG = (size_t)M * G;
  const int nq = NT > 0 ? NT : (b + kReq - 1) / kReq;  // request tiles

  // Stage request tile q: load j of wavefront w fills slots (8j + w) * 64 +
  // lane, which hold request j, groups 4w .. 4w+3 (wk_slot), so each load
  // reads 1 KB of one request's row; a lane reads the block that the slot's
  // swizzle puts there.  Requests past b re-read request b - 1 and groups past
  // G re-read group G - 1: neither reaches a stored output (columns past b are
  // not stored, and the weights of groups past G are zero).  The request row
  // is uniform, so only a 32-bit byte offset per lane and load remains in
  // vector registers.
  const uint32_t xoff = (uint32_t)gc * (kGroup * 2);
  auto stage_x = [&](int q) __attribute__((always_inline)) {
    // opaque per stage: the compiler would otherwise hoist the sixteen 64-bit
    // addresses of every stage to the start and spill them
    uint32_t xo = xoff;
    asm volatile("" : "+v"(xo));
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const char *row = reinterpret_cast<const char *>(X + (size_t)min(q * kReq + j, b - 1) * ldx);
      __builtin_amdgcn_global_load_lds(
          (const void *)(row + (xo + (uint32_t)((r ^ j) << 4))),
          (__attribute__((address_space(3))) void *)(xs + (j * kWkWaves + wave) * 64), 16, 0, 0);
    }
  };

  // this lane's sign words and scales first (the decode waits for them), then
  // the first request tile's stage, then the pull-in below
  MfW<P> wo;
  {
    const u32x4 *tb = bits + ((size_t)t * G + gc) * kTileRows + r;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      wo.bits[i] = tb[i * plane_blocks];
      wo.a[i] = *reinterpret_cast<const unsigned short *>(alpha + i * MG + (size_t)m * G + gc);
    }
    wo.z = *reinterpret_cast<const unsigned short *>(zero + (size_t)m * G + gc);
  }
  __builtin_amdgcn_sched_barrier(0);
  stage_x(0);
  __builtin_amdgcn_sched_barrier(0);
  // Requests 16.. (the later request tiles) are pulled into L2 now, one
  // 2-byte load per 128-byte line, so that their stages later hit L2 instead
  // of each missing to HBM in turn.  Workgroups go to the eight XCDs
  // round-robin, so the workgroups sharing an XCD split its lines: workgroup
  // i touches part i / 8 of them, a line per thread (a part larger than the
  // workgroup is pulled in only in part).  The load is unconditional (threads
  // past the part re-touch its last line): a load under a branch would be
  // waited for where the branches join.  The value is consumed by an empty
  // asm at the end and never used.
  uint32_t touch = 0;
  {
    const int parts = max(1, (int)gridDim.x >> 3);
    const int per_row = G * 2;  // 128-byte lines of a request's K columns
    const int lines = (b - kReq) * per_row;
    const int per_part = (lines + parts - 1) / parts;
    const int l = min((((int)blockIdx.x >> 3) % parts) * per_part + min(tid, per_part - 1),
                      lines - 1);
    touch = *reinterpret_cast<const unsigned short *>(X + (size_t)(kReq + l / per_row) * ldx +
                                                       (size_t)(l % per_row) * 64);
  }
  __builtin_amdgcn_sched_barrier(0);

  // the tile's weights, decoded once (zero for groups past G)
  half8 aw[kMfBlocks];
  {
    uint32_t wp[P][4], mag[P];
    mf_prep<P>(wo, wp, mag);
    const uint32_t z2 = wo.z * 0x10001u;
#pragma unroll
    for (int n = 0; n < kMfBlocks; ++n) {
      aw[n] = mf_sum_block<P>(wp, mag, z2, n);
      if (g >= G) aw[n] = half8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  if constexpr (NT > 0) {
    // NT request tiles (up to 64 requests): the tiles' partials stay in
    // registers, and the eight wavefronts' partials meet once, in the stage,
    // after the last tile
    floatx4 acc[NT];
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      if (q > 0) stage_x(q);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      half8 bq[kMfBlocks];
#pragma unroll
      for (int n = 0; n < kMfBlocks; ++n) bq[n] = __builtin_bit_cast(half8, xs[wk_slot(r, g, n)]);
      acc[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int n = 0; n < kMfBlocks; ++n)
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw[n], bq[n], acc[q], 0, 0, 0);
      __syncthreads();
    }
    // [wave][q][lane]; lane (c, h) holds rows 4h .. 4h+3 for request 16q + c
    floatx4 *part = reinterpret_cast<floatx4 *>(xs);
#pragma unroll
    for (int q = 0; q < NT; ++q) part[(wave * NT + q) * 64 + lane] = acc[q];
    __syncthreads();
#pragma unroll
    for (int e0 = 0; e0 < NT * 256; e0 += 64 * kWkWaves) {
      const int e = e0 + tid;
      if (e < NT * 256) {
        const int q = e >> 8;
        const int l = (e >> 2) & 63, v = e & 3;
        const int c = q * kReq + (l & 15);
        const int mm = t * kTileRows + 4 * (l >> 4) + v;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < kWkWaves; ++w) sum += part[(w * NT + q) * 64 + l][v];
        if (c < b && mm < M) Y[(size_t)c * ldy + mm] = (half_t)sum;
      }
    }
  } else {
    // Request tile q: wait for its stage, contract it, and once every
    // wavefront is done (the stage is then free) request tile q + 1's stage
    // and sum tile q's eight wavefront partials in wavefront order.  The
    // partials area is rewritten only after the next tile's first barrier,
    // which every thread passes only once its sums are done.
    for (int q = 0; q < nq; ++q) {
      // the stage's loads land in LDS: wait for this wavefront's, then for
      // every wavefront's
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      // every B operand of the request tile is read before the products, so the
      // LDS latency is paid once rather than before each product
      half8 bq[kMfBlocks];
  #pragma unroll
      for (int n = 0; n < kMfBlocks; ++n) bq[n] = __builtin_bit_cast(half8, xs[wk_slot(r, g, n)]);
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
  #pragma unroll
      for (int n = 0; n < kMfBlocks; ++n)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(aw[n], bq[n], acc, 0, 0, 0);
      // lane (c, h) holds rows 4h .. 4h+3 for request 16q + c
      red[wave][lane] = acc;
      __syncthreads();
      if (q + 1 < nq) stage_x(q + 1);
      if (tid < 256) {
        const int l = tid >> 2, v = tid & 3;
        const int c = q * kReq + (l & 15);
        const int mm = t * kTileRows + 4 * (l >> 4) + v;
        float sum = 0.f;
  #pragma unroll
        for (int w = 0; w < kWkWaves; ++w) sum += red[w][l][v];
        if (c < b && mm < M) Y[(size_t)c * ldy + mm] = (half_t)sum;
      }
    }
  }
  asm volatile("" ::"v"(touch));
}

// The streamed whole-K kernel serves uniform-precision calls of 17 to 256
// requests (one launch each) with 16 < G <= 32 on 129 to 256 row tiles (one
// per compute unit; more than half of them busy).  Same-process A/B against the
// split kernel, cold, us: 4096x4096 b = 17 / 32 / 48 / 64 (p = 4) 10.67 /
// 11.95 / 13.49 / 15.27 -> 10.14 / 10.24 / 11.78 / 13.42, b = 64 p = 2 13.44
// -> 11.60; 4096x3072 b = 64 13.61 -> 12.66; 4096x2176 b = 40 11.31 ->
// 10.88; 2048x4096 b = 64 12.57 -> 12.30 (a tie), 1024x4096 b = 64 11.37 ->
// 12.42 (a loss: 64 workgroups).
bool use_wkx(int M, int K, int n, bool mixed) {
  const int G = K / kGroup;
  const int MT = row_tiles(M);
  return !mixed && n > 16 && n <= BCQ_MAX_BATCH && G > kWkMaxGroups / 2 && G <= kWkMaxGroups &&
         MT > kMfSlots / 2 && MT <= kMfSlots;
}

// The whole-K kernel serves a launch when it has one request tile and K fits
// its 32 groups, except at 16 groups or fewer on more tiles than compute units
// (there half its wavefronts idle on every tile and the split kernel wins).
// Measured against the split kernel: 4096x4096 b = 16 10.2 -> 8.7 us,
// 1024x4096 b = 4 7.7 -> 6.2 us, 4096x1024 b = 8 7.4 -> 5.6 us; 14336x2048
// b = 16 16.1 -> 18.4 us.
bool use_wk(int M, int K, int n) {
  const int G = K / kGroup;
  return n <= 16 && G <= kWkMaxGroups && (G > kWkMaxGroups / 2 || row_tiles(M) <= kMfSlots);
}

// Steps per slice and slice count for (M, K) and W wavefronts per workgroup.
// One workgroup is resident per compute unit (the register or LDS budget of
// either size allows no second), so a launch runs in rounds of kMfSlots
// workgroups.  A round costs its steps per slice plus about one step of start-up
// (the first loads' latency, measured near one step's compute); the split
// minimises rounds x (steps per slice + 1), the fewest slices (least
// partial-sum traffic) among equals.  The count is MI355X's, fixed rather than
// queried, because the workspace size follows from it and must not depend on
// which device is current.

void mfma_split(int M, int K, int W, int *sps, int *slices) {
  const int G = K / kGroup;
  const int nsteps = (G + kMfGroups - 1) / kMfGroups;
  const long wgs = (row_tiles(M) + W - 1) / W;
  long best = -1;
  for (int s = 1; s <= nsteps; ++s) {
    const int sp = (nsteps + s - 1) / s;  // steps per slice
    const int sl = (nsteps + sp - 1) / sp;  // slices actually used
    if (sl != s) continue;                  // same split as a smaller s
    const long cost = (wgs * sl + kMfSlots - 1) / kMfSlots * (sp + 1);
    if (best < 0 || cost < best) {
      best = cost;
      *sps = sp;
      *slices = sl;
    }
  }
}

// Workspace of one launch of n requests: fp32 partials [slice][request][row].
size_t launch_workspace_bytes(int M, int K, int n) {
  if (use_wk(M, K, n)) return 0;
  int sps, s;
  mfma_split(M, K, mf_waves((n + 15) / 16), &sps, &s);
  return s > 1 ? (size_t)s * n * M * sizeof(float) : 0;
}

// Arguments of one split-kernel launch.
struct MfArgs {
  const u32x4 *bits;
  const half_t *alpha, *zero, *X;
  int ldx, b;
  half_t *Y;
  int ldy;
  float *ws;
  int M, G, MT, sps;
  MfPrec prec;
};

// Instantiates only the variants the dispatch can reach: the per-plane form
// for one or two request tiles, the summed form from two.
template <int NTV, int PV>
void launch_mf(bool sum, dim3 grid, hipStream_t s, const MfArgs &g) {
  constexpr int W = mf_waves(NTV);
  if constexpr (NTV >= 2) {
    if (sum) {
      hipLaunchKernelGGL((gemm_mfma_kernel<NTV, PV, true, W>), grid, dim3(64 * W), 0, s, g.bits,
                         g.alpha, g.zero, g.X, g.ldx, g.b, g.Y, g.ldy, g.ws, g.M, g.G, g.MT, g.sps,
                         g.prec);
      return;
    }
  }
  if constexpr (NTV <= 2)
    hipLaunchKernelGGL((gemm_mfma_kernel<NTV, PV, false, W>), grid, dim3(64 * W), 0, s, g.bits,
                       g.alpha, g.zero, g.X, g.ldx, g.b, g.Y, g.ldy, g.ws, g.M, g.G, g.MT, g.sps,
                       g.prec);
}

template <int PV>
void launch_mf_nt(int NT, bool sum, dim3 grid, hipStream_t s, const MfArgs &g) {
  if (NT <= 1)
    launch_mf<1, PV>(sum, grid, s, g);
  else if (NT == 2)
    launch_mf<2, PV>(sum, grid, s, g);
  else if (NT == 3)
    launch_mf<3, PV>(sum, grid, s, g);
  else
    launch_mf<4, PV>(sum, grid, s, g);
}

}  // namespace

bool mfma_whole_k(int M, int K, int n) { return use_wk(M, K, n); }
bool mfma_streamed(int M, int K, int n) { return use_wkx(M, K, n, false); }

size_t mfma_workspace_bytes(int M, int K, int b) {
  // the launches of one call run in order and reuse the workspace; a call
  // splits b into launches of kMfMaxBatch requests (one precision) or of
  // kMfMaxMixed (per-request precisions), the last launch taking the rest
  size_t need = 0;
  for (int chunk : {kMfMaxBatch, kMfMaxMixed}) {
    const int sizes[2] = {b < chunk ? b : chunk, b > chunk ? b % chunk : 0};
    for (int n : sizes) {
      if (n == 0) continue;
      const size_t r = launch_workspace_bytes(M, K, n);
      need = r > need ? r : need;
    }
  }
  return need;
}

bool mfma_gate_up_ok(int K, int n) { return n <= 16 && K / kGroup <= kWkMaxGroups; }

hipError_t launch_gemm_gate_up(const uint32_t *bits, int M, int K, int p, const void *alpha,
                               const void *zero, const void *x, int ldx, int b, void *y, int ldy,
                               const int32_t *p_req, hipStream_t s) {
  const int G = K / kGroup;
  const int MT = row_tiles(M);
  const u32x4 *b4 = reinterpret_cast<const u32x4 *>(bits);
  const half_t *a = static_cast<const half_t *>(alpha);
  const half_t *z = static_cast<const half_t *>(zero);
  const half_t *X = static_cast<const half_t *>(x);
  half_t *Y = static_cast<half_t *>(y);
  MfPrec prec;
  bool mixed = false;
  for (int q = 0; q < kMfMaxBatch; ++q) {
    prec.p[q] = (uint8_t)(p_req != nullptr && q < b ? p_req[q] : p);
    mixed = mixed || (q < b && prec.p[q] != p);
  }
  const dim3 grid(MT < kMfSlots ? MT : kMfSlots), block(64 * kWkWaves);
#define BCQ_WKGU(PV)                                                                          \
  if (mixed)                                                                                  \
    hipLaunchKernelGGL((gemm_wk_kernel<PV, true, true>), grid, block, 0, s, b4, a, z, X, ldx, b, \
                       Y, ldy, M, G, MT, prec);                                               \
  else                                                                                        \
    hipLaunchKernelGGL((gemm_wk_kernel<PV, false, true>), grid, block, 0, s, b4, a, z, X, ldx, \
                       b, Y, ldy, M, G, MT, prec)
  switch (p) {
    case 1: BCQ_WKGU(1); break;
    case 2: BCQ_WKGU(2); break;
    case 3: BCQ_WKGU(3); break;
    default: BCQ_WKGU(4); break;
  }
#undef BCQ_WKGU
  return hipGetLastError();
}

hipError_t launch_gemm_mfma(const uint32_t *bits, int M, int K, int p, const void *alpha,
                            const void *zero, const void *x, int ldx, int b, void *y, int ldy,
                            void *ws, const int32_t *p_req, hipStream_t s) {
  const int G = K / kGroup;
  const int MT = row_tiles(M);
  const int NT = (b + 15) / 16;
  const u32x4 *b4 = reinterpret_cast<const u32x4 *>(bits);
  const half_t *a = static_cast<const half_t *>(alpha);
  const half_t *z = static_cast<const half_t *>(zero);
  const half_t *X = static_cast<const half_t *>(x);
  half_t *Y = static_cast<half_t *>(y);
  MfPrec prec;
  for (int q = 0; q < kMfMaxBatch; ++q)
    prec.p[q] = (uint8_t)(p_req != nullptr && q < b ? p_req[q] : p);
  if (use_wk(M, K, b)) {
    dim3 grid(MT < kMfSlots ? MT : kMfSlots), block(64 * kWkWaves);
    bool mixed = false;
    for (int q = 0; q < b; ++q) mixed = mixed || prec.p[q] != p;
#define BCQ_WK(PV)                                                                           \
  if (mixed)                                                                                 \
    hipLaunchKernelGGL((gemm_wk_kernel<PV, true>), grid, block, 0, s, b4, a, z, X, ldx, b, Y, \
                       ldy, M, G, MT, prec);                                                 \
  else                                                                                       \
    hipLaunchKernelGGL((gemm_wk_kernel<PV, false>), grid, block, 0, s, b4, a, z, X, ldx, b, Y, \
                       ldy, M, G, MT, prec)
    switch (p) {
      case 1: BCQ_WK(1); break;
      case 2: BCQ_WK(2); break;
      case 3: BCQ_WK(3); break;
      default: BCQ_WK(4); break;
    }
#undef BCQ_WK
    return hipGetLastError();
  }
  if (use_wkx(M, K, b, p_req != nullptr)) {
    // up to 64 requests: the request tiles unrolled, partials summed once;
    // more: a loop over request tiles, each tile's partials summed in turn
    const dim3 grid(MT), block(64 * kWkWaves);  // MT <= kMfSlots: one tile per workgroup
    const int nt = b <= kMfMaxBatch ? NT : 0;
#define BCQ_WKX(PV)                                                                          \
  switch (nt) {                                                                              \
    case 2: hipLaunchKernelGGL((gemm_wkx_kernel<PV, 2>), grid, block, 0, s, b4, a, z, X, ldx, \
                               b, Y, ldy, M, G, MT); break;                                  \
    case 3: hipLaunchKernelGGL((gemm_wkx_kernel<PV, 3>), grid, block, 0, s, b4, a, z, X, ldx, \
                               b, Y, ldy, M, G, MT); break;                                  \
    case 4: hipLaunchKernelGGL((gemm_wkx_kernel<PV, 4>), grid, block, 0, s, b4, a, z, X, ldx, \
                               b, Y, ldy, M, G, MT); break;                                  \
    default: hipLaunchKernelGGL((gemm_wkx_kernel<PV, 0>), grid, block, 0, s, b4, a, z, X, ldx, \
                                b, Y, ldy, M, G, MT); break;                                 \
  }
    switch (p) {
      case 1: BCQ_WKX(1); break;
      case 2: BCQ_WKX(2); break;
      case 3: BCQ_WKX(3); break;
      default: BCQ_WKX(4); break;
    }
#undef BCQ_WKX
    return hipGetLastError();
  }
  const int W = mf_waves(NT);
  int sps, S;
  mfma_split(M, K, W, &sps, &S);
  float *w = S > 1 ? static_cast<float *>(ws) : nullptr;
  // summed decode from two request tiles at one precision (measured 6-11%
  // faster at 32 requests: half the MFMAs for one packed add per pair and
  // plane); per-plane accumulators for one tile or per-request precisions
  const bool sum = NT >= 3 || (NT == 2 && p_req == nullptr);
  const MfArgs args{b4, a, z, X, ldx, b, Y, ldy, w, M, G, MT, sps, prec};
  dim3 grid((MT + W - 1) / W, S);
  switch (p) {
    case 1: launch_mf_nt<1>(NT, sum, grid, s, args); break;
    case 2: launch_mf_nt<2>(NT, sum, grid, s, args); break;
    case 3: launch_mf_nt<3>(NT, sum, grid, s, args); break;
    default: launch_mf_nt<4>(NT, sum, grid, s, args); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || w == nullptr) return e;
  const size_t n = (size_t)b * M;
  const int vec_y = M % 4 == 0 && ldy % 4 == 0 && reinterpret_cast<uintptr_t>(Y) % 8 == 0;
  if (M % 4 == 0 && reinterpret_cast<uintptr_t>(w) % 16 == 0)
    hipLaunchKernelGGL(splitk_finalize_kernel<true>, dim3((unsigned)((n / 4 + 255) / 256)),
                       dim3(256), 0, s, w, S, b, M, Y, ldy, vec_y);
  else
    hipLaunchKernelGGL(splitk_finalize_kernel<false>, dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, s, w, S, b, M, Y, ldy, 0);
  return hipGetLastError();
}

}  // namespace bcq
