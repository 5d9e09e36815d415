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
//  * Tables.  For every 4-column chunk c of x (the 4 columns one nibble of a
//    packed sign word covers, see chunk_base) the workgroup builds the 16 sums
//    T_c[e] = sum_t (bit t of e ? +x_{c,t} : -x_{c,t}) in fp32 in LDS.  One
//    table read then replaces four signed adds: the 4 sign bits of one row in
//    one plane are the table index.  (A 16-entry table per 4 columns keeps the
//    build at 4 entries per column, cheap enough to repeat in every
//    workgroup; 256-entry byte tables would cost 32 entries per column.)
//  * Scales fuse at the group boundary: acc += alpha_i * P_i after the 32
//    lookups of a group, and acc += z * S_j with S_j the group's activation sum
//    (asymmetric BCQ offset, AnyBCQ paper notes, "Training strategy").
//  * Batch 1 (gemv_res_kernel, gemv_h16_kernel, gemv_stream_kernel): a
//    workgroup owns 16-row tiles; lane (r, hs) takes row r and half-group slot
//    hs of a 16-group window of tables (64 columns, two packed words per
//    plane).  K <= 4096 keeps the fp32 tables of all of K resident while the
//    workgroup walks several tiles; fp16 stores up to K = 28672 keep fp16
//    tables resident (in two passes past K = 14336), and so do fp16 stores
//    with 2048 < K <= 4096 when each workgroup takes one tile; other K stream
//    windows of tables through two buffers (with two or more planes, 1024
//    lanes split the planes of each window).  gemv_direct_kernel is the
//    table-free form, kept behind a switch for comparison.
//  * LDS banks.  Table c sits at 80-byte stride (16 entries + 16 B pad) so that
//    the 16-byte writes of 16 consecutive chunks cover distinct banks, and the
//    four slots of a wavefront read disjoint quarters of the 64 banks.
//  * Batches of 2..8 (skinny_lut_kernel): tables hold several requests'
//    sums per entry, see the section below.
//  * Every reduction over lanes and wavefronts runs in a fixed order, so
//    results are deterministic.
#include <stdlib.h>

#include <atomic>
#include <type_traits>

#include "bcq_internal.h"

namespace bcq {
namespace {

using half_t = _Float16;

constexpr int kChunksPerGroup = kGroup / 4;  // 32 four-column chunks per group
constexpr int kEntries = 16;                 // table entries per chunk

// ---------------------------------------------------------------- activations
//
// Table chunk c (0..31) of a group is nibble c % 8 of the group's packed sign
// word c / 8.  The packed word holds the even columns of its 32 in the low half
// and the odd columns in the high half (pack.hip), so the chunk's 4 columns are
// 32*(c/8) + 8*(c%4) + par + {0, 2, 4, 6} with par = (c/4) % 2, and bit t of the
// nibble is the column at offset 2t.  fp16 loads the 8 contiguous activations
// from 32*(c/8) + 8*(c%4) (one 16-byte load) and keeps those of its parity;
// fp32 loads the 4 it needs.

__device__ __forceinline__ int chunk_base(int c) { return 32 * (c >> 3) + 8 * (c & 3); }
__device__ __forceinline__ int chunk_parity(int c) { return (c >> 2) & 1; }

template <typename T>
struct Act;

// Native vector types for values kept in registers (HIP's float4 / uint4 are
// structs copied with memcpy, which can keep arrays of them in scratch memory).
typedef float act_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int act_u32x4 __attribute__((ext_vector_type(4)));

template <>
struct Act<float> {
  using raw = act_f32x4;  // the chunk's 4 activations (every other column)
  static __device__ __forceinline__ raw load(const float *p, int par) {
    return raw{p[par], p[par + 2], p[par + 4], p[par + 6]};
  }
  static __device__ __forceinline__ void cvt(const raw &v, int, float (&f)[4]) {
    f[0] = v.x;
    f[1] = v.y;
    f[2] = v.z;
    f[3] = v.w;
  }
};

template <>
struct Act<half_t> {
  using raw = act_u32x4;  // 8 contiguous fp16 activations; cvt keeps one parity
  static __device__ __forceinline__ raw load(const half_t *p, int) {
    return *reinterpret_cast<const act_u32x4 *>(p);
  }
  static __device__ __forceinline__ void cvt(const raw &v, int par, float (&f)[4]) {
    const int sh = 16 * par;
    f[0] = (float)__builtin_bit_cast(half_t, (unsigned short)(v.x >> sh));
    f[1] = (float)__builtin_bit_cast(half_t, (unsigned short)(v.y >> sh));
    f[2] = (float)__builtin_bit_cast(half_t, (unsigned short)(v.z >> sh));
    f[3] = (float)__builtin_bit_cast(half_t, (unsigned short)(v.w >> sh));
  }
};

// Scales and offsets are loaded as raw bits into a full 32-bit register and
// converted at their use.  (Loading fp16 values straight into _Float16
// variables lets the compiler pack two into one register, which forces a wait
// on each load before the pack and serialises the loads.)
template <typename T>
__device__ __forceinline__ uint32_t load_raw(const T *p) {
  if constexpr (sizeof(T) == 2)
    return (uint32_t)(*reinterpret_cast<const unsigned short *>(p));
  else
    return *reinterpret_cast<const uint32_t *>(p);
}

template <typename T>
__device__ __forceinline__ float raw_to_float(uint32_t v) {
  if constexpr (sizeof(T) == 2)
    return (float)__builtin_bit_cast(half_t, (unsigned short)v);
  else
    return __builtin_bit_cast(float, v);
}

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

// Sum over the 8 consecutive lanes of an aligned block, returned in all 8 (DPP
// lane moves within quad and half-row, no LDS traffic).  The additions run in
// the same pairwise order in every lane, so all 8 hold identical bits.
__device__ __forceinline__ float sum8_lanes(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF,
                                                         0xF, true));  // quad_perm 1,0,3,2
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF,
                                                         0xF, true));  // quad_perm 2,3,0,1
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF,
                                                         0xF, true));  // row_half_mirror
  return v;
}

// Sum over the 32 lanes of an aligned half-wavefront, returned in all 32:
// sum8_lanes, then the other 8-lane block of the 16-lane row (DPP
// row_mirror), then the other row of the half (ds_swizzle, xor 16 within 32
// lanes).  No bounds checks or address arithmetic, unlike a generic shuffle.
__device__ __forceinline__ float sum32_lanes(float v) {
  v = sum8_lanes(v);
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF,
                                                         0xF, true));  // row_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v),
                                                            0x401F));  // xor 16
  return v;
}

// v + the value of lane (lane xor 16) and lane (lane xor 32): the sum over the
// four 16-lane rows at the same position, in all lanes.  xor32 is the LDS
// byte address ((lane ^ 32) * 4) for ds_bpermute, computed once by the caller.
__device__ __forceinline__ float sum_rows4(float v, int xor32) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, v), 0x401F));
  v += __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(xor32, __builtin_bit_cast(int, v)));
  return v;
}

// ---------------------------------------------------------------- batch 1

constexpr int kG1Ksub = 16;         // groups per window of tables
constexpr int kG1ChunkStride = 80;  // bytes per chunk table: 16 entries + 16 B pad

// Gate/up stores (bcq_gemv_gate_up): rows 0..7 of every 16-row tile t are gate
// rows 8t..8t+7 and rows 8..15 the up rows of the same outputs, so a tile's
// writeback holds both products of its 8 outputs: out = silu(g) * u with
// silu(g) = g / (1 + exp(-g)), from the fp32 sums, rounded once.
constexpr int kGuRows = kTileRows / 2;
__device__ __forceinline__ float gate_up_out(float g, float u) { return silu_mul(g, u); }

// ------------------------------------------------ batch 1, whole-K tables
//
// For K <= 4096 the tables of all of K stay resident in LDS (NW <= 2 windows of
// 16 groups).
// A workgroup of 512 lanes per window (at K = 4096 four wavefronts per SIMD,
// so the others hide one's LDS latency) builds them once, then walks its row
// tiles (tile blockIdx.x + k * gridDim.x), loading the next tile's sign words
// while it looks up the current one, and reduces all its tiles at the end.  With
// grid = min(row tiles, CUs) every CU holds one workgroup that streams several
// tiles, so table builds are amortised and loads overlap lookups.  With few
// tiles (RS = 2 or 4 workgroups per tile, see gemv_res_tiles) each workgroup
// takes 16 / RS rows of one tile and its lanes split the planes instead.
//
// Lane (r, hs) of wavefronts 8w..8w+7: row r of the tile, half-group slot
// hs = 0..31 of window w (group hs/2, columns 64*(hs%2) .. +63).  A wavefront's four slots are two
// groups x two halves; in LDS the second half of a group sits 16 banks after
// the first and consecutive groups 32 banks apart, so the four slots read
// disjoint quarters of the 64 banks.

constexpr int kRThreads = 512;
constexpr int kRWaves = kRThreads / 64;
constexpr int kRHalfPad = 64;                        // bytes between the two halves
constexpr int kRGroupStride = kChunksPerGroup * kG1ChunkStride + kRHalfPad + 64;  // 2688
constexpr int kRWindowBytes = kG1Ksub * kRGroupStride;                           // 43008

// Binary low-rank correction fused into the writeback (bcq_gemv_lowrank, the
// BiLoCo summary's inference step): z_r = alpha_r (v_r . x) comes from a launch
// before the product; the product kernel turns z into 16-entry tables of sign
// combinations over 4 consecutive ranks (the primitive of the activation
// tables) and lane (r, slot ls) adds the 8 lookups of its row's u word ls to
// its partial, so the correction rides the product's own reduction and the
// output is rounded once.  Up to kLrMaxWords u words (1024 ranks) per row: one
// word per (row, slot) lane.  The 8 tables of word w sit at float w * 144, so
// the four words a wavefront reads start in different quarters of the banks.
constexpr int kLrMaxWords = 32;
constexpr int kLrWordStride = 8 * kEntries + 16;  // floats: 8 tables + 64 B pad

__device__ __forceinline__ int r_chunk_offset(int c) {  // chunk c (0..31) within its group
  return c * kG1ChunkStride + (c >= 16 ? kRHalfPad : 0);
}

// Sum over the 16 chunks of one half group of T_c[nibble].  base is the LDS
// byte offset of the half's first table; the second 8 chunks follow the
// first 8 at the same stride.
__device__ __forceinline__ float r_half_sum(const uint2 bw, uint32_t base) {
  constexpr int S = kG1ChunkStride / 4;  // chunk stride in floats
  const uint32_t wd[2] = {bw.x, bw.y};
  float s[4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
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

// Scales and offsets of a tile are staged through LDS: in the caller's
// [p][M][G] layout the 16 rows of a tile are one contiguous run of 16*G
// values per plane, so consecutive threads load consecutive elements
// (coalesced), and each lane then reads its own (row, group) values from
// LDS.  Loading them per lane straight from memory instead touches one
// cache line per row for every 2-byte value and more than doubles the
// kernel's time.  Every tile's are staged before the table-build barrier,
// the (tile, array) loads spread evenly over all lanes; the lookups then run
// through all tiles with no further barrier.  (Staging later tiles behind a
// barrier of their own was measured slower at 2 and 4 tiles per workgroup:
// each barrier idles the SIMDs while the last wavefronts finish.)
//
// The workgroup has 512 lanes per window (NW * 8 wavefronts): wavefronts
// 8w..8w+7 look up window w.  At K = 4096 that is four wavefronts per SIMD,
// enough to hide the LDS latency of the lookups, and every lane builds one
// chunk's table.
template <typename T, int NW, int P, int TMAX, int RS = 1, bool GU = false, bool LR = false>
__global__ __launch_bounds__(kRThreads * NW) void gemv_res_kernel(
    const uint4 *__restrict__ bits, const T *__restrict__ alpha, const T *__restrict__ zero,
    const T *__restrict__ x, T *__restrict__ y, int M, int G, int MT,
    const uint32_t *__restrict__ lr_u, const float *__restrict__ lr_z, int R) {
  constexpr int kMaxG = NW * kG1Ksub;
  constexpr int kWaves = kRWaves * NW;
  constexpr int kPos = kTileRows * kMaxG;        // staging positions of one tile
  constexpr int kParts = kRThreads * NW / kPos;  // thread sets sharing a tile's arrays
  constexpr int kPairs = TMAX * (P + 1);                 // (tile, array) pairs to stage
  constexpr int kPerThread = (kPairs + kParts - 1) / kParts;
  static_assert(kRThreads * NW == kParts * kPos, "staging positions tile the workgroup");
  __shared__ __attribute__((aligned(16))) char lut[NW * kRWindowBytes];
  __shared__ float gsum[NW * kG1Ksub];
  __shared__ float part[kWaves][TMAX][kTileRows];
  // staged scales: [tile][plane P = offsets][row][group], as raw bits of the
  // store's type (fp16 scales in 16-bit slots, so eight tiles fit); rows
  // padded to an odd number of words so the 16 rows x 2 groups one wavefront
  // reads hit distinct banks
  using SRaw = typename std::conditional<sizeof(T) == 2, unsigned short, uint32_t>::type;
  constexpr int kSclRow = sizeof(T) == 2 ? kMaxG + 2 : kMaxG + 1;
  __shared__ SRaw scl[TMAX][P + 1][kTileRows][kSclRow];
  // low-rank correction tables (LR): u word w of a row at float w * kLrWordStride
  __shared__ __attribute__((aligned(16))) float lrt[LR ? kLrMaxWords * kLrWordStride : 1];
  static_assert(!LR || !GU, "the correction applies to plain products");
  static_assert(kLrMaxWords <= kRWaves * 4, "one u word per (row, slot) lane");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int win = wave / kRWaves;                      // the window this wavefront looks up
  const int r = lane & 15;
  const int hs = (wave % kRWaves) * 4 + (lane >> 4);  // half-group slot 0..31
  const int gw = hs >> 1;                              // group within the window
  const int half = hs & 1;
  // RS > 1 (one tile per workgroup, few tiles): RS workgroups share tile
  // blockIdx.x / RS, each taking 16 / RS of its rows; lane (r, hs) takes row
  // r % (16 / RS) of that part and planes PC * (r / (16 / RS)) ..  + PC - 1,
  // so the lookups of a tile spread over RS times as many compute units.
  static_assert(RS == 1 || TMAX == 1, "row parts only for one tile per workgroup");
  static_assert(!GU || RS == 1, "a gate/up tile's two halves must meet in one workgroup");
  constexpr int kPartRows = kTileRows / RS;
  constexpr int PC = (P + RS - 1) / RS;  // planes per lane
  const int rl = r % kPartRows;          // row within the part
  const int ph = r / kPartRows;          // plane part of this lane
  const int prow = ((int)blockIdx.x % RS) * kPartRows + rl;  // row within the tile
  const int nt = RS > 1 ? 1 : (MT - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const size_t plane_stride = (size_t)MT * G * kTileRows;  // in uint4
  const size_t MG = (size_t)M * G;
  const uint2 *bits2 = reinterpret_cast<const uint2 *>(bits);

  // ---- activations for the tables: thread tid builds chunk tid % 512 of
  // window tid / 512 (a 32-bit offset from the uniform base x)
  const int bc = tid % kChunksPerGroup;
  const int bj = tid / kChunksPerGroup;  // group of K whose chunk this thread builds
  const typename Act<T>::raw xr = Act<T>::load(
      x + (unsigned)(min(bj, G - 1) * kGroup + chunk_base(bc)), chunk_parity(bc));

  // ---- scales and offsets of every tile.  Thread (row, group) =
  // ((tid % kPos) / kMaxG, tid % kMaxG) owns one position of a tile's 16 x G
  // run per array, for the pairs n = spart, spart + kParts, ... of
  // (tile n / (P+1), array n % (P+1)) (planes, then offsets at array P):
  // consecutive threads read consecutive groups of a row, so the loads are
  // coalesced.  A thread whose last pair index passes the end re-reads the
  // last pair and stages nothing from it.
  const int spart = tid / kPos;
  const int srow = (tid % kPos) / kMaxG;
  const int sg = tid % kMaxG;
  const int sgc = min(sg, G - 1);
  uint32_t sv[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int n = min(u * kParts + spart, kPairs - 1);
    const int k = n / (P + 1), a = n % (P + 1);
    const int row = min((RS > 1 ? (int)blockIdx.x / RS
                                : (int)blockIdx.x + min(k, nt - 1) * (int)gridDim.x) *
                                kTileRows + srow,
                        M - 1);
    const T *src = a < P ? alpha + a * MG : zero;
    sv[u] = load_raw(src + (size_t)row * G + sgc);
  }

  // ---- low-rank correction (LR): lane (r, slot ls) takes u word ls of its
  // row in every tile, and thread tid < 8 * nwu builds the table of ranks
  // 4 tid .. 4 tid + 3 from z (written by the launch before this one).
  const int nwu = LR ? (R + 31) / 32 : 0;
  const int ls = wave * 4 + (lane >> 4);
  uint32_t uw[TMAX];
  float zf[4];
  if constexpr (LR) {
    const int wl = min(ls, nwu - 1);
#pragma unroll
    for (int k = 0; k < TMAX; ++k) {
      const int t = RS > 1 ? (int)blockIdx.x / RS
                           : (int)blockIdx.x + min(k, nt - 1) * (int)gridDim.x;
      const int m = min(t * kTileRows + (RS > 1 ? prow : r), M - 1);
      uw[k] = lr_u[(size_t)m * nwu + wl];
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) zf[q] = 4 * tid + q < R ? lr_z[4 * tid + q] : 0.f;
  }

  // ---- sign words of this lane's half group, one uint2 per plane.  Past my
  // last tile a fetch re-reads my own last tile (lines already in flight), so
  // the load phase stays branch-free.
  // A tile's block of one plane is G * 16 uint4 (G * 32 uint2) from a base
  // that is uniform across the workgroup; a lane's uint2 within it is the
  // 32-bit lq, so each load is a scalar base plus a vector 32-bit offset.
  uint2 tiles[2][P];
  const int js = min(win * kG1Ksub + gw, G - 1);
  const unsigned lq = (unsigned)((js * kTileRows + (RS > 1 ? prow : r)) * 2 + half);
  // planes [u0, u1) of tile k (of the lane's PC planes with RS > 1)
  auto fetch = [&](int k, uint2 (&o)[P], int u0 = 0, int u1 = P) {
    if constexpr (RS > 1) {
      const uint2 *tb = bits2 + (size_t)((int)blockIdx.x / RS) * G * (kTileRows * 2);
#pragma unroll
      for (int u = 0; u < PC; ++u)
        if (u >= u0 && u < u1) o[u] = tb[(size_t)min(ph * PC + u, P - 1) * plane_stride * 2 + lq];
    } else {
      const int t = (int)blockIdx.x + min(k, nt - 1) * (int)gridDim.x;
      const uint2 *tb = bits2 + (size_t)t * G * (kTileRows * 2);
#pragma unroll
      for (int i = 0; i < P; ++i) {
        const uint2 *pb = tb + (size_t)i * plane_stride * 2;
        if (i >= u0 && i < u1) o[i] = pb[lq];
      }
    }
  };
  // tile 0's sign words after the scales (the barrier below waits for those);
  // later tiles' are requested after the barrier, one ahead of the tile being
  // looked up, so the small loads the barrier waits for are not queued behind
  // every tile's sign words.  A short sleep first (about 0.4 us) lets the
  // activation and scale requests of workgroups that start later reach
  // memory before this one's sign words: workgroups start over about 0.6 us,
  // and without it their small loads queue behind the early ones' bulk
  // (measured 4096x4096: 5.60 -> 5.31 us at p = 4; 8192x4096: 7.72 -> 7.35;
  // 14336x4096 within noise).  No sleep at all and requesting the sign words
  // only after the table barrier were both slower.  With one tile and at
  // least three planes, only the first half of the planes goes before the
  // barrier and the rest right after it (4096x4096: p = 3 4.72 -> 4.54 us,
  // p = 4 5.52 -> 5.28; at p = 2 and with several tiles per workgroup the
  // split was 2-11% slower).
  constexpr bool kSplitFirst = TMAX == 1 && RS == 1 && P >= 3;
  constexpr int kFirstPlanes = kSplitFirst ? (P + 1) / 2 : PC;
  __builtin_amdgcn_s_sleep(12);
  fetch(0, tiles[0], 0, kFirstPlanes);

  // ---- build the tables and group sums
  {
    float f[4];
    Act<T>::cvt(xr, chunk_parity(bc), f);
    float4 v[4];
    chunk_entries(f, v);
    float4 *dst = reinterpret_cast<float4 *>(lut + (tid / kRThreads) * kRWindowBytes +
                                             (bj % kG1Ksub) * kRGroupStride + r_chunk_offset(bc));
    dst[0] = v[0];
    dst[1] = v[1];
    dst[2] = v[2];
    dst[3] = v[3];
    const float cs = sum32_lanes((f[0] + f[1]) + (f[2] + f[3]));
    if ((tid & 31) == 0) gsum[bj] = cs;
  }
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int n = u * kParts + spart;
    if (n < kPairs) scl[n / (P + 1)][n % (P + 1)][srow][sg] = (SRaw)sv[u];
  }
  if constexpr (LR) {
    if (tid < 8 * nwu) {
      float4 v[4];
      chunk_entries(zf, v);
      float4 *dst =
          reinterpret_cast<float4 *>(lrt + (tid >> 3) * kLrWordStride + (tid & 7) * kEntries);
      dst[0] = v[0];
      dst[1] = v[1];
      dst[2] = v[2];
      dst[3] = v[3];
    }
  }
  __syncthreads();
  if (kSplitFirst) fetch(0, tiles[0], kFirstPlanes, PC);
  if (TMAX > 1) fetch(1, tiles[1]);

  const int j = win * kG1Ksub + gw;
  const uint32_t base =
      lds_addr(lut + win * kRWindowBytes + gw * kRGroupStride + r_chunk_offset(16 * half));
  auto consume = [&](int k, const uint2 (&o)[P]) -> float {
    float a = 0.f;
    if (j < G) {
      if constexpr (RS > 1) {
        // a plane index past P (P not a multiple of RS) looks up with scale 0
#pragma unroll
        for (int u = 0; u < PC; ++u) {
          const int i = ph * PC + u;
          const float sc = i < P ? raw_to_float<T>(scl[k][min(i, P - 1)][prow][j]) : 0.f;
          a = fmaf(sc, r_half_sum(o[u], base), a);
        }
        if (half == 0 && ph == 0) a = fmaf(raw_to_float<T>(scl[k][P][prow][j]), gsum[j], a);
      } else {
#pragma unroll
        for (int i = 0; i < P; ++i)
          a = fmaf(raw_to_float<T>(scl[k][i][r][j]), r_half_sum(o[i], base), a);
        if (half == 0) a = fmaf(raw_to_float<T>(scl[k][P][r][j]), gsum[j], a);
      }
    }
    return a;
  };

  float acc[TMAX];
#pragma unroll
  for (int k = 0; k < TMAX; ++k) {
    acc[k] = 0.f;
    if (k < nt) acc[k] = consume(k, tiles[k % 2]);
    if (k + 2 < TMAX) fetch(k + 2, tiles[k % 2]);  // refill the slot just read
  }

  // ---- low-rank correction: sum_r u_mr z_r of this lane's 32 ranks (8
  // table reads) joins the row's slot partials; one lane per (row, slot)
  if constexpr (LR) {
    if (ls < nwu && (RS == 1 || ph == 0)) {
      const float *zt = lrt + ls * kLrWordStride;
#pragma unroll
      for (int k = 0; k < TMAX; ++k) {
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) s += zt[q * kEntries + ((uw[k] >> (4 * q)) & 15u)];
        acc[k] += s;
      }
    }
  }

  // ---- reduce the slot partials of each row of each tile, fixed order
  const int xor32 = (lane ^ 32) << 2;
#pragma unroll
  for (int k = 0; k < TMAX; ++k) {
    acc[k] = sum_rows4(acc[k], xor32);
    // plane parts: lanes r, r + 16/RS, .. of a row hold one row's planes
    // (rotations within the 16-lane row, DPP row_ror)
    if constexpr (RS == 4)
      acc[k] += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                              __builtin_bit_cast(int, acc[k]), 0x124, 0xF, 0xF, true));
    if constexpr (RS >= 2)
      acc[k] += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(
                                              __builtin_bit_cast(int, acc[k]), 0x128, 0xF, 0xF, true));
    if (lane < 16) part[wave][k][lane] = acc[k];
  }
  __syncthreads();
  if constexpr (GU) {
    if (tid < TMAX * kGuRows) {
      const int k = tid / kGuRows;
      const int rr = tid % kGuRows;
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        g += part[v][k][rr];
        u += part[v][k][rr + kGuRows];
      }
      const int jo = ((int)blockIdx.x + k * (int)gridDim.x) * kGuRows + rr;
      if (k < nt && jo < M / 2) y[jo] = (T)gate_up_out(g, u);
    }
  } else if (tid < TMAX * kTileRows) {
    const int k = tid / kTileRows;
    const int rr = tid % kTileRows;  // lane rr holds row rr (RS = 1) or part row rr
    const int mm = RS > 1 ? ((int)blockIdx.x / RS) * kTileRows +
                                ((int)blockIdx.x % RS) * kPartRows + rr
                          : ((int)blockIdx.x + k * (int)gridDim.x) * kTileRows + rr;
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) sum += part[v][k][rr];
    if (k < nt && rr < kPartRows && mm < M) y[mm] = (T)sum;
  }
}

// ------------------------------------------------ batch 1, direct add/subtract
//
// The pages name two ways to form B_i x ("AnyBCQ paper notes", direct
// bit-plane kernel): adding and subtracting the activations under each sign
// bit, or looking up sums of sign combinations (the tables above).  This is
// the direct form, for fp16 stores with K <= 4096, in the lane mapping of
// gemv_res_kernel (lane (r, hs): row r, 64 columns of half-group hs; one
// 16-row tile per workgroup) with no tables: each lane loads its 64
// activations as 32 fp16 pairs, turns each plane's sign bits into +-|alpha|
// fp16 pairs (the sign of alpha folded into the bits; one 64-bit shift serves
// the same pair of both 32-column words, as in the matrix-core decode) and
// adds alpha * (x_2t, x_2t+1) per pair with one v_dot2_f32_f16 (fp16
// products are exact in fp32; the sum is fp32).  The offset term is the same
// instruction with (z, z) pairs.  So a weight bit costs 1.25 vector
// instructions, against about 0.6 for a table lookup, but nothing waits for
// tables: the barrier only publishes the staged scales, which are requested
// first.  Selected with BCQ_B1_DIRECT=1 (measured against the tables).
template <int P>
__global__ __launch_bounds__(kRThreads * 2) void gemv_direct_kernel(
    const uint4 *__restrict__ bits, const half_t *__restrict__ alpha,
    const half_t *__restrict__ zero, const half_t *__restrict__ x, half_t *__restrict__ y, int M,
    int G, int MT) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  constexpr int NW = 2;
  constexpr int kMaxG = NW * kG1Ksub;  // 32 groups: K <= 4096
  constexpr int kThreads = kRThreads * NW;
  constexpr int kWaves = kThreads / 64;
  constexpr int kPos = kTileRows * kMaxG;  // staging positions of one array
  constexpr int kParts = kThreads / kPos;  // thread sets sharing the arrays
  constexpr int kPerThread = (P + 1 + kParts - 1) / kParts;
  // staged scales and offsets as fp16 bits, [array][row][group], rows padded
  // to an odd number of words
  __shared__ unsigned short scl[P + 1][kTileRows][kMaxG + 2];
  __shared__ float part[kWaves][kTileRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int win = wave / kRWaves;
  const int r = lane & 15;
  const int hs = (wave % kRWaves) * 4 + (lane >> 4);  // half-group slot 0..31 of window win
  const int j = win * kG1Ksub + (hs >> 1);             // group of this lane
  const int half = hs & 1;
  const int jc = min(j, G - 1);  // a group past G reads the last one and adds nothing
  const int tile = blockIdx.x;
  const size_t plane_stride = (size_t)MT * G * kTileRows;  // in uint4
  const size_t MG = (size_t)M * G;
  const uint2 *bits2 = reinterpret_cast<const uint2 *>(bits);

  // ---- scales and offsets first (the barrier waits for them only): thread
  // (row, group) = ((tid % kPos) / kMaxG, tid % kMaxG) of part tid / kPos
  // loads arrays spart, spart + kParts, ...; consecutive threads read
  // consecutive groups of a row
  const int spart = tid / kPos;
  const int srow = (tid % kPos) / kMaxG;
  const int sg = tid % kMaxG;
  const int srowc = min(tile * kTileRows + srow, M - 1);
  uint32_t sv[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int a = min(u * kParts + spart, P);
    sv[u] = load_raw((a < P ? alpha + (size_t)a * MG : zero) + (size_t)srowc * G + min(sg, G - 1));
  }

  // ---- this lane's 64 activations (32 fp16 pairs), then its sign words
  // (kept as 32 plain words: component indexing into an array of vector
  // registers read the wrong component)
  uint32_t xw[32];
  const half_t *xl = x + (unsigned)(jc * kGroup + half * 64);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const act_u32x4 v = *reinterpret_cast<const act_u32x4 *>(xl + 8 * u);
    xw[4 * u] = v.x;
    xw[4 * u + 1] = v.y;
    xw[4 * u + 2] = v.z;
    xw[4 * u + 3] = v.w;
  }
  uint2 w[P];
  const unsigned lq = (unsigned)(((tile * G + jc) * kTileRows + r) * 2 + half);
#pragma unroll
  for (int i = 0; i < P; ++i) w[i] = bits2[(size_t)i * plane_stride * 2 + lq];

#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int a = u * kParts + spart;
    if (a <= P && sg < G) scl[a][srow][sg] = (unsigned short)sv[u];
  }
  __syncthreads();

  float acc = 0.f;
  if (j < G) {
    auto xp = [&](int q) -> h2_t { return __builtin_bit_cast(h2_t, xw[q]); };
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const uint32_t a16 = scl[i][r][j];
      const uint32_t neg = (uint32_t)((int32_t)(a16 << 16) >> 31);
      const uint32_t mag = (a16 & 0x7FFFu) * 0x10001u;
      // a set bit (+1) gives +|alpha| when alpha >= 0: invert the word, so
      // that the sign bit placed in the fp16 sign position is clear
      const uint64_t wd = (uint64_t)(~(w[i].y ^ neg)) << 32 | (uint32_t)(~(w[i].x ^ neg));
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        int sh = 15 - t;
        asm("" : "+s"(sh));  // one 64-bit shift for both words (see the decode in gemm_mfma.hip)
        const uint64_t m = wd << sh;
        const uint32_t lo = ((uint32_t)m & 0x80008000u) | mag;
        const uint32_t hi = ((uint32_t)(m >> 32) & 0x80008000u) | mag;
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, lo), xp(t), acc, false);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, hi), xp(16 + t), acc, false);
      }
    }
    const uint32_t z2 = (uint32_t)scl[P][r][j] * 0x10001u;
#pragma unroll
    for (int q = 0; q < 32; ++q) acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, z2), xp(q), acc, false);
  }

  // ---- the 64 slot partials of each row, then the wavefronts, fixed order
  acc = sum_rows4(acc, (lane ^ 32) << 2);
  if (lane < 16) part[wave][lane] = acc;
  __syncthreads();
  if (tid < kTileRows) {
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) sum += part[v][tid];
    const int mm = tile * kTileRows + tid;
    if (mm < M) y[mm] = (half_t)sum;
  }
}

bool gemv_direct_route() {
  const char *e = getenv("BCQ_B1_DIRECT");
  return e != nullptr && e[0] == '1';
}

// ------------------------------------------------ batch 1, K past the resident tables
//
// For fp32 stores with K > 4096 (and fp16 ones past K = 28672, or with the
// resident fp16 tables switched off) the fp32 tables of all of K do not fit in
// LDS, so a workgroup (one
// 16-row tile, 512 lanes, the lane mapping of gemv_res_kernel) streams K in
// windows of 16 groups with two table buffers and one barrier per window:
// after the barrier it builds window w+1's tables (one chunk per lane) and
// stages its scales into the other buffer, then looks up window w.  Sign
// words, activations and scales of window w+kStreamRing are requested when
// window w is done with its ring slot, so kStreamRing windows of loads are in
// flight; every path issues the same loads (a window past the end re-reads the
// last one) and the loop's only exit is its header, so the waits stay
// partial.  Two windows in flight measured faster than four at every
// streaming shape tried (p = 4: 4096x14336 16.1 -> 14.1 us, 4096x8192 11.6 ->
// 10.1, 14336x8192 39.4 -> 34.2, 12288x6144 23.4 -> 20.0); three, six and
// eight were slower than four.  Before the first build only the activations
// and scales of the first two windows and the first window's sign words are
// requested.  Scales are staged through LDS with row-contiguous loads, as in
// gemv_res_kernel.  A group's activation sum is kept as four 8-chunk partials
// (DPP within 8 lanes, no LDS round trips) that the lookup adds in order.
constexpr int kStreamRing = 2;  // windows of loads in flight

template <typename T, int P>
struct StreamSlot {
  uint2 bits[P];                   // this lane's half-group, one uint2 per plane
  typename Act<T>::raw x;          // the activations of the chunk this lane builds
  uint32_t sc[4];                  // four scales or offsets this lane stages
};

template <typename T, int P, bool GU = false>
__global__ __launch_bounds__(kRThreads) void gemv_stream_kernel(
    const uint4 *__restrict__ bits, const T *__restrict__ alpha, const T *__restrict__ zero,
    const T *__restrict__ x, T *__restrict__ y, int M, int G, int MT) {
  __shared__ __attribute__((aligned(16))) char lut[2][kRWindowBytes];
  __shared__ float gsum[2][kG1Ksub][4];
  // staged scales: [buffer][plane, then offsets][row][group of the window],
  // rows padded to 17 words so 16 rows x 2 groups hit distinct banks
  __shared__ uint32_t scl[2][P + 1][kTileRows][kG1Ksub + 1];
  __shared__ float part[kRWaves][kTileRows];
  using Slot = StreamSlot<T, P>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int hs = wave * 4 + (lane >> 4);  // half-group slot 0..31 of the window
  const int gw = hs >> 1;                 // group within the window
  const int half = hs & 1;
  const int tile = blockIdx.x;
  const int nwin = (G + kG1Ksub - 1) / kG1Ksub;
  const size_t plane_stride = (size_t)MT * G * kTileRows;  // in uint4
  const size_t MG = (size_t)M * G;
  const uint2 *bits2 = reinterpret_cast<const uint2 *>(bits);
  // staging task of this lane: array sa (planes, then offsets), row srow, groups 4*sq..+3
  const bool stager = tid < (P + 1) * kTileRows * 4;
  const int sa = min(tid / (kTileRows * 4), P);
  const int srow = (tid / 4) % kTileRows;
  const int sq = tid % 4;
  // scalar base of this wavefront's staging array (sa is the same for all 64
  // lanes) plus a 32-bit row offset within the tile
  const T *sbase = (sa < P ? alpha + (size_t)__builtin_amdgcn_readfirstlane(sa) * MG : zero) +
                   (size_t)tile * kTileRows * G +
                   (unsigned)(min(srow, M - 1 - tile * kTileRows) * G);

  auto fetch_bits = [&](int v, Slot &o) __attribute__((always_inline)) {
    const int w = min(v, nwin - 1);
    const int js = min(w * kG1Ksub + gw, G - 1);
    const unsigned lq = (unsigned)((js * kTileRows + r) * 2 + half);  // uint2 within the tile
    const uint2 *tb = bits2 + (size_t)tile * G * (kTileRows * 2);
#pragma unroll
    for (int i = 0; i < P; ++i) {
      const uint2 *pb = tb + (size_t)i * plane_stride * 2;
      o.bits[i] = pb[lq];
    }
  };
  auto fetch_small = [&](int v, Slot &o) __attribute__((always_inline)) {
    const int w = min(v, nwin - 1);
    const int c = tid % kChunksPerGroup;
    const int jx = min(w * kG1Ksub + tid / kChunksPerGroup, G - 1);
    o.x = Act<T>::load(x + (unsigned)(jx * kGroup + chunk_base(c)), chunk_parity(c));
#pragma unroll
    for (int e = 0; e < 4; ++e) o.sc[e] = load_raw(sbase + (unsigned)min(w * kG1Ksub + 4 * sq + e, G - 1));
  };
  auto fetch = [&](int v, Slot &o) __attribute__((always_inline)) {
    fetch_bits(v, o);
    fetch_small(v, o);
  };
  // tables, group sums and scales of the window held in slot o -> buffer buf
  auto build = [&](const Slot &o, int buf) __attribute__((always_inline)) {
    const int c = tid % kChunksPerGroup;
    float f[4];
    Act<T>::cvt(o.x, chunk_parity(c), f);
    float4 v[4];
    chunk_entries(f, v);
    float4 *dst = reinterpret_cast<float4 *>(lut[buf] + (tid / kChunksPerGroup) * kRGroupStride +
                                             r_chunk_offset(c));
    dst[0] = v[0];
    dst[1] = v[1];
    dst[2] = v[2];
    dst[3] = v[3];
    const float cs = sum8_lanes((f[0] + f[1]) + (f[2] + f[3]));
    if ((tid & 7) == 0) gsum[buf][tid / kChunksPerGroup][(tid / 8) % 4] = cs;
    if (stager) {
#pragma unroll
      for (int e = 0; e < 4; ++e) scl[buf][sa][srow][4 * sq + e] = o.sc[e];
    }
  };
  float acc = 0.f;
  auto consume = [&](int w, const Slot &o, int buf) __attribute__((always_inline)) {
    const int j = w * kG1Ksub + gw;
    if (j < G) {
      const uint32_t base = lds_addr(lut[buf] + gw * kRGroupStride + r_chunk_offset(16 * half));
#pragma unroll
      for (int i = 0; i < P; ++i)
        acc = fmaf(raw_to_float<T>(scl[buf][i][r][gw]), r_half_sum(o.bits[i], base), acc);
      if (half == 0) {
        const float *gs = gsum[buf][gw];
        acc = fmaf(raw_to_float<T>(scl[buf][P][r][gw]), (gs[0] + gs[1]) + (gs[2] + gs[3]), acc);
      }
    }
  };

  Slot ring[kStreamRing];
  fetch_small(0, ring[0]);
  fetch_small(1, ring[1]);
  fetch_bits(0, ring[0]);
  build(ring[0], 0);
  fetch_bits(1, ring[1]);
#pragma unroll
  for (int k = 2; k < kStreamRing; ++k) fetch(k, ring[k]);
  // window w: barrier (window w's tables are built; window w-1's lookups are
  // done with the other buffer), build w+1 there, look up w, refill w's slot
  for (int w0 = 0; w0 < nwin; w0 += kStreamRing) {
#pragma unroll
    for (int k = 0; k < kStreamRing; ++k) {
      const int w = w0 + k;
      __syncthreads();
      if (w + 1 < nwin) build(ring[(k + 1) % kStreamRing], (w + 1) & 1);  // uniform
      if (w < nwin) consume(w, ring[k], w & 1);                            // uniform
      fetch(w + kStreamRing, ring[k]);
    }
  }

  // ---- reduce the 32 slot partials of each row in a fixed order
  acc = sum_rows4(acc, (lane ^ 32) << 2);
  if (lane < 16) part[wave][lane] = acc;
  __syncthreads();
  if constexpr (GU) {
    if (tid < kGuRows) {
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int v = 0; v < kRWaves; ++v) {
        g += part[v][tid];
        u += part[v][tid + kGuRows];
      }
      const int jo = tile * kGuRows + tid;
      if (jo < M / 2) y[jo] = (T)gate_up_out(g, u);
    }
  } else if (tid < kTileRows) {
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < kRWaves; ++v) sum += part[v][tid];
    const int mm = tile * kTileRows + tid;
    if (mm < M) y[mm] = (T)sum;
  }
}

// 1024-lane variant for two or more planes.  Wavefronts 8..15 look up planes
// PA..P-1 (PA = ceil(P/2)) of the same half-group slots in the same tables,
// so a SIMD holds four wavefronts instead of two; wavefronts 0..7 build the
// tables, stage the scales and look up planes 0..PA-1 and the offset term.
// The halves run separate straight-line code, each issuing its own loads in a
// fixed order so that its waits stay partial, and meet at the same barriers.
template <typename T, int P>
struct StreamShared {
  __attribute__((aligned(16))) char lut[2][kRWindowBytes];
  float gsum[2][kG1Ksub][4];
  uint32_t scl[2][P + 1][kTileRows][kG1Ksub + 1];
  float part[2 * kRWaves][kTileRows];
};

template <typename T, int P, bool UPPER>
__device__ __forceinline__ void stream_half(StreamShared<T, P> &sm, const uint4 *__restrict__ bits,
                                            const T *__restrict__ alpha,
                                            const T *__restrict__ zero, const T *__restrict__ x,
                                            int M, int G, int MT, int tid) {
  constexpr int PA = (P + 1) / 2;
  constexpr int I0 = UPPER ? PA : 0;       // first plane of this half
  constexpr int NP = UPPER ? P - PA : PA;  // planes of this half
  const int lane = tid & 63;
  const int wave = tid >> 6;  // 0..7 within the half
  const int r = lane & 15;
  const int hs = wave * 4 + (lane >> 4);  // half-group slot 0..31 of the window
  const int gw = hs >> 1;
  const int half = hs & 1;
  const int tile = blockIdx.x;
  const int nwin = (G + kG1Ksub - 1) / kG1Ksub;
  const size_t plane_stride = (size_t)MT * G * kTileRows;  // in uint4
  const size_t MG = (size_t)M * G;
  const uint2 *bits2 = reinterpret_cast<const uint2 *>(bits);
  const bool stager = tid < (P + 1) * kTileRows * 4;
  const int sa = min(tid / (kTileRows * 4), P);
  const int srow = (tid / 4) % kTileRows;
  const int sq = tid % 4;
  // scalar base of this wavefront's staging array (sa is the same for all 64
  // lanes) plus a 32-bit row offset within the tile
  const T *sbase = (sa < P ? alpha + (size_t)__builtin_amdgcn_readfirstlane(sa) * MG : zero) +
                   (size_t)tile * kTileRows * G +
                   (unsigned)(min(srow, M - 1 - tile * kTileRows) * G);

  struct Slot {
    uint2 bits[NP];
    typename Act<T>::raw x;
    uint32_t sc[4];
  };
  auto fetch_bits = [&](int v, Slot &o) __attribute__((always_inline)) {
    const int w = min(v, nwin - 1);
    const int js = min(w * kG1Ksub + gw, G - 1);
    const unsigned lq = (unsigned)((js * kTileRows + r) * 2 + half);  // uint2 within the tile
    const uint2 *tb = bits2 + (size_t)tile * G * (kTileRows * 2);
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const uint2 *pb = tb + (size_t)(I0 + u) * plane_stride * 2;
      o.bits[u] = pb[lq];
    }
  };
  auto fetch_small = [&](int v, Slot &o) __attribute__((always_inline)) {
    if constexpr (!UPPER) {
      const int w = min(v, nwin - 1);
      const int c = tid % kChunksPerGroup;
      const int jx = min(w * kG1Ksub + tid / kChunksPerGroup, G - 1);
      o.x = Act<T>::load(x + (unsigned)(jx * kGroup + chunk_base(c)), chunk_parity(c));
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o.sc[e] = load_raw(sbase + (unsigned)min(w * kG1Ksub + 4 * sq + e, G - 1));
    }
  };
  auto fetch = [&](int v, Slot &o) __attribute__((always_inline)) {
    fetch_bits(v, o);
    fetch_small(v, o);
  };
  auto build = [&](const Slot &o, int buf) __attribute__((always_inline)) {
    if constexpr (!UPPER) {
      const int c = tid % kChunksPerGroup;
      float f[4];
      Act<T>::cvt(o.x, chunk_parity(c), f);
      float4 v[4];
      chunk_entries(f, v);
      float4 *dst = reinterpret_cast<float4 *>(sm.lut[buf] + (tid / kChunksPerGroup) * kRGroupStride +
                                               r_chunk_offset(c));
      dst[0] = v[0];
      dst[1] = v[1];
      dst[2] = v[2];
      dst[3] = v[3];
      const float cs = sum8_lanes((f[0] + f[1]) + (f[2] + f[3]));
      if ((tid & 7) == 0) sm.gsum[buf][tid / kChunksPerGroup][(tid / 8) % 4] = cs;
      if (stager) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.scl[buf][sa][srow][4 * sq + e] = o.sc[e];
      }
    }
  };
  float acc = 0.f;
  auto consume = [&](int w, const Slot &o, int buf) __attribute__((always_inline)) {
    const int j = w * kG1Ksub + gw;
    if (j < G) {
      const uint32_t base = lds_addr(sm.lut[buf] + gw * kRGroupStride + r_chunk_offset(16 * half));
#pragma unroll
      for (int u = 0; u < NP; ++u)
        acc = fmaf(raw_to_float<T>(sm.scl[buf][I0 + u][r][gw]), r_half_sum(o.bits[u], base), acc);
      if (!UPPER && half == 0) {
        const float *gs = sm.gsum[buf][gw];
        acc = fmaf(raw_to_float<T>(sm.scl[buf][P][r][gw]), (gs[0] + gs[1]) + (gs[2] + gs[3]), acc);
      }
    }
  };

  Slot ring[kStreamRing];
  fetch_small(0, ring[0]);
  fetch_small(1, ring[1]);
  fetch_bits(0, ring[0]);
  build(ring[0], 0);
  fetch_bits(1, ring[1]);
#pragma unroll
  for (int k = 2; k < kStreamRing; ++k) fetch(k, ring[k]);
  for (int w0 = 0; w0 < nwin; w0 += kStreamRing) {
#pragma unroll
    for (int k = 0; k < kStreamRing; ++k) {
      const int w = w0 + k;
      __syncthreads();
      if (w + 1 < nwin) build(ring[(k + 1) % kStreamRing], (w + 1) & 1);  // uniform
      if (w < nwin) consume(w, ring[k], w & 1);                            // uniform
      fetch(w + kStreamRing, ring[k]);
    }
  }
  acc = sum_rows4(acc, (lane ^ 32) << 2);
  if (lane < 16) sm.part[(UPPER ? kRWaves : 0) + wave][lane] = acc;
}

template <typename T, int P, bool GU = false>
__global__ __launch_bounds__(2 * kRThreads) void gemv_stream2_kernel(
    const uint4 *__restrict__ bits, const T *__restrict__ alpha, const T *__restrict__ zero,
    const T *__restrict__ x, T *__restrict__ y, int M, int G, int MT) {
  __shared__ StreamShared<T, P> sm;
  const int tid = threadIdx.x;
  if (tid < kRThreads)
    stream_half<T, P, false>(sm, bits, alpha, zero, x, M, G, MT, tid);
  else
    stream_half<T, P, true>(sm, bits, alpha, zero, x, M, G, MT, tid - kRThreads);
  // ---- reduce the 64 slot partials of each row in a fixed order
  __syncthreads();
  if constexpr (GU) {
    if (tid < kGuRows) {
      float g = 0.f, u = 0.f;
#pragma unroll
      for (int v = 0; v < 2 * kRWaves; ++v) {
        g += sm.part[v][tid];
        u += sm.part[v][tid + kGuRows];
      }
      const int jo = (int)blockIdx.x * kGuRows + tid;
      if (jo < M / 2) y[jo] = (T)gate_up_out(g, u);
    }
  } else if (tid < kTileRows) {
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < 2 * kRWaves; ++v) sum += sm.part[v][tid];
    const int mm = blockIdx.x * kTileRows + tid;
    if (mm < M) y[mm] = (T)sum;
  }
}

// ------------------------------------------------ batch 1, fp16 tables for K up to 28672
//
// For fp16 stores with 4096 < K <= 14336 the tables of all of K fit in LDS
// when each entry is held in fp16 (32 bytes per chunk; 126 KB of tables at
// K = 14336), so a workgroup builds them once, behind one barrier, instead of
// streaming windows through two buffers with a barrier each, and with more
// row tiles than compute units walks several tiles with them (gemv_h16_route
// has the measurements); up to K = 28672 it takes K in two passes of at most
// 14336 columns.  An entry is the fp32 sum of its four signed
// activations rounded once to fp16 (relative error at most 2^-11 of the
// entry); lookups are summed in fp32.
//
// 1024 lanes: lane (r, s) takes row r of the tile and half-group slots
// s, s + 64, s + 128, ... (s = wave * 4 + lane / 16); every thread builds
// chunks tid, tid + 1024, ... of K.  In LDS a group's 32 tables take 1152
// bytes (the second half of the group 64 bytes after the first), so the four
// slots of a wavefront, two groups x two halves, start in different quarters
// of the banks and each reads its own eight.
constexpr int kHThreads = 1024;
constexpr int kHWaves = kHThreads / 64;
constexpr int kHMaxG = 112;  // groups resident: K <= 14336
constexpr int kHChunkBytes = 2 * kEntries;
constexpr int kHHalfPad = 64;
constexpr int kHGroupStride = kChunksPerGroup * kHChunkBytes + kHHalfPad + 64;  // 1152

__device__ __forceinline__ int h_chunk_offset(int c) {
  return c * kHChunkBytes + (c >= 16 ? kHHalfPad : 0);
}

typedef __attribute__((address_space(3))) const _Float16 lds_half;
template <int B>
__device__ __forceinline__ _Float16 lds_h(uint32_t base, uint32_t v, int off) {
  return ((lds_half *)(size_t)add_byte<B>(base, v))[off];
}

// Sum over the 16 chunks of one half group of T_c[nibble] with fp16 tables:
// byte b of ev (od) is twice nibble 2b (2b + 1) of a packed word, the entry's
// byte offset in its chunk's table.  Each entry joins an fp32 sum through a
// mixed-precision multiply-add (fp16 entry times 1, v_fma_mix_f32), so a
// lookup costs one address add and one add, as with fp32 tables.
__device__ __forceinline__ float h_half_sum(const uint2 bw, uint32_t base) {
  constexpr int S = kHChunkBytes / 2;  // chunk stride in halves
  // 1.0 through an empty asm, so that entry * 1 + sum is not folded into a
  // conversion and an add
  float one = 1.f;
  asm("" : "+s"(one));
  const uint32_t wd[2] = {bw.x, bw.y};
  float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t ev = (wd[q] << 1) & 0x1E1E1E1Eu;
    const uint32_t od = (wd[q] >> 3) & 0x1E1E1E1Eu;
    const int c = q * 8;
    s[0] = fmaf((float)lds_h<0>(base, ev, (c + 0) * S), one, s[0]);
    s[1] = fmaf((float)lds_h<0>(base, od, (c + 1) * S), one, s[1]);
    s[2] = fmaf((float)lds_h<1>(base, ev, (c + 2) * S), one, s[2]);
    s[3] = fmaf((float)lds_h<1>(base, od, (c + 3) * S), one, s[3]);
    s[0] = fmaf((float)lds_h<2>(base, ev, (c + 4) * S), one, s[0]);
    s[1] = fmaf((float)lds_h<2>(base, od, (c + 5) * S), one, s[1]);
    s[2] = fmaf((float)lds_h<3>(base, ev, (c + 6) * S), one, s[2]);
    s[3] = fmaf((float)lds_h<3>(base, od, (c + 7) * S), one, s[3]);
  }
  return (s[0] + s[1]) + (s[2] + s[3]);
}

// The same sum in two parts, for a software pipeline over planes: the 16
// entries are read into registers first, then added in h_half_sum's order
// (so the result is the same).
__device__ __forceinline__ void h_half_read(const uint2 bw, uint32_t base, _Float16 (&e)[16]) {
  constexpr int S = kHChunkBytes / 2;
  const uint32_t wd[2] = {bw.x, bw.y};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t ev = (wd[q] << 1) & 0x1E1E1E1Eu;
    const uint32_t od = (wd[q] >> 3) & 0x1E1E1E1Eu;
    const int c = q * 8;
    e[c + 0] = lds_h<0>(base, ev, (c + 0) * S);
    e[c + 1] = lds_h<0>(base, od, (c + 1) * S);
    e[c + 2] = lds_h<1>(base, ev, (c + 2) * S);
    e[c + 3] = lds_h<1>(base, od, (c + 3) * S);
    e[c + 4] = lds_h<2>(base, ev, (c + 4) * S);
    e[c + 5] = lds_h<2>(base, od, (c + 5) * S);
    e[c + 6] = lds_h<3>(base, ev, (c + 6) * S);
    e[c + 7] = lds_h<3>(base, od, (c + 7) * S);
  }
}
__device__ __forceinline__ float h_half_add(const _Float16 (&e)[16]) {
  float one = 1.f;
  asm("" : "+s"(one));
  float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 16; ++c) s[c & 3] = fmaf((float)e[c], one, s[c & 3]);
  return (s[0] + s[1]) + (s[2] + s[3]);
}

// NG: groups of K the tables hold (32: K <= 4096, 64: K <= 8192, 112: K <=
// 14336).
// NB = 1: one tile per workgroup (grid = row tiles).  NB = 2: the workgroup
// walks tiles blockIdx.x + k * gridDim.x with the tables built once; the next
// tile's scales are staged into the other of two buffers during the current
// tile's lookups, and its sign words are requested one tile ahead, so each
// tile costs one barrier.
// RS > 1 (few row tiles, one per workgroup): RS workgroups share tile
// blockIdx.x / RS, each taking 16 / RS of its rows; lane (r, s) takes row
// r % (16 / RS) of that part and planes PC * (r / (16 / RS)) .. + PC - 1, as
// in gemv_res_kernel, so the lookups of a tile spread over RS compute units.
// MP (NG < G <= 2 NG, one tile per workgroup): K is walked in two passes with
// the tables of one pass resident; the second pass's activations, scales and
// sign words are requested during the first pass's lookups, and two barriers
// free the tables and publish the new ones.
template <int P, bool GU, int NG, int NB, int RS = 1, bool MP = false>
__global__ __launch_bounds__(kHThreads) void gemv_h16_kernel(
    const uint4 *__restrict__ bits, const half_t *__restrict__ alpha,
    const half_t *__restrict__ zero, const half_t *__restrict__ x, half_t *__restrict__ y, int M,
    int G, int MT) {
  static_assert(NG <= kHMaxG && (NB == 1 || NB == 2), "resident groups, scale buffers");
  static_assert(RS == 1 || (NB == 1 && !GU), "row parts: one tile per workgroup, plain products");
  static_assert(!MP || NB == 1, "passes over K: one tile per workgroup");
  constexpr int kPartRows = kTileRows / RS;
  constexpr int PC = (P + RS - 1) / RS;  // planes per lane
  constexpr int kRounds = (NG * kChunksPerGroup + kHThreads - 1) / kHThreads;
  constexpr int kSW = NG / 2 + 1;  // staged scale row in 32-bit words (odd)
  // staging: kSG threads per (array, row) run of G <= NG values
  constexpr int kSG = NG <= 64 ? 64 : 128;
  constexpr int kRuns = (P + 1) * kTileRows;
  constexpr int kRunsAtOnce = kHThreads / kSG;
  constexpr int kScalePerThread = (kRuns + kRunsAtOnce - 1) / kRunsAtOnce;
  constexpr int kSlots = (2 * NG + 63) / 64;  // half-group slots per lane
  __shared__ __attribute__((aligned(16))) char lut[NG * kHGroupStride];
  __shared__ float gsum[NG];
  __shared__ float part[NB][kHWaves][kTileRows];
  // staged scales and offsets as fp16 bits: [buffer][array][row][group], rows
  // at an odd number of words so the 16 rows a wavefront reads hit distinct
  // banks
  __shared__ uint32_t scl[NB][kRuns * kSW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15;
  const int s = wave * 4 + (lane >> 4);  // half-group slot 0..63
  const int rl = r % kPartRows;          // row within the part
  const int ph = r / kPartRows;          // plane part of this lane
  const int prow = RS > 1 ? ((int)blockIdx.x % RS) * kPartRows + rl : r;  // row within the tile
  const int G0 = MP ? NG : G;  // groups of the first pass (G <= NG without MP)
  const int nt = NB == 1 ? 1 : (MT - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const size_t plane_stride = (size_t)MT * G * kTileRows;  // in uint4
  const size_t MG = (size_t)M * G;
  const uint2 *bits2 = reinterpret_cast<const uint2 *>(bits);
  // tile k of this workgroup; past its last tile a load re-reads the last
  // one (lines already fetched), so the load phase stays branch-free
  auto tile_of = [&](int k) {
    return RS > 1 ? (int)blockIdx.x / RS : (int)blockIdx.x + min(k, nt - 1) * (int)gridDim.x;
  };

  // ---- activations of the chunks this thread builds in the pass of Gp
  // groups from group g0 (a past-the-end chunk re-reads the last one and
  // builds nothing)
  typename Act<half_t>::raw xr[kRounds];
  auto xload = [&](int g0, int Gp) {
    const int NCp = kChunksPerGroup * Gp;
#pragma unroll
    for (int t = 0; t < kRounds; ++t) {
      const int c = min(tid + kHThreads * t, NCp - 1);
      xr[t] = Act<half_t>::load(x + (unsigned)((g0 + c / kChunksPerGroup) * kGroup +
                                               chunk_base(c % kChunksPerGroup)),
                                0);
    }
  };
  xload(0, G0);

  // ---- scales and offsets of a tile: thread tid stages group tid % kSG of
  // runs tid / kSG + kRunsAtOnce * u (run = array * 16 + row; planes, then
  // offsets), so consecutive threads read consecutive groups of a row
  // (coalesced); a group or run past the end re-reads a valid value and
  // stages nothing
  const int sg = tid % kSG;
  unsigned short sv[kScalePerThread];
  auto sload = [&](int k, int g0, int Gp) {
    const int tl = tile_of(k);
    const int sgc = g0 + min(sg, Gp - 1);
#pragma unroll
    for (int u = 0; u < kScalePerThread; ++u) {
      const int run = min(tid / kSG + kRunsAtOnce * u, kRuns - 1);
      const int a = run / kTileRows;
      const int row = min(tl * kTileRows + run % kTileRows, M - 1);
      const half_t *src = (a < P ? alpha + (size_t)a * MG : zero) + (size_t)row * G + sgc;
      sv[u] = *reinterpret_cast<const unsigned short *>(src);
    }
  };
  auto sstore = [&](int b, int Gp) {
    unsigned short *s16 = reinterpret_cast<unsigned short *>(scl[b]);
#pragma unroll
    for (int u = 0; u < kScalePerThread; ++u) {
      const int run = tid / kSG + kRunsAtOnce * u;
      if (run < kRuns && sg < Gp) s16[run * kSW * 2 + sg] = sv[u];
    }
  };

  // ---- sign words of this lane's half groups in a tile, one uint2 per
  // plane it looks up, planes [u0, u1) of slot t (a slot past the last half
  // group re-reads the last one and adds nothing; so does a plane past P)
  uint2 wa[kSlots][PC], wb[kSlots][PC];
  auto wfetch = [&](int k, int t, uint2 (&w)[kSlots][PC], int g0, int Gp, int u0 = 0,
                    int u1 = P) {
    const int h = min(s + 64 * t, 2 * Gp - 1);
    const unsigned q =
        (unsigned)((((size_t)tile_of(k) * G + g0 + (h >> 1)) * kTileRows + prow) * 2 + (h & 1));
#pragma unroll
    for (int u = 0; u < PC; ++u) {
      const int i = RS > 1 ? min(ph * PC + u, P - 1) : u;
      if (u >= u0 && u < u1) w[t][u] = bits2[(size_t)i * plane_stride * 2 + q];
    }
  };

  // ---- first tile: scales, then only the first slot's sign words before the
  // table barrier.  The barrier waits for the activations; sign words
  // requested ahead of it queue in front of other workgroups' activation and
  // scale loads and hold every barrier back (4096x14336, p = 4: 14.7 us with
  // all slots requested first, 12.3 with one).  Two slots go first where a
  // slot carries few sign words (at most two planes per lane with the
  // 112-group tables, rows split four ways) and when a workgroup walks
  // several tiles; with the 64-group tables and one tile per workgroup a
  // short sleep precedes the first slot's words, as in gemv_res_kernel
  // (same-process A/B, six repeats: 1024x14336 p = 4 7.75 -> 7.02 us,
  // 4096x14336 p = 2 9.01 -> 8.59, 14336x8192 p = 3 18.62 -> 18.30,
  // 4096x8192 p = 4 8.14 -> 7.74; within 1% or slower elsewhere).
  // With one slot per lane (32 groups) and at least three planes, only the
  // first half of the slot's planes goes before the barrier and the rest
  // right after it, as in gemv_res_kernel.
  constexpr int kBefore = (RS == 4 || NB == 2 || (NG == 112 && PC <= 2)) ? 2 : 1;
  constexpr bool kSplitPlanes = kSlots == 1 && NB == 1 && RS == 1 && P >= 3;
  constexpr int kFirstPlanes = kSplitPlanes ? (PC + 1) / 2 : PC;
  // Lookups pipelined over planes (h_half_read / h_half_add) with the 64- and
  // 112-group tables; with 32 groups the compiler's own interleave was
  // faster.  Same-process A/B, six repeats, p = 2 / 3 / 4, us: 4096x14336
  // 8.50 / 10.42 / 12.36 -> 8.37 / 10.44 / 12.11, 4096x10240 7.28 / 8.64 /
  // 10.07 -> 7.18 / 8.64 / 9.85, 14336x8192 13.91 / 18.12 / 22.99 -> 13.42 /
  // 17.45 / 22.09; 4096x4096 4.26 / 4.59 / 5.07 -> 4.35 / 4.73 / 5.12.  Not
  // with 112 groups and several tiles per workgroup, where it spilled at p = 3.
  constexpr bool kPipe = NG > 32 && !(NG == 112 && NB == 2);
  sload(0, 0, G0);
  if constexpr (NG <= 64 && NB == 1 && RS == 1) __builtin_amdgcn_s_sleep(12);
#pragma unroll
  for (int t = 0; t < kSlots; ++t)
    if (t < kBefore) wfetch(0, t, wa, 0, G0, 0, kFirstPlanes);

  // ---- build the tables and group sums of a pass of Gp groups.  Every round
  // computes its chunk (a past-the-end one its clamped copy) and only the
  // stores are guarded: an activation load used only under the guard is sunk
  // below the sign words by the compiler, and its wait then covers all of them.
  auto build = [&](int Gp) {
    const int NCp = kChunksPerGroup * Gp;
#pragma unroll
    for (int t = 0; t < kRounds; ++t) {
      const int c = tid + kHThreads * t;
      const int cg = c % kChunksPerGroup;
      float f[4];
      Act<half_t>::cvt(xr[t], chunk_parity(cg), f);
      float4 v[4];
      chunk_entries(f, v);
      // entries rounded to fp16 in pairs (one packed conversion each)
      typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
      uint32_t hv[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hv[2 * e] = __builtin_bit_cast(uint32_t, h2_t{(_Float16)v[e].x, (_Float16)v[e].y});
        hv[2 * e + 1] = __builtin_bit_cast(uint32_t, h2_t{(_Float16)v[e].z, (_Float16)v[e].w});
      }
      const float cs = sum32_lanes((f[0] + f[1]) + (f[2] + f[3]));
      if (c < NCp) {  // whole aligned 32-lane blocks (NCp is a multiple of 32)
        uint4 *dst = reinterpret_cast<uint4 *>(lut + (c / kChunksPerGroup) * kHGroupStride +
                                               h_chunk_offset(cg));
        dst[0] = make_uint4(hv[0], hv[1], hv[2], hv[3]);
        dst[1] = make_uint4(hv[4], hv[5], hv[6], hv[7]);
        if ((tid & 31) == 0) gsum[c / kChunksPerGroup] = cs;
      }
    }
  };
  build(G0);
  sstore(0, G0);
  __syncthreads();
#pragma unroll
  for (int t = kBefore; t < kSlots; ++t) wfetch(0, t, wa, 0, G0);
  if constexpr (kSplitPlanes) wfetch(0, 0, wa, 0, G0, kFirstPlanes, PC);

  // ---- lookups of slot t in a pass of Gp groups of one tile, scales from
  // buffer b, added to this lane's partial acc
  auto lookup_slot = [&](int b, const uint2 (&w)[kSlots][PC], int Gp, int t, float acc) -> float {
    const unsigned short *s16 = reinterpret_cast<const unsigned short *>(scl[b]);
    auto scale = [&](int a, int j) -> float {
      return (float)__builtin_bit_cast(half_t, s16[((a * kTileRows + prow) * kSW) * 2 + j]);
    };
    {
      const int h = s + 64 * t;
      if (h < 2 * Gp) {
        const int j = h >> 1, half = h & 1;
        const uint32_t base = lds_addr(lut + j * kHGroupStride + h_chunk_offset(16 * half));
        // a plane index past P (P not a multiple of RS) looks up with scale 0
        auto plane_scale = [&](int u) -> float {
          const int i = RS > 1 ? ph * PC + u : u;
          return i < P ? scale(min(i, P - 1), j) : 0.f;
        };
        if constexpr (kPipe) {
          // plane u + 1's 16 entries are requested before plane u's are
          // added, so each wavefront keeps up to 16 table reads in flight
          float sc[PC];
#pragma unroll
          for (int u = 0; u < PC; ++u) sc[u] = plane_scale(u);
          _Float16 eb[2][16];
          h_half_read(w[t][0], base, eb[0]);
#pragma unroll
          for (int u = 0; u < PC; ++u) {
            if (u + 1 < PC) h_half_read(w[t][u + 1], base, eb[(u + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            acc = fmaf(sc[u], h_half_add(eb[u & 1]), acc);
          }
        } else {
#pragma unroll
          for (int u = 0; u < PC; ++u) acc = fmaf(plane_scale(u), h_half_sum(w[t][u], base), acc);
        }
        if (half == 0 && (RS == 1 || ph == 0)) acc = fmaf(scale(P, j), gsum[j], acc);
      }
    }
    return acc;
  };
  auto lookups = [&](int b, const uint2 (&w)[kSlots][PC], int Gp) -> float {
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < kSlots; ++t) acc = lookup_slot(b, w, Gp, t, acc);
    return acc;
  };
  // the 64 slot partials of each row, reduced in a fixed order; then the
  // plane parts, lanes r, r + 16/RS, .. of the 16-lane row (DPP row_ror)
  auto reduce_rows = [&](float acc) -> float {
    acc = sum_rows4(acc, (lane ^ 32) << 2);
    if constexpr (RS == 4)
      acc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, acc), 0x124,
                                                                0xF, 0xF, true));
    if constexpr (RS >= 2)
      acc += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, acc), 0x128,
                                                                0xF, 0xF, true));
    return acc;
  };
  // ---- the 16 wavefront partials of each row of tile k, in a fixed order
  auto finish = [&](int k, int b) {
    const int tl = tile_of(k);
    if constexpr (GU) {
      if (tid < kGuRows) {
        float g = 0.f, u = 0.f;
#pragma unroll
        for (int v = 0; v < kHWaves; ++v) {
          g += part[b][v][tid];
          u += part[b][v][tid + kGuRows];
        }
        const int jo = tl * kGuRows + tid;
        if (jo < M / 2) y[jo] = (half_t)gate_up_out(g, u);
      }
    } else if (tid < kPartRows) {
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < kHWaves; ++v) sum += part[b][v][tid];
      const int mm = tl * kTileRows + (RS > 1 ? ((int)blockIdx.x % RS) * kPartRows : 0) + tid;
      if (mm < M) y[mm] = (half_t)sum;
    }
  };

  if constexpr (NB == 1) {
    float acc;
    if constexpr (MP) {
      // two passes (NG < G <= 2 NG), straight-line: the second pass's
      // activations and scales are requested as the first starts, and each
      // slot's sign words for it as soon as the slot has been looked up (one
      // register set).  (As a loop over passes the compiler's waits for these
      // loop-carried loads degraded to full drains.)
      const int G1 = G - NG;
      xload(NG, G1);
      sload(0, NG, G1);
      acc = 0.f;
#pragma unroll
      for (int t = 0; t < kSlots; ++t) {
        acc = lookup_slot(0, wa, NG, t, acc);
        wfetch(0, t, wa, NG, G1);
      }
      __syncthreads();  // every lookup of the first pass done: tables and scales free
      sstore(0, G1);    // first, so its registers are free during the build
      build(G1);
      __syncthreads();
#pragma unroll
      for (int t = 0; t < kSlots; ++t) acc = lookup_slot(0, wa, G1, t, acc);
    } else {
      acc = lookups(0, wa, G0);
    }
    acc = reduce_rows(acc);
    if (lane < 16) part[0][wave][lane] = acc;
    __syncthreads();
    finish(0, 0);
  } else {
    // tile k: request tile k + 1's scales and sign words, look up tile k,
    // stage tile k + 1's scales into the other buffer (its last readers, tile
    // k - 1's lookups, finished before the previous barrier), then one
    // barrier before tile k's rows are summed
    auto step = [&](int k, const uint2 (&wc)[kSlots][PC], uint2 (&wn)[kSlots][PC]) {
      const int b = k & 1;
      sload(k + 1, 0, G);
#pragma unroll
      for (int t = 0; t < kSlots; ++t) wfetch(k + 1, t, wn, 0, G);
      const float acc = reduce_rows(lookups(b, wc, G));
      if (lane < 16) part[b][wave][lane] = acc;
      sstore(b ^ 1, G);
      __syncthreads();
      finish(k, b);
    };
    for (int k = 0; k < nt; k += 2) {
      step(k, wa, wb);
      if (k + 1 < nt) step(k + 1, wb, wa);
    }
  }
}

// Compute units of the current device, cached per device (atomics: calls may
// come from several host threads).  Only the grid size depends on it.
int compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int v = 0;
    n = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0
            ? v
            : 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <typename T, int NW, int TMAX, int RS = 1, bool GU = false, bool LR = false>
void gemv_res_launch(dim3 grid, hipStream_t s, const uint4 *b4, const T *a, const T *z,
                     const T *xx, T *yy, int M, int G, int MT, int p, const uint32_t *lu,
                     const float *lz, int R) {
  switch (p) {
    case 1:
      hipLaunchKernelGGL((gemv_res_kernel<T, NW, 1, TMAX, RS, GU, LR>), grid, dim3(kRThreads * NW),
                         0, s, b4, a, z, xx, yy, M, G, MT, lu, lz, R);
      break;
    case 2:
      hipLaunchKernelGGL((gemv_res_kernel<T, NW, 2, TMAX, RS, GU, LR>), grid, dim3(kRThreads * NW),
                         0, s, b4, a, z, xx, yy, M, G, MT, lu, lz, R);
      break;
    case 3:
      hipLaunchKernelGGL((gemv_res_kernel<T, NW, 3, TMAX, RS, GU, LR>), grid, dim3(kRThreads * NW),
                         0, s, b4, a, z, xx, yy, M, G, MT, lu, lz, R);
      break;
    default:
      hipLaunchKernelGGL((gemv_res_kernel<T, NW, 4, TMAX, RS, GU, LR>), grid, dim3(kRThreads * NW),
                         0, s, b4, a, z, xx, yy, M, G, MT, lu, lz, R);
      break;
  }
}

// At most one tile per compute unit: with a quarter (half) of the compute
// units or fewer holding a tile, each tile's rows are split over 4 (2)
// workgroups.  More tiles than compute units: tiles dealt round-robin, up to 4
// per workgroup, and for fp16 stores up to 8 (their scales staged in 16-bit
// slots leave room for eight tiles'), so that up to 8 tiles per compute unit
// take one round of workgroups, each building its tables once (measured
// 20000x4096: 20.1 -> 15.0 us at p = 4; 28672x4096: 21.1 -> 18.0 us).
template <typename T, int NW, bool GU, bool LR = false>
void gemv_res_tiles(hipStream_t s, const uint4 *b4, const T *a, const T *z, const T *xx, T *yy,
                    int M, int G, int MT, int p, const uint32_t *lu = nullptr,
                    const float *lz = nullptr, int R = 0) {
  const int cus = compute_units();
  const int tmax = (MT + cus - 1) / cus;
  if (!GU && 4 * MT <= cus)
    gemv_res_launch<T, NW, 1, 4, false, LR>(dim3(MT * 4), s, b4, a, z, xx, yy, M, G, MT, p, lu,
                                            lz, R);
  else if (!GU && 2 * MT <= cus)
    gemv_res_launch<T, NW, 1, 2, false, LR>(dim3(MT * 2), s, b4, a, z, xx, yy, M, G, MT, p, lu,
                                            lz, R);
  else if (tmax <= 1)
    gemv_res_launch<T, NW, 1, 1, GU, LR>(dim3(MT), s, b4, a, z, xx, yy, M, G, MT, p, lu, lz, R);
  else if (tmax <= 2)
    gemv_res_launch<T, NW, 2, 1, GU, LR>(dim3((MT + 1) / 2), s, b4, a, z, xx, yy, M, G, MT, p, lu,
                                         lz, R);
  else if (sizeof(T) != 2 || tmax <= 4)
    gemv_res_launch<T, NW, 4, 1, GU, LR>(dim3((MT + 3) / 4 > cus ? (MT + 3) / 4 : cus), s, b4, a,
                                         z, xx, yy, M, G, MT, p, lu, lz, R);
  else if constexpr (sizeof(T) == 2)  // eight tiles' fp16 scales fit in LDS, fp32 ones do not
    gemv_res_launch<T, NW, 8, 1, GU, LR>(dim3((MT + 7) / 8 > cus ? (MT + 7) / 8 : cus), s, b4, a,
                                         z, xx, yy, M, G, MT, p, lu, lz, R);
}

// Product plus fused low-rank correction, resident tables only (K <= 4096).
template <typename T>
hipError_t gemv_lowrank_dispatch(const uint32_t *bits, int M, int K, int p, const void *alpha,
                                 const void *zero, const void *x, void *y, const uint32_t *u,
                                 const float *z, int R, hipStream_t s) {
  const int G = K / kGroup;
  const int MT = row_tiles(M);
  const uint4 *b4 = reinterpret_cast<const uint4 *>(bits);
  const T *a = static_cast<const T *>(alpha);
  const T *zz = static_cast<const T *>(zero);
  const T *xx = static_cast<const T *>(x);
  T *yy = static_cast<T *>(y);
  if (G <= kG1Ksub)
    gemv_res_tiles<T, 1, false, true>(s, b4, a, zz, xx, yy, M, G, MT, p, u, z, R);
  else
    gemv_res_tiles<T, 2, false, true>(s, b4, a, zz, xx, yy, M, G, MT, p, u, z, R);
  return hipGetLastError();
}

template <int P, bool GU, int NG>
void gemv_h16_tiles(hipStream_t s, const uint4 *b4, const half_t *a, const half_t *z,
                    const half_t *xx, half_t *yy, int M, int G, int MT) {
  // more row tiles than compute units: one workgroup per unit walks several
  // tiles with the tables built once (two scale buffers; at K > 8192, p = 4
  // they do not fit beside the tables, and every tile takes a workgroup).
  // At most a quarter (a half) of the units holding a tile: each tile's rows
  // split over 4 (2) workgroups.
  const int cus = compute_units();
  if constexpr (!GU) {
    if (4 * MT <= cus) {
      hipLaunchKernelGGL((gemv_h16_kernel<P, GU, NG, 1, 4>), dim3(4 * MT), dim3(kHThreads), 0, s, b4,
                         a, z, xx, yy, M, G, MT);
      return;
    }
    if (2 * MT <= cus) {
      hipLaunchKernelGGL((gemv_h16_kernel<P, GU, NG, 1, 2>), dim3(2 * MT), dim3(kHThreads), 0, s, b4,
                         a, z, xx, yy, M, G, MT);
      return;
    }
  }
  if constexpr (NG == 64 || P <= 3) {
    if (MT > cus) {
      hipLaunchKernelGGL((gemv_h16_kernel<P, GU, NG, 2>), dim3(cus), dim3(kHThreads), 0, s, b4, a,
                         z, xx, yy, M, G, MT);
      return;
    }
  }
  hipLaunchKernelGGL((gemv_h16_kernel<P, GU, NG, 1>), dim3(MT), dim3(kHThreads), 0, s, b4, a, z,
                     xx, yy, M, G, MT);
}

// K past 112 groups, up to 224: one tile per workgroup (rows split when few
// tiles), K walked in two passes of at most 112 groups.
template <int P, bool GU>
void gemv_h16_passes(hipStream_t s, const uint4 *b4, const half_t *a, const half_t *z,
                     const half_t *xx, half_t *yy, int M, int G, int MT) {
  const int cus = compute_units();
  if constexpr (!GU) {
    if (4 * MT <= cus) {
      hipLaunchKernelGGL((gemv_h16_kernel<P, GU, kHMaxG, 1, 4, true>), dim3(4 * MT), dim3(kHThreads),
                         0, s, b4, a, z, xx, yy, M, G, MT);
      return;
    }
    if (2 * MT <= cus) {
      hipLaunchKernelGGL((gemv_h16_kernel<P, GU, kHMaxG, 1, 2, true>), dim3(2 * MT), dim3(kHThreads),
                         0, s, b4, a, z, xx, yy, M, G, MT);
      return;
    }
  }
  hipLaunchKernelGGL((gemv_h16_kernel<P, GU, kHMaxG, 1, 1, true>), dim3(MT), dim3(kHThreads), 0, s,
                     b4, a, z, xx, yy, M, G, MT);
}

template <bool GU>
void gemv_h16_launch(hipStream_t s, const uint4 *b4, const half_t *a, const half_t *z,
                     const half_t *xx, half_t *yy, int M, int G, int MT, int p) {
  if (G > kHMaxG) {  // the caller routes at most 2 * kHMaxG groups here
    switch (p) {
      case 1: gemv_h16_passes<1, GU>(s, b4, a, z, xx, yy, M, G, MT); break;
      case 2: gemv_h16_passes<2, GU>(s, b4, a, z, xx, yy, M, G, MT); break;
      case 3: gemv_h16_passes<3, GU>(s, b4, a, z, xx, yy, M, G, MT); break;
      default: gemv_h16_passes<4, GU>(s, b4, a, z, xx, yy, M, G, MT); break;
    }
    return;
  }
  if (G <= 64) {
    switch (p) {
      case 1: gemv_h16_tiles<1, GU, 64>(s, b4, a, z, xx, yy, M, G, MT); break;
      case 2: gemv_h16_tiles<2, GU, 64>(s, b4, a, z, xx, yy, M, G, MT); break;
      case 3: gemv_h16_tiles<3, GU, 64>(s, b4, a, z, xx, yy, M, G, MT); break;
      default: gemv_h16_tiles<4, GU, 64>(s, b4, a, z, xx, yy, M, G, MT); break;
    }
  } else {
    switch (p) {
      case 1: gemv_h16_tiles<1, GU, kHMaxG>(s, b4, a, z, xx, yy, M, G, MT); break;
      case 2: gemv_h16_tiles<2, GU, kHMaxG>(s, b4, a, z, xx, yy, M, G, MT); break;
      case 3: gemv_h16_tiles<3, GU, kHMaxG>(s, b4, a, z, xx, yy, M, G, MT); break;
      default: gemv_h16_tiles<4, GU, kHMaxG>(s, b4, a, z, xx, yy, M, G, MT); break;
    }
  }
}

// Batch 1, fp16, 4096 < K <= 28672: resident fp16 tables (gemv_h16_kernel,
// in two passes past K = 14336) or streamed fp32 windows (gemv_stream*_kernel).
// Measured same-run at p = 2..4 over 16 shapes from 256x12288 to 28672x8192
// (K = 4224 to 14336), the resident tables won everywhere: by 4-30% with few
// row tiles and by up to 2x with many (28672x5120, p = 2: 16.9 against 33.6
// us); in two passes over six shapes with K = 16384 to 28672, by 3-44%
// (4096x28672: 14.9 / 18.6 / 22.0 against 20.1 / 23.4 / 23.9 us at
// p = 2 / 3 / 4).  BCQ_H16=0 forces the stream (A/B runs and tests); BCQ_H16=1
// the resident tables.
// fp16 stores with 2048 < K <= 4096: the fp16 tables (32 groups, one slot
// per lane, the first half of the planes requested before the table barrier)
// against gemv_res_kernel's fp32 tables, same-process A/B, six repeats, us at
// p = 2 / 3 / 4: 4096x4096 4.56 / 4.63 / 5.38 -> 4.23 / 4.62 / 5.13,
// 4096x3072 4.39 / 4.39 / 5.10 -> 4.11 / 4.34 / 4.80 with one tile per
// workgroup; with several tiles per workgroup (8192x4096 to 28672x4096) or
// rows split over workgroups (1024x4096, 2048x4096) the fp32 tables were
// 3-18% faster.  So the fp16 tables take exactly the launches of one tile per
// workgroup on more than half of the compute units.
bool gemv_h16_small_route(int MT) {
  const int cus = compute_units();
  return MT <= cus && 2 * MT > cus;
}

bool gemv_h16_route(int G, int p) {
  (void)G;
  (void)p;
  const char *e = getenv("BCQ_H16");
  return !(e != nullptr && e[0] == '0');
}

template <typename T, bool GU>
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
  if (nwin <= 1) {
    gemv_res_tiles<T, 1, GU>(s, b4, a, z, xx, yy, M, G, MT, p);
    return hipGetLastError();
  }
  if constexpr (sizeof(T) == 2 && !GU) {
    if (nwin <= 2 && gemv_direct_route()) {  // direct add/subtract, measured against the tables
      switch (p) {
        case 1:
          hipLaunchKernelGGL(gemv_direct_kernel<1>, dim3(MT), dim3(2 * kRThreads), 0, s, b4, a, z, xx,
                             yy, M, G, MT);
          break;
        case 2:
          hipLaunchKernelGGL(gemv_direct_kernel<2>, dim3(MT), dim3(2 * kRThreads), 0, s, b4, a, z, xx,
                             yy, M, G, MT);
          break;
        case 3:
          hipLaunchKernelGGL(gemv_direct_kernel<3>, dim3(MT), dim3(2 * kRThreads), 0, s, b4, a, z, xx,
                             yy, M, G, MT);
          break;
        default:
          hipLaunchKernelGGL(gemv_direct_kernel<4>, dim3(MT), dim3(2 * kRThreads), 0, s, b4, a, z, xx,
                             yy, M, G, MT);
          break;
      }
      return hipGetLastError();
    }
    // 2048 < K <= 4096 with one row tile per workgroup and every compute unit
    // busy: fp16 tables of all of K (gemv_h16_small_route)
    if (nwin == 2 && gemv_h16_small_route(MT) && gemv_h16_route(G, p)) {
      switch (p) {
        case 1:
          hipLaunchKernelGGL((gemv_h16_kernel<1, false, 32, 1>), dim3(MT), dim3(kHThreads), 0, s, b4,
                             a, z, xx, yy, M, G, MT);
          break;
        case 2:
          hipLaunchKernelGGL((gemv_h16_kernel<2, false, 32, 1>), dim3(MT), dim3(kHThreads), 0, s, b4,
                             a, z, xx, yy, M, G, MT);
          break;
        case 3:
          hipLaunchKernelGGL((gemv_h16_kernel<3, false, 32, 1>), dim3(MT), dim3(kHThreads), 0, s, b4,
                             a, z, xx, yy, M, G, MT);
          break;
        default:
          hipLaunchKernelGGL((gemv_h16_kernel<4, false, 32, 1>), dim3(MT), dim3(kHThreads), 0, s, b4,
                             a, z, xx, yy, M, G, MT);
          break;
      }
      return hipGetLastError();
    }
  }
  if (nwin <= 2) {
    gemv_res_tiles<T, 2, GU>(s, b4, a, z, xx, yy, M, G, MT, p);
    return hipGetLastError();
  }
  if constexpr (sizeof(T) == 2) {
    // fp16: tables resident as fp16, of all of K up to K = 14336 and in two
    // passes up to K = 28672 (gemv_h16_route)
    if (G <= 2 * kHMaxG && gemv_h16_route(G, p)) {
      gemv_h16_launch<GU>(s, b4, a, z, xx, yy, M, G, MT, p);
      return hipGetLastError();
    }
  }
  // larger K: one tile per workgroup, tables streamed window by window
  dim3 grid(MT), block(kRThreads), block2(2 * kRThreads);
  switch (p) {
    case 1:
      hipLaunchKernelGGL((gemv_stream_kernel<T, 1, GU>), grid, block, 0, s, b4, a, z, xx, yy, M, G, MT);
      break;
    case 2:
      hipLaunchKernelGGL((gemv_stream2_kernel<T, 2, GU>), grid, block2, 0, s, b4, a, z, xx, yy, M, G,
                         MT);
      break;
    case 3:
      hipLaunchKernelGGL((gemv_stream2_kernel<T, 3, GU>), grid, block2, 0, s, b4, a, z, xx, yy, M, G,
                         MT);
      break;
    default:
      hipLaunchKernelGGL((gemv_stream2_kernel<T, 4, GU>), grid, block2, 0, s, b4, a, z, xx, yy, M, G,
                         MT);
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- batches of 2..8
//
// A workgroup of four wavefronts owns a tile of 16 rows and walks K in
// windows of 4 groups; wavefront v handles group v of the window.  Lane
// (r, k, c) takes row r, plane 2u + k of each plane pair u, and the 64-column
// half c of the group (two 32-bit sign words per plane).  Table entries hold
// the sums of up to 4 requests side by side, so one lookup address serves
// every request of the launch.
//
// Why planes and not column quarters across the lanes: a 16-byte LDS read is
// conflict-free only when the 32 lanes of each half-wavefront read within one
// 256-byte table (measured on gfx950: four tables per wavefront cost 46% bank
// conflicts and 1.85x the cycles per read).  Lanes of a half-wavefront here
// share the column half, so at every lookup they read the same chunk's table,
// two planes x 16 rows at random entries.
//
// Per-request precision (AnyBCQ paper notes, per-request precision; the
// abstract's negligible-overhead selection): planes up to the largest
// precision are read once for all requests, and a request whose precision is
// lower gets a zero scale for the planes it does not use.  Scales are staged
// per window through LDS: each distinct [M][G] array of the launch (a plane
// of alpha[p], or zero[p]) is loaded once and written into the slots of the
// requests that read it; slots that nothing writes stay zero from the start.
//
// The offset term z * S_j is split over the four lanes of a row: each adds z
// times one quarter's activation sum, so no lane needs a branch (the four
// quarter terms sum to z * S_j).  With an odd largest precision the last pair
// has one plane; its other lanes read a clamped plane and a zero scale.

constexpr int kSkThreads = 256;
constexpr int kSkGroups = 4;                                // groups per window
constexpr int kSkChunks = kSkGroups * kChunksPerGroup;      // 128 tables per window
constexpr int kSkQuarters = kGroup / 32;                    // 32-column quarters per group
constexpr int kSkConcurrent = 2;                            // windows in flight per workgroup
constexpr int kSkDepth = 2;                                 // operand sets in the prefetch ring

// Table geometry for NB requests.  An entry holds up to 4 requests' fp32 sums
// side by side; with 8 requests a chunk holds two 16-entry halves, so the
// byte offset of an entry is nibble * entry_bytes and always fits the
// byte-select add.  The chunk stride staggers consecutive chunks over the LDS
// banks for the writes of the build.
template <int NB>
struct SkGeom {
  static constexpr int per_entry = NB < 4 ? NB : 4;              // requests per entry
  static constexpr int entry_bytes = per_entry * 4;              // 8 or 16
  static constexpr int half_bytes = kEntries * entry_bytes;      // 128 or 256
  static constexpr int halves = NB / per_entry;                  // 1 or 2
  static constexpr int chunk_stride = halves * half_bytes + (NB == 2 ? 8 : 16);
  static constexpr int group_stride = kChunksPerGroup * chunk_stride;
  static constexpr int lut_bytes = kSkGroups * group_stride;
  static constexpr int rpt = NB / 2;                             // requests built per thread
};

template <int NB>
__device__ __forceinline__ void sk_read(uint32_t addr, float *v) {
  if constexpr (NB == 2) {
    const f32x2 a = *(lds_float2 *)(size_t)addr;
    v[0] = a.x;
    v[1] = a.y;
  } else {
#pragma unroll
    for (int h = 0; h < NB / 4; ++h) {
      const f32x4 a = *(lds_float4 *)(size_t)(addr + h * SkGeom<NB>::half_bytes);
      v[4 * h + 0] = a.x;
      v[4 * h + 1] = a.y;
      v[4 * h + 2] = a.z;
      v[4 * h + 3] = a.w;
    }
  }
}

// The table entries of one 32-column quarter: t[c] = T_c[nibble c] for its 8
// chunks c, all requests.  base is the LDS byte offset of the quarter's first
// table.  All 8 reads are issued before any is used.
template <int NB>
__device__ __forceinline__ void sk_quarter_reads(uint32_t wd, uint32_t base, float (&t)[8][NB]) {
  using Gm = SkGeom<NB>;
  uint32_t ev, od;  // nibble * entry_bytes, one per byte (even nibbles, odd nibbles)
  if constexpr (Gm::entry_bytes == 8) {
    ev = (wd << 3) & 0x78787878u;
    od = (wd >> 1) & 0x78787878u;
  } else {
    ev = (wd << 4) & 0xF0F0F0F0u;
    od = wd & 0xF0F0F0F0u;
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t v = e ? od : ev;
      uint32_t a;
      if (b == 0) a = add_byte<0>(base, v);
      else if (b == 1) a = add_byte<1>(base, v);
      else if (b == 2) a = add_byte<2>(base, v);
      else a = add_byte<3>(base, v);
      sk_read<NB>(a + (2 * b + e) * Gm::chunk_stride, t[2 * b + e]);
    }
  }
}

// Per-request plane sums over the quarter, in a fixed pairwise order.
template <int NB>
__device__ __forceinline__ float sk_quarter_sum(const float (&t)[8][NB], int q) {
  return ((t[0][q] + t[1][q]) + (t[2][q] + t[3][q])) + ((t[4][q] + t[5][q]) + (t[6][q] + t[7][q]));
}

// Operands of one window, double-buffered across the window loop.
template <typename T, int NB, int P, int UMAX>
struct SkOperands {
  uint2 bits[(P + 1) / 2];                    // this lane's two sign words, per plane pair
  typename Act<T>::raw x[SkGeom<NB>::rpt];    // the chunk this thread builds, per request
  uint32_t sc[UMAX];                          // staged scale values (raw)
};

// P is the largest precision of the launch; UMAX * 4 >= the number of staged
// arrays.  NH windows are processed at once, each by its own 256-lane half of
// the workgroup with its own tables, so every step has NH windows of work to
// cover the loads of the next step.  The load phase has no branches: windows
// past the end, groups past G, rows past M and requests past nreq read clamped
// in-range addresses whose values are never used.
template <typename T, int NB, int P, int UMAX, int NH, bool UNI>
__global__ __launch_bounds__(kSkThreads * NH) __attribute__((amdgpu_waves_per_eu(1, 2))) void
skinny_lut_kernel(const uint32_t *__restrict__ bits, ReqTables st, int nreq,
                  const T *__restrict__ x, int ldx, T *__restrict__ y, int ldy, int M, int G,
                  int MT) {
  using Gm = SkGeom<NB>;
  using Ops = SkOperands<T, NB, P, UMAX>;
  constexpr int kPairs = (P + 1) / 2;
  constexpr int kZSlot = sk_zero_slot(P);  // plane slots (an even number), then offsets
  constexpr int kSlots = kZSlot + 1;
  // With one precision for every request (UNI) all requests share one scale
  // per (row, group, plane): one float per record.  Otherwise each request
  // has its own slot, per_entry requests side by side in a record.
  constexpr int kQB = UNI ? 1 : Gm::halves;         // request blocks
  constexpr int kSR = UNI ? 4 : Gm::entry_bytes;    // bytes of one (slot, block, row) record
  constexpr int kStageBytes = kSkGroups * kSlots * kQB * kTileRows * kSR;
  constexpr int kWaves = kSkGroups * NH;
  __shared__ __attribute__((aligned(16))) char lut_all[NH][Gm::lut_bytes];
  __shared__ __attribute__((aligned(16))) char stage_all[NH][kStageBytes];
  __shared__ __attribute__((aligned(16))) float qsum_all[NH][kSkGroups][kSkQuarters][NB];
  static_assert(kWaves * kTileRows * NB * 4 <= Gm::lut_bytes, "partials fit the tables");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave / kSkGroups;      // which of the NH concurrent windows
  const int wl = wave % kSkGroups;        // group of the window
  const int tl = tid % kSkThreads;        // thread within the half
  char *lut = lut_all[half];
  char *stage = stage_all[half];
  float(*qsum)[kSkQuarters][NB] = qsum_all[half];
  const int r = lane & 15;         // row of the tile (lookups and staging)
  const int k = (lane >> 4) & 1;   // plane within a pair (lookups)
  const int c = lane >> 5;         // 64-column half of the group (lookups)
  const int h = lane >> 4;         // group of the window (staging)
  const int tile = blockIdx.x;
  const int nwin = (G + kSkGroups - 1) / kSkGroups;
  const int nstep = (nwin + NH - 1) / NH;
  const size_t plane_words = (size_t)MT * G * kTileRows * 4;
  const uint2 *tb = reinterpret_cast<const uint2 *>(bits + ((size_t)tile * G * kTileRows + r) * 4) + c;
  // build role: chunk bc of the window, requests q0 .. q0 + rpt - 1.  Lane bits
  // 3 and 4 are swapped in the chunk index so that the 16-byte table writes of
  // lanes l and l + 16 (serviced together) land 32 banks apart.
  const int bc = ((tl & 0x67) | ((tl & 8) << 1) | ((tl & 16) >> 1)) & (kSkChunks - 1);
  const int bg = bc / kChunksPerGroup;
  const int bcl = bc % kChunksPerGroup;
  const int q0 = (tl / kSkChunks) * Gm::rpt;
  // staging role: row r, window group h, arrays wl + 4u (their descriptors are
  // wave-uniform and read once, before the loop)
  const int srow = min(tile * kTileRows + r, M - 1);
  const T *sptr[UMAX];
  int sslot[UMAX];
  uint32_t smask[UMAX];
#pragma unroll
  for (int u = 0; u < UMAX; ++u) {
    const int a = wl + 4 * u;
    const int ac = min(a, st.n - 1);
    sptr[u] = static_cast<const T *>(st.arr[ac]) + (size_t)srow * G;
    sslot[u] = __builtin_amdgcn_readfirstlane(st.slot[ac]);
    smask[u] = __builtin_amdgcn_readfirstlane(a < st.n ? st.mask[ac] : 0u);
  }

  // slots no array writes (planes past a request's precision, padding
  // requests) must read as zero
  for (int o = tid * 16; o < NH * kStageBytes; o += kSkThreads * NH * 16)
    *reinterpret_cast<float4 *>(&stage_all[0][0] + o) = make_float4(0.f, 0.f, 0.f, 0.f);

  float acc[NB];
#pragma unroll
  for (int q = 0; q < NB; ++q) acc[q] = 0.f;

  auto fetch = [&](int step, Ops &o) {
    const int w = min(step * NH + half, nwin - 1);
    const int j = min(w * kSkGroups + wl, G - 1);
#pragma unroll
    for (int u = 0; u < kPairs; ++u) {
      const int i = min(2 * u + k, P - 1);
      o.bits[u] = tb[(i * plane_words + (size_t)j * kTileRows * 4) / 2];
    }
    const int jx = min(w * kSkGroups + bg, G - 1);
#pragma unroll
    for (int u = 0; u < Gm::rpt; ++u) {
      const int qs = min(q0 + u, nreq - 1);
      o.x[u] = Act<T>::load(x + (size_t)qs * ldx + (size_t)jx * kGroup + chunk_base(bcl),
                            chunk_parity(bcl));
    }
    const int js = min(w * kSkGroups + h, G - 1);
#pragma unroll
    for (int u = 0; u < UMAX; ++u) o.sc[u] = load_raw(sptr[u] + js);
  };

  auto consume = [&](int step, const Ops &o) {
    __syncthreads();  // the previous step's lookups are done with lut, stage, qsum
    // ---- tables of chunk bc for this thread's requests
    {
      float A[Gm::rpt], D[Gm::rpt], C[Gm::rpt], E[Gm::rpt];
#pragma unroll
      for (int u = 0; u < Gm::rpt; ++u) {
        float f[4];
        Act<T>::cvt(o.x[u], chunk_parity(bcl), f);
        A[u] = f[0] + f[1];
        D[u] = f[0] - f[1];
        C[u] = f[2] + f[3];
        E[u] = f[2] - f[3];
      }
      char *dst = lut + bg * Gm::group_stride + bcl * Gm::chunk_stride +
                  (q0 / Gm::per_entry) * Gm::half_bytes + (q0 % Gm::per_entry) * 4;
#pragma unroll
      for (int e = 0; e < kEntries; ++e) {
        // bit t of e selects +x_t: low two bits pick -A, D, -D, A; high two -C, E, -E, C
        float v[Gm::rpt];
#pragma unroll
        for (int u = 0; u < Gm::rpt; ++u) {
          const float lo = (e & 3) == 0 ? -A[u] : (e & 3) == 1 ? D[u] : (e & 3) == 2 ? -D[u] : A[u];
          const float hi = (e >> 2) == 0 ? -C[u] : (e >> 2) == 1 ? E[u] : (e >> 2) == 2 ? -E[u] : C[u];
          v[u] = lo + hi;
        }
        char *ed = dst + e * Gm::entry_bytes;
        if constexpr (Gm::rpt == 1)
          *reinterpret_cast<float *>(ed) = v[0];
        else if constexpr (Gm::rpt == 2)
          *reinterpret_cast<float2 *>(ed) = make_float2(v[0], v[1]);
        else
          *reinterpret_cast<float4 *>(ed) = make_float4(v[0], v[1], v[2], v[3]);
      }
      // quarter sums: the 8 chunks of a quarter are 8 consecutive lanes
      float cs[Gm::rpt];
#pragma unroll
      for (int u = 0; u < Gm::rpt; ++u) cs[u] = sum8_lanes(A[u] + C[u]);
      if ((tid & 7) == 0) {
#pragma unroll
        for (int u = 0; u < Gm::rpt; ++u) qsum[bg][bcl / 8][q0 + u] = cs[u];
      }
    }
    // ---- scales: array wl + 4u, position (row r, group h of the window)
#pragma unroll
    for (int u = 0; u < UMAX; ++u) {
      const float v = raw_to_float<T>(o.sc[u]);
      if constexpr (UNI) {
        if (smask[u] != 0u)
          *reinterpret_cast<float *>(stage + ((h * kSlots + sslot[u]) * kTileRows + r) * kSR) = v;
      } else {
#pragma unroll
        for (int q = 0; q < NB; ++q)
          if ((smask[u] >> q) & 1u)
            *reinterpret_cast<float *>(
                stage + (((h * kSlots + sslot[u]) * kQB + q / Gm::per_entry) * kTileRows + r) * kSR +
                (q % Gm::per_entry) * 4) = v;
      }
    }
    __syncthreads();

    // ---- lookups for this lane's (plane, column half), then scales and offsets
    const int j = (step * NH + half) * kSkGroups + wl;
    if (j < G) {
      const uint32_t base = lds_addr(lut + wl * Gm::group_stride + (16 * c) * Gm::chunk_stride);
      const uint32_t sbase = lds_addr(stage + ((wl * kSlots) * kQB * kTileRows + r) * kSR);
      constexpr int kSlotBytes = kQB * kTileRows * kSR;
      // scale and offset slots first, then the sign words software-pipelined:
      // the reads of word n + 1 are in flight while word n is summed
      float al[kPairs][NB], zz[NB], qs[NB];
      if constexpr (UNI) {
#pragma unroll
        for (int u = 0; u < kPairs; ++u) {
          const float a = *(lds_float *)(size_t)(sbase + (2 * u + k) * kSlotBytes);
#pragma unroll
          for (int q = 0; q < NB; ++q) al[u][q] = a;
        }
        const float z = *(lds_float *)(size_t)(sbase + kZSlot * kSlotBytes);
#pragma unroll
        for (int q = 0; q < NB; ++q) zz[q] = z;
      } else {
#pragma unroll
        for (int u = 0; u < kPairs; ++u) sk_read<NB>(sbase + (2 * u + k) * kSlotBytes, al[u]);
        sk_read<NB>(sbase + kZSlot * kSlotBytes, zz);
      }
#pragma unroll
      for (int q = 0; q < NB; ++q) qs[q] = qsum[wl][2 * c + k][q];
      constexpr int kWords = 2 * kPairs;
      auto word = [&](int n) { return (n & 1) ? o.bits[n >> 1].y : o.bits[n >> 1].x; };
      float t[2][8][NB];
      sk_quarter_reads<NB>(word(0), base, t[0]);
#pragma unroll
      for (int n = 0; n < kWords; ++n) {
        if (n + 1 < kWords)
          sk_quarter_reads<NB>(word(n + 1), base + ((n + 1) & 1) * 8 * Gm::chunk_stride,
                               t[(n + 1) & 1]);
#pragma unroll
        for (int q = 0; q < NB; ++q)
          acc[q] = fmaf(al[n >> 1][q], sk_quarter_sum<NB>(t[n & 1], q), acc[q]);
      }
#pragma unroll
      for (int q = 0; q < NB; ++q) acc[q] = fmaf(zz[q], qs[q], acc[q]);
    }
  };

  // a ring of kSkDepth operand sets: the loads of step s + kSkDepth - 1 are
  // issued before step s is computed, so memory latency (about 1.5 us under
  // load, several steps' worth of work) is covered by the steps in between
  constexpr int D = kSkDepth;
  Ops ring[D];
#pragma unroll
  for (int d = 0; d < D - 1; ++d) fetch(d, ring[d]);
  for (int s0 = 0; s0 < nstep; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (s0 + d >= nstep) break;  // uniform
      fetch(s0 + d + D - 1, ring[(d + D - 1) % D]);
      consume(s0 + d, ring[d]);
    }
  }

  // ---- reduce: the 4 lanes of a row in the wavefront, then the groups
  // (wavefronts) through LDS, in a fixed order
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    acc[q] += __shfl_xor(acc[q], 16);
    acc[q] += __shfl_xor(acc[q], 32);
  }
  __syncthreads();  // the tables are free: reuse them for the partials
  float *part = reinterpret_cast<float *>(&lut_all[0][0]);  // [wave][row][request]
  if (lane < kTileRows) {
#pragma unroll
    for (int q = 0; q < NB; ++q) part[(wave * kTileRows + lane) * NB + q] = acc[q];
  }
  __syncthreads();
  if (tid < kTileRows * NB) {
    const int q = tid / kTileRows;
    const int rr = tid % kTileRows;
    const int m = tile * kTileRows + rr;
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) sum += part[(v * kTileRows + rr) * NB + q];
    if (q < nreq && m < M) y[(size_t)q * ldy + m] = (T)sum;
  }
}

template <typename T, int NB, int UMAX, bool UNI, int NH = kSkConcurrent>
void skinny_launch_p(dim3 grid, hipStream_t s, const uint32_t *b, const ReqTables &t, int nreq,
                     const T *xx, int ldx, T *yy, int ldy, int M, int G, int MT, int p_max) {
  const dim3 block(kSkThreads * NH);
#define BCQ_SKP(PP)                                                                          \
  hipLaunchKernelGGL((skinny_lut_kernel<T, NB, PP, UMAX, NH, UNI>), grid, block, 0, s, b, t, \
                     nreq, xx, ldx, yy, ldy, M, G, MT)
  switch (p_max) {
    case 1: BCQ_SKP(1); break;
    case 2: BCQ_SKP(2); break;
    case 3: BCQ_SKP(3); break;
    default: BCQ_SKP(4); break;
  }
#undef BCQ_SKP
}

// One precision for every request: the host lists exactly p + 1 arrays (the
// planes and offsets of that precision), each read by every request.
template <typename T, int NB>
void skinny_launch_u(dim3 grid, hipStream_t s, const uint32_t *b, const ReqTables &t, int nreq,
                     const T *xx, int ldx, T *yy, int ldy, int M, int G, int MT, int p_max) {
  if (t.n == p_max + 1)
    skinny_launch_p<T, NB, 2, true>(grid, s, b, t, nreq, xx, ldx, yy, ldy, M, G, MT, p_max);
  else if (t.n <= 8)
    skinny_launch_p<T, NB, 2, false>(grid, s, b, t, nreq, xx, ldx, yy, ldy, M, G, MT, p_max);
  else
    skinny_launch_p<T, NB, 4, false>(grid, s, b, t, nreq, xx, ldx, yy, ldy, M, G, MT, p_max);
}

template <typename T>
hipError_t skinny_dispatch(const uint32_t *bits, int M, int K, int p_max, const ReqTables &t,
                           int nreq, const void *x, int ldx, void *y, int ldy, hipStream_t s) {
  const int G = K / kGroup;
  const int MT = row_tiles(M);
  const T *xx = static_cast<const T *>(x);
  T *yy = static_cast<T *>(y);
  const dim3 grid(MT);
  if (nreq <= 2)
    skinny_launch_u<T, 2>(grid, s, bits, t, nreq, xx, ldx, yy, ldy, M, G, MT, p_max);
  else if (nreq <= 4)
    skinny_launch_u<T, 4>(grid, s, bits, t, nreq, xx, ldx, yy, ldy, M, G, MT, p_max);
  else
    skinny_launch_u<T, 8>(grid, s, bits, t, nreq, xx, ldx, yy, ldy, M, G, MT, p_max);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_lut(const uint32_t *bits, int M, int K, int p, const void *alpha,
                           const void *zero, const void *x, void *y, bcq_dtype dt,
                           hipStream_t s) {
  if (dt == BCQ_F16) return gemv_dispatch<half_t, false>(bits, M, K, p, alpha, zero, x, y, s);
  return gemv_dispatch<float, false>(bits, M, K, p, alpha, zero, x, y, s);
}

bool gemv_lowrank_fused_ok(int K, int R) {
  return K <= 2 * kG1Ksub * kGroup && R >= 1 && R <= 32 * kLrMaxWords;
}

hipError_t launch_gemv_lowrank(const uint32_t *bits, int M, int K, int p, const void *alpha,
                               const void *zero, const void *x, void *y, const uint32_t *u,
                               const float *z, int R, bcq_dtype dt, hipStream_t s) {
  if (!gemv_lowrank_fused_ok(K, R)) return hipErrorInvalidValue;
  if (dt == BCQ_F16)
    return gemv_lowrank_dispatch<half_t>(bits, M, K, p, alpha, zero, x, y, u, z, R, s);
  return gemv_lowrank_dispatch<float>(bits, M, K, p, alpha, zero, x, y, u, z, R, s);
}

hipError_t launch_gemv_gate_up(const uint32_t *bits, int M, int K, int p, const void *alpha,
                               const void *zero, const void *x, void *y, bcq_dtype dt,
                               hipStream_t s) {
  if (dt == BCQ_F16) return gemv_dispatch<half_t, true>(bits, M, K, p, alpha, zero, x, y, s);
  return gemv_dispatch<float, true>(bits, M, K, p, alpha, zero, x, y, s);
}

hipError_t launch_skinny_lut(const uint32_t *bits, int M, int K, int p_max, const ReqTables &t,
                             int nreq, const void *x, int ldx, void *y, int ldy, bcq_dtype dt,
                             hipStream_t s) {
  if (dt == BCQ_F16) return skinny_dispatch<half_t>(bits, M, K, p_max, t, nreq, x, ldx, y, ldy, s);
  return skinny_dispatch<float>(bits, M, K, p_max, t, nreq, x, ldx, y, ldy, s);
}

}  // namespace bcq
