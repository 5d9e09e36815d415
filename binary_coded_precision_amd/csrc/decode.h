// decode.h -- the fp16 weight decode shared by the batched decode kernel and
// the matrix-core kernel.
//
// A BCQ weight is w = z + sum_{i<p} alpha_i s_i with s_i = +-1 the plane's sign
// bit (AnyBCQ paper notes, "Method / key designs").  Weights are decoded as
// fp16 pairs (columns 2t, 2t+1) of one 32-column packed sign word: the packed
// word holds even columns in its low half and odd columns in its high half
// (pack.hip), so the pair's sign bits are bits t and t+16 and one shift moves
// both to the fp16 sign positions (bits 15 and 31).  Per plane and pair:
//   m   = word' << (15 - t)                       one shift
//   +-a = (m & 0x80008000) | |alpha| in both       one bit-field insert
//   w  += +-a                                      one packed fp16 add
// where word' is the sign word inverted, or not when alpha < 0, so that a set
// bit yields +alpha.  The decoded weight is rounded to fp16 after every
// addition (relative 2^-11 each).
#pragma once

#include "bcq_internal.h"

namespace bcq {

typedef _Float16 dq_half2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ dq_half2 dq_as_h2(uint32_t u) { return __builtin_bit_cast(dq_half2, u); }

constexpr int kDqPairs = 16;  // fp16 pairs per 32-column sign word

// w[t] = (z, z) for every pair; z16 is the raw fp16 offset in the low half.
__device__ __forceinline__ void dq_init(dq_half2 (&w)[kDqPairs], uint32_t z16) {
  const dq_half2 z2 = dq_as_h2((z16 & 0xFFFFu) * 0x10001u);
#pragma unroll
  for (int t = 0; t < kDqPairs; ++t) w[t] = z2;
}

// One plane's contribution to the 16 pairs of a word: w[t] += +-alpha.
// a16 is the raw fp16 scale in the low half of a register.
__device__ __forceinline__ void dq_plane(dq_half2 (&w)[kDqPairs], uint32_t word, uint32_t a16) {
  const uint32_t mag = (a16 & 0x7FFFu) * 0x10001u;               // |alpha| in both halves
  const uint32_t neg = (uint32_t)((int32_t)(a16 << 16) >> 31);  // all ones when alpha < 0
  const uint32_t wp = ~(word ^ neg);  // sign bit 0 (+|alpha|) where s * alpha is positive
#pragma unroll
  for (int t = 0; t < kDqPairs; ++t) {
    const uint32_t m = wp << (15 - t);  // bits t, t+16 (columns 2t, 2t+1) -> 15, 31
    w[t] += dq_as_h2((m & 0x80008000u) | mag);
  }
}

}  // namespace bcq
