// Whole-row units of eight rows: the eight rows of one 64-row tile hold,
// chunk after chunk, whole 128-byte lines of the tiled layout (4- and
// 8-bit), so a workgroup of four wavefronts that takes eight rows and all
// of K reads only whole lines: lane l takes row l % 8 and 64-groups
// l / 8 + 8 w + 32 i (w: its wavefront), a butterfly adds the 32 group
// lanes of a row in the wavefront and LDS the four wavefronts.  Used by the
// stacked decode and by the small-batch decode launches.
#pragma once
#include "decode_impl.h"

namespace moeq {

constexpr int kDW = 16;   // dwords of one group's codes in one lane (8-bit: 4 chunks of 4)

// One 64-group of one row of a matrix, for one lane: its codes (CPG
// chunks) and the group's scale/zero word.
struct Grp {
  uint32_t d[kDW];
  uint32_t w;
};

// Loads group g of row `row` (K columns) when `on`, else zeros (every element
// assigned, so that no older value is carried across loops).
template <int BITS>
MOEQ_DEV void grp_load(Grp& G, const uint8_t* q, const uint32_t* sz, size_t row, int K, int g, bool on) {
  using F = Fmt<BITS>;
  constexpr int CPG = F::CHUNKS_PER_GROUP;
#pragma unroll
  for (int i = 0; i < kDW; ++i) G.d[i] = 0;
  G.w = 0;
  if (on) {
    const size_t cpr = (size_t)(K / F::CODES), gpr = (size_t)(K / 64);
#pragma unroll
    for (int c = 0; c < CPG; ++c) {
      uint32_t t[F::DW];
      decode_detail::load_chunk_g<BITS>((gbytes)(q + chunk_offset<BITS>(row, (size_t)g * CPG + c, cpr)), t);
#pragma unroll
      for (int i = 0; i < F::DW; ++i) G.d[c * F::DW + i] = t[i];
    }
    G.w = load_word_g((gbytes)(sz + sz_index(row, (size_t)g, gpr)));
  }
}

// The group's dot product with the activations xl (LDS, bf16, 64 of them)
// whose sum is xsum: s (sum of code x activation - (z + offset) xsum).
template <int BITS>
MOEQ_DEV float grp_dot(const Grp& G, const uint16_t* xl, float xsum) {
  using F = Fmt<BITS>;
  constexpr int CPG = F::CHUNKS_PER_GROUP;
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int c = 0; c < CPG; ++c) {
    uint32_t t[F::DW], P[F::PAIRS];
#pragma unroll
    for (int i = 0; i < F::DW; ++i) t[i] = G.d[c * F::DW + i];
    chunk_pairs<BITS>(t, P);
    const uint4* xp = reinterpret_cast<const uint4*>(xl + c * F::CODES);
#pragma unroll
    for (int p = 0; p < F::PAIRS; p += 4) {
      const uint4 X = xp[p / 4];
      a0 = dot2_bf16(P[p], X.x, a0);
      a1 = dot2_bf16(P[p + 1], X.y, a1);
      a0 = dot2_bf16(P[p + 2], X.z, a0);
      a1 = dot2_bf16(P[p + 3], X.w, a1);
    }
  }
  const float s = f16_bits_to_f32(G.w & 0xFFFFu);
  const float zc = f16_bits_to_f32(G.w >> 16) + F::OFFSET;
  return s * ((a0 + a1) - zc * xsum);
}

// Unit of the i-th of n workgroups that take units (workgroup b runs on XCD
// b mod 8, and i = b - a multiple of 8): with n a multiple of 64, each XCD
// takes runs of eight consecutive units, the eight 8-row units of one
// 64-row tile, so that all the 128-byte lines of a tile's chunks are read
// through one L2, one unit right after the other.
MOEQ_DEV int xcd_unit(int i, int n) {
  if (n % 64) return i;
  const int x = i % 8, s = i / 8;
  return ((s / 8) * 8 + x) * 8 + s % 8;
}

// Sum over the eight lanes of a wavefront that share lane % 8 (a butterfly:
// every one of them ends with the same value).
MOEQ_DEV float sum_stride8(float v) {
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace moeq
