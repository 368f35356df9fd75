// Device view of the packed weight format: where a code lives in memory and
// how one lane turns a "chunk" of codes into bf16 pairs for v_dot2_f32_bf16.
//
// A chunk is the unit one lane loads with one vector load:
//   4-bit: 16 bytes = 32 codes (dwordx4); a 64-group spans 2 chunks
//   6-bit: 12 bytes = 16 codes (dwordx3); a 64-group spans 4 chunks
//   8-bit: 16 bytes = 16 codes (dwordx4); a 64-group spans 4 chunks
//
// Layout in memory (per projection, all experts' rows r = 0 .. n_mats*N-1):
// rows come in tiles of 64, and inside a tile chunk-major: chunk c of row r
// starts at byte ((r / 64) * CPR + c) * 64 * BYTES + (r % 64) * BYTES, CPR =
// K / CODES.  A wavefront whose lane l handles row 64 t + l thus reads one
// contiguous 64 * BYTES block per chunk.  The scale/zero word of group g of
// row r sits at index ((r / 64) * GPR + g) * 64 + r % 64, GPR = K / 64.
//
// Inside a chunk the codes sit in "fields" (4-bit: nibble n = byte n/2, low
// nibble first; 6-bit: bits 6n..6n+5 of the little-endian chunk; 8-bit:
// byte n) in an order chosen so that the in-register unpacking below yields
// the bf16 pairs (code 2p, code 2p+1) with one AND-OR per pair: field_code()
// gives the code held by field n.
//
// Codes become bf16 values exactly: 4- and 6-bit codes are OR-ed into the
// mantissa of bf16 128.0 (giving 128 + q, "OFFSET" = 128); 8-bit codes are
// converted through fp32 (OFFSET = 0).
#pragma once
#include "common.h"

template <int BITS> struct Fmt;
template <> struct Fmt<4> {
  static constexpr int BYTES = 16, CODES = 32, PAIRS = 16, DW = 4, CHUNKS_PER_GROUP = 2;
  static constexpr float OFFSET = 128.0f;
};
template <> struct Fmt<6> {
  static constexpr int BYTES = 12, CODES = 16, PAIRS = 8, DW = 3, CHUNKS_PER_GROUP = 4;
  static constexpr float OFFSET = 128.0f;
};
template <> struct Fmt<8> {
  static constexpr int BYTES = 16, CODES = 16, PAIRS = 8, DW = 4, CHUNKS_PER_GROUP = 4;
  static constexpr float OFFSET = 0.0f;
};

// Code index (within the chunk) in the low (half=0) or high (half=1) bf16 of
// pair p: natural for every width (the field order makes it so).
template <int BITS>
MOEQ_DEV constexpr int pair_code(int p, int half) { return 2 * p + half; }

// Code held by field n of a chunk.  4-bit: nibbles 8d + j and 8d + 4 + j
// (j < 4) of dword d hold codes 8d + 2j and 8d + 2j + 1, so (w >> 4j) &
// 0x000F000F of that dword is pair 4d + j.  6-bit: the fields chunk_pairs<6>
// combines into pair p are (lo[p], hi[p]) = (0,3) (1,4) (5,8) (6,9) (10,13)
// (11,14) (2,7) (12,15); they hold codes 2p and 2p + 1.  8-bit: natural.
template <int BITS>
MOEQ_HD constexpr int field_code(int n) {
  if constexpr (BITS == 4) {
    return 8 * (n >> 3) + 2 * (n & 3) + ((n >> 2) & 1);
  } else if constexpr (BITS == 6) {
    // nibble n: code of field n = 0, 2, 12, 1, 3, 4, 6, 13, 5, 7, 8, 10, 14, 9, 11, 15
    return (int)((0xFB9EA875D6431C20ull >> (4 * n)) & 0xF);
  } else {
    return n;
  }
}

// Byte offset of chunk c of row r, and index of the scale/zero word of
// group g of row r, in the tiled layout (cpr chunks and gpr groups per row).
template <int BITS>
MOEQ_HD size_t chunk_offset(size_t r, size_t c, size_t cpr) {
  return ((r >> 6) * cpr + c) * (64 * (size_t)Fmt<BITS>::BYTES) + (r & 63) * (size_t)Fmt<BITS>::BYTES;
}
MOEQ_HD size_t sz_index(size_t r, size_t g, size_t gpr) { return ((r >> 6) * gpr + g) * 64 + (r & 63); }

typedef uint32_t moeq_u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t moeq_u32x3 __attribute__((ext_vector_type(3)));

template <int BITS>
MOEQ_DEV void load_chunk(const uint8_t* __restrict__ p, uint32_t (&d)[Fmt<BITS>::DW]) {
  if constexpr (Fmt<BITS>::DW == 4) {
    moeq_u32x4 v = *reinterpret_cast<const moeq_u32x4*>(p);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  } else {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    d[0] = q[0];
    d[1] = q[1];
    d[2] = q[2];
  }
}

// Values the compiler cannot see are the same on every lane (they are: all
// their inputs are wave-uniform), moved to scalar registers so that addresses
// built from them stay scalar.  A load address is then a scalar base plus
// one 32-bit lane offset (the global_load "saddr" form): no per-chunk
// address occupies vector registers.
MOEQ_DEV int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// global-memory pointer (address space 1): loads through it are global_load,
// not flat loads
typedef const __attribute__((address_space(1))) uint8_t* gbytes;
MOEQ_DEV gbytes uniform_ptr(const uint8_t* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<gbytes>(((uint64_t)hi << 32) | lo);
}

MOEQ_DEV uint32_t load_word_g(gbytes p) { return *reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(p); }

MOEQ_DEV uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) { return (a & m) | o; }

// The bf16 128.0 pair lives in a VGPR (an empty asm makes it opaque) so that
// v_and_or_b32 can take the mask from an SGPR and the OR operand from this
// register: gfx9 VOP3 encodings read at most one scalar operand.
MOEQ_DEV uint32_t magic_128_pair() {
  uint32_t m = 0x43004300u;
  asm volatile("" : "+v"(m));
  return m;
}

// 6-bit chunk -> the 8 pairs (code 2p, code 2p+1), each code OR-ed into the
// low mantissa bits of the 16-bit float pair M (bf16 128.0 or fp16 1024.0).
MOEQ_DEV void pairs6(const uint32_t (&d)[3], uint32_t M, uint32_t (&P)[8]) {
  // code c of the chunk sits at bits 6c..6c+5 of the 96-bit little-endian
  // chunk.  e0/e1/e2 are 32-bit windows starting at codes 0, 5 and 10.
  uint32_t e0 = d[0];
  uint32_t e1 = __builtin_amdgcn_alignbit(d[1], d[0], 30);
  uint32_t e2 = __builtin_amdgcn_alignbit(d[2], d[1], 28);
  const uint32_t e[3] = {e0, e1, e2};
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    // codes at bits 0 and 18 -> halves 0 and 16
    P[2 * i + 0] = and_or(e[i] >> 2, 0x003F0000u, and_or(e[i], 0x3Fu, M));
    // codes at bits 6 and 24
    P[2 * i + 1] = and_or(e[i] >> 8, 0x003F0000u, and_or(e[i] >> 6, 0x3Fu, M));
  }
  P[6] = and_or(e1 << 4, 0x003F0000u, and_or(e0 >> 12, 0x3Fu, M));     // codes 2, 7
  P[7] = and_or(d[2] >> 10, 0x003F0000u, and_or(e2 >> 12, 0x3Fu, M));  // codes 12, 15
}

template <int BITS>
MOEQ_DEV void chunk_pairs(const uint32_t (&d)[Fmt<BITS>::DW], uint32_t (&P)[Fmt<BITS>::PAIRS]) {
  const uint32_t M = magic_128_pair();   // bf16 128.0 in both halves
  if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = d[j];
      P[4 * j + 0] = and_or(w, 0x000F000Fu, M);
      P[4 * j + 1] = and_or(w >> 4, 0x000F000Fu, M);
      P[4 * j + 2] = and_or(w >> 8, 0x000F000Fu, M);
      P[4 * j + 3] = and_or(w >> 12, 0x000F000Fu, M);
    }
  } else if constexpr (BITS == 6) {
    pairs6(d, M, P);
  } else {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w = d[j];
      bf16x2 a = {(__bf16)(float)(w & 0xFFu), (__bf16)(float)((w >> 8) & 0xFFu)};
      bf16x2 b = {(__bf16)(float)((w >> 16) & 0xFFu), (__bf16)(float)(w >> 24)};
      P[2 * j + 0] = __builtin_bit_cast(uint32_t, a);
      P[2 * j + 1] = __builtin_bit_cast(uint32_t, b);
    }
  }
}

typedef __bf16 moeq_bf16x2 __attribute__((ext_vector_type(2)));

// acc + lo(a)*lo(b) + hi(a)*hi(b), fp32 accumulate (v_dot2_f32_bf16)
MOEQ_DEV float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(moeq_bf16x2, a),
                                         __builtin_bit_cast(moeq_bf16x2, b), acc, false);
}
