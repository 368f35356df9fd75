// The weight boundary of the library: codes in the plain packed form an
// offline quantiser writes (rows of K*bits/8 bytes, codes in natural order)
// and fp16 scale and zero arrays, laid out once into the tiled, field-ordered
// form the kernels stream (format.h).  HQQ assets are made once, before the
// hot path, by a preprocessing stage (Krasis update, "Latest updates"); this
// is the step that hands them to it.
//
// Plain packing of a row of codes c_0 .. c_{K-1}:
//   4-bit: byte i = c_{2i} | c_{2i+1} << 4
//   6-bit: bytes 3i, 3i+1, 3i+2 = the 24-bit little-endian word
//          c_{4i} | c_{4i+1} << 6 | c_{4i+2} << 12 | c_{4i+3} << 18
//   8-bit: byte i = c_i
#include "format.h"

#include <string.h>

using namespace moeq;

namespace {

// One thread per (row, chunk): the chunk's codes in natural order from the
// plain row, then written field by field in the tiled chunk.  Threads of a
// block take consecutive rows of one chunk, so the writes are contiguous.
template <int BITS>
__global__ __launch_bounds__(256) void load_codes_kernel(const uint8_t* __restrict__ src, long rows, int K,
                                                         uint8_t* __restrict__ dst) {
  using F = Fmt<BITS>;
  const long cpr = K / F::CODES;
  const long n = rows * cpr;
  const size_t rb = row_bytes(K, BITS);
  for (long t = (long)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (long)gridDim.x * blockDim.x) {
    // t -> (tile, chunk, row in tile): consecutive t = consecutive rows
    const long tile = t / (64 * cpr);
    const long c = (t / 64) % cpr;
    const long r = tile * 64 + (t % 64);
    const uint8_t* s = src + (size_t)r * rb + (size_t)c * F::BYTES;
    uint32_t code[F::CODES];
    if constexpr (BITS == 4) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        code[2 * i] = s[i] & 0xFu;
        code[2 * i + 1] = s[i] >> 4;
      }
    } else if constexpr (BITS == 6) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = (uint32_t)s[3 * i] | ((uint32_t)s[3 * i + 1] << 8) | ((uint32_t)s[3 * i + 2] << 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) code[4 * i + j] = (w >> (6 * j)) & 0x3Fu;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) code[i] = s[i];
    }
    uint8_t out[F::BYTES];
    if constexpr (BITS == 4) {
#pragma unroll
      for (int b = 0; b < 16; ++b)
        out[b] = (uint8_t)(code[field_code<4>(2 * b)] | (code[field_code<4>(2 * b + 1)] << 4));
    } else if constexpr (BITS == 6) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = code[field_code<6>(4 * i)] | (code[field_code<6>(4 * i + 1)] << 6) |
                           (code[field_code<6>(4 * i + 2)] << 12) | (code[field_code<6>(4 * i + 3)] << 18);
        out[3 * i] = (uint8_t)w;
        out[3 * i + 1] = (uint8_t)(w >> 8);
        out[3 * i + 2] = (uint8_t)(w >> 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) out[i] = (uint8_t)code[field_code<8>(i)];
    }
    uint8_t* d = dst + chunk_offset<BITS>((size_t)r, (size_t)c, (size_t)cpr);
#pragma unroll
    for (int i = 0; i < F::BYTES; ++i) d[i] = out[i];
  }
}

// One thread per (row, group): the scale/zero word at its tiled index.
__global__ __launch_bounds__(256) void load_sz_kernel(const uint16_t* __restrict__ scale,
                                                      const uint16_t* __restrict__ zero, long rows, int gpr,
                                                      uint32_t* __restrict__ sz) {
  const long n = rows * gpr;
  for (long t = (long)blockIdx.x * blockDim.x + threadIdx.x; t < n; t += (long)gridDim.x * blockDim.x) {
    const long tile = t / (64 * (long)gpr);
    const long g = (t / 64) % gpr;
    const long r = tile * 64 + (t % 64);
    const size_t i = (size_t)r * gpr + g;
    sz[sz_index((size_t)r, (size_t)g, (size_t)gpr)] = (uint32_t)scale[i] | ((uint32_t)zero[i] << 16);
  }
}

int grid_for(long n) {
  long b = (n + 255) / 256;
  return (int)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

}  // namespace

extern "C" int moe_pack(const uint8_t* codes, long N, int K, int bits, uint8_t* packed) {
  if (!codes || !packed || N < 0 || K <= 0)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_pack: NULL pointer or N=%ld K=%d", N, K);
  if (!bits_ok(bits)) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_pack: bits=%d not in {4,6,8}", bits);
  if (K % 4) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_pack: K=%d not a multiple of 4", K);
  const uint32_t qmax = (1u << bits) - 1u;
  const size_t total = (size_t)N * K;
  for (size_t i = 0; i < total; ++i)
    if (codes[i] > qmax) return set_error(MOEQ_ERR_INVALID_ARG, "moe_pack: code %u at %zu exceeds %u", codes[i], i, qmax);
  const size_t rb = row_bytes(K, bits);
  for (long r = 0; r < N; ++r) {
    const uint8_t* c = codes + (size_t)r * K;
    uint8_t* p = packed + (size_t)r * rb;
    if (bits == 8) {
      memcpy(p, c, (size_t)K);
    } else if (bits == 4) {
      for (int i = 0; i < K / 2; ++i) p[i] = (uint8_t)(c[2 * i] | (c[2 * i + 1] << 4));
    } else {
      for (int i = 0; i < K / 4; ++i) {
        const uint32_t w = (uint32_t)c[4 * i] | ((uint32_t)c[4 * i + 1] << 6) | ((uint32_t)c[4 * i + 2] << 12) |
                           ((uint32_t)c[4 * i + 3] << 18);
        p[3 * i] = (uint8_t)w;
        p[3 * i + 1] = (uint8_t)(w >> 8);
        p[3 * i + 2] = (uint8_t)(w >> 16);
      }
    }
  }
  return MOEQ_OK;
}

extern "C" int moe_qweight_load(const uint8_t* packed, const uint16_t* scale, const uint16_t* zero, long rows, int K,
                                int bits, uint8_t* q, uint32_t* sz, hipStream_t stream) {
  if (!packed || !scale || !zero || !q || !sz || rows < 0 || K <= 0)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_qweight_load: NULL pointer or rows=%ld K=%d", rows, K);
  if (!bits_ok(bits)) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_qweight_load: bits=%d not in {4,6,8}", bits);
  if (K % MOEQ_GROUP || rows % 64)
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_qweight_load: K=%d and rows=%ld must be multiples of 64", K, rows);
  if (!aligned16(q) || !aligned16(sz))
    return set_error(MOEQ_ERR_MISALIGNED, "moe_qweight_load: q and sz must be 16-byte aligned");
  if (rows == 0) return MOEQ_OK;
  const long cpr = K / (bits == 4 ? 32 : 16);
  const long nc = rows * cpr;
  switch (bits) {
    case 4: load_codes_kernel<4><<<grid_for(nc), 256, 0, stream>>>(packed, rows, K, q); break;
    case 6: load_codes_kernel<6><<<grid_for(nc), 256, 0, stream>>>(packed, rows, K, q); break;
    default: load_codes_kernel<8><<<grid_for(nc), 256, 0, stream>>>(packed, rows, K, q); break;
  }
  int rc = check_launch("moe_qweight_load (codes)");
  if (rc != MOEQ_OK) return rc;
  const int gpr = K / MOEQ_GROUP;
  load_sz_kernel<<<grid_for(rows * gpr), 256, 0, stream>>>(scale, zero, rows, gpr, sz);
  return check_launch("moe_qweight_load (scale/zero)");
}
