// Group-quantised KV-cache codec: bf16 cache rows <-> codes + fp16 scale/zero
// per 64 values, the weight format's quantiser on the cache (Krasis update,
// "Latest updates": 4- and 6-bit KV cache).  Rows are stored one after the
// other, each as its packed codes in natural order (4-bit: code 2i in the low
// nibble of byte i; 6-bit: code c at bits 6c .. 6c + 5 of the row's
// little-endian bit string; 8-bit: one byte per code), the scale/zero words
// [row][group] beside them.
#include "quant_group.h"

using namespace moeq;

namespace {

// Minimum / maximum over the 16 lanes of a DPP row (every lane gets it).
MOEQ_DEV float row_min16(float v) {
  v = fminf(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fminf(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fminf(v, dpp_f<0x141>(v));   // row_half_mirror
  return fminf(v, dpp_f<0x140>(v));   // row_mirror
}
MOEQ_DEV float row_max16(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  return fmaxf(v, dpp_f<0x140>(v));
}

// Four groups per wavefront: the 16 lanes of row r hold group 4 w + r, lane
// j of the row its values 4 j .. 4 j + 3 (one 8-byte load).  The row's
// packed bytes (8 / 12 / 16 dwords) are assembled from the lanes' 16 / 24 /
// 32-bit pieces and written as dwords.
template <int BITS>
__global__ __launch_bounds__(256) void kv_encode_kernel(const uint16_t* __restrict__ x, long ngroups,
                                                        uint32_t* __restrict__ q, uint32_t* __restrict__ sz) {
  constexpr int NDW = 64 * BITS / 32;   // dwords of packed codes per group
  const int lane = threadIdx.x & 63, j = lane & 15, row0 = lane & 48;
  const long stride = (long)gridDim.x * 16;
  for (long g0 = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4; g0 < ngroups; g0 += stride) {
    const long g = g0 + (lane >> 4);
    const bool valid = g < ngroups;   // a whole row is valid or not
    uint2 raw = make_uint2(0u, 0u);
    if (valid) raw = *reinterpret_cast<const uint2*>(x + g * 64 + 4 * j);
    const float v[4] = {bf16_bits_to_f32(raw.x & 0xFFFFu), bf16_bits_to_f32(raw.x >> 16),
                        bf16_bits_to_f32(raw.y & 0xFFFFu), bf16_bits_to_f32(raw.y >> 16)};
    const float mn = row_min16(fminf(fminf(v[0], v[1]), fminf(v[2], v[3])));
    const float mx = row_max16(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
    const GroupQuant gq = minmax_from<BITS>(mn, mx);
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = group_code(gq, v[i], gq.zf);
    if constexpr (BITS == 4) {
      // dword m = lanes 2m, 2m + 1 of the row (16 bits each)
      const uint32_t h = c[0] | (c[1] << 4) | (c[2] << 8) | (c[3] << 12);
      const uint32_t hn = __shfl_xor(h, 1);
      if (valid && !(j & 1)) q[g * NDW + (j >> 1)] = h | (hn << 16);
    } else if constexpr (BITS == 8) {
      if (valid) q[g * NDW + j] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
    } else {
      // lane j holds bits 24 j .. 24 j + 23 of the row's string; dword m
      // takes them from lanes a = 4m / 3 (from bit 32 m - 24 a on) and a + 1
      const uint32_t t = c[0] | (c[1] << 6) | (c[2] << 12) | (c[3] << 18);
      const int m = j < NDW ? j : 0;
      const int a = (4 * m) / 3, off = 32 * m - 24 * a;
      const uint32_t ta = __shfl(t, row0 + a), tb = __shfl(t, row0 + a + 1);
      if (valid && j < NDW) q[g * NDW + m] = (ta >> off) | (tb << (24 - off));
    }
    if (valid && j == 0) sz[g] = gq.s16 | (gq.z16 << 16);
  }
}

// One thread per 8 codes: (q - z) * s in fp32 (two roundings, no fused
// multiply-add), rounded to bf16, stored as 16 bytes.
template <int BITS>
__global__ __launch_bounds__(256) void kv_decode_kernel(const uint8_t* __restrict__ q,
                                                        const uint32_t* __restrict__ sz, long n8,
                                                        uint16_t* __restrict__ out) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n8; i += (long)gridDim.x * blockDim.x) {
    uint32_t c[8];
    if constexpr (BITS == 4) {
      const uint32_t d = reinterpret_cast<const uint32_t*>(q)[i];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = (d >> (4 * j)) & 0xFu;
    } else if constexpr (BITS == 6) {
      const uint16_t* p = reinterpret_cast<const uint16_t*>(q + 6 * i);
      const uint64_t d = (uint64_t)p[0] | ((uint64_t)p[1] << 16) | ((uint64_t)p[2] << 32);
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = (uint32_t)(d >> (6 * j)) & 0x3Fu;
    } else {
      const uint2 d = reinterpret_cast<const uint2*>(q)[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = (d.x >> (8 * j)) & 0xFFu;
        c[4 + j] = (d.y >> (8 * j)) & 0xFFu;
      }
    }
    const uint32_t w = sz[i >> 3];   // 8 threads per group of 64
    const float s = f16_bits_to_f32(w & 0xFFFFu), z = f16_bits_to_f32(w >> 16);
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = ((float)c[2 * j] - z) * s, b = ((float)c[2 * j + 1] - z) * s;
      o[j] = f32_to_bf16_bits(a) | (f32_to_bf16_bits(b) << 16);
    }
    *reinterpret_cast<uint4*>(out + 8 * i) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

int grid_for(long work, int per_block) {
  long b = (work + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > 65536) b = 65536;
  return (int)b;
}

int kv_check(const char* fn, const void* a, const void* b, const void* c, long rows, int D, int bits) {
  if (!a || !b || !c) return set_error(MOEQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (rows < 0 || D <= 0) return set_error(MOEQ_ERR_INVALID_ARG, "%s: rows=%ld D=%d", fn, rows, D);
  if (!bits_ok(bits)) return set_error(MOEQ_ERR_UNSUPPORTED, "%s: bits=%d not in {4,6,8}", fn, bits);
  if (D % MOEQ_GROUP) return set_error(MOEQ_ERR_UNSUPPORTED, "%s: D=%d not a multiple of 64", fn, D);
  return MOEQ_OK;
}

}  // namespace

extern "C" int moe_kv_encode(const uint16_t* x, long rows, int D, int bits, uint8_t* q, uint32_t* sz,
                             hipStream_t stream) {
  int rc = kv_check("moe_kv_encode", x, q, sz, rows, D, bits);
  if (rc != MOEQ_OK) return rc;
  if (!aligned16(x) || !aligned16(q) || ((uintptr_t)sz & 3u))
    return set_error(MOEQ_ERR_MISALIGNED, "moe_kv_encode: x and q must be 16-byte aligned, sz 4-byte");
  const long ngroups = rows * (D / MOEQ_GROUP);
  if (ngroups == 0) return MOEQ_OK;
  uint32_t* qw = reinterpret_cast<uint32_t*>(q);
  const int grid = grid_for(ngroups, 16);   // 4 groups per wavefront, 4 wavefronts per block
  switch (bits) {
    case 4: kv_encode_kernel<4><<<grid, 256, 0, stream>>>(x, ngroups, qw, sz); break;
    case 6: kv_encode_kernel<6><<<grid, 256, 0, stream>>>(x, ngroups, qw, sz); break;
    default: kv_encode_kernel<8><<<grid, 256, 0, stream>>>(x, ngroups, qw, sz); break;
  }
  return check_launch("moe_kv_encode");
}

extern "C" int moe_kv_decode(const uint8_t* q, const uint32_t* sz, long rows, int D, int bits, uint16_t* out,
                             hipStream_t stream) {
  int rc = kv_check("moe_kv_decode", q, sz, out, rows, D, bits);
  if (rc != MOEQ_OK) return rc;
  if (!aligned16(q) || !aligned16(out) || ((uintptr_t)sz & 3u))
    return set_error(MOEQ_ERR_MISALIGNED, "moe_kv_decode: q and out must be 16-byte aligned, sz 4-byte");
  const long n8 = rows * (long)D / 8;
  if (n8 == 0) return MOEQ_OK;
  const int grid = grid_for(n8, 256);
  switch (bits) {
    case 4: kv_decode_kernel<4><<<grid, 256, 0, stream>>>(q, sz, n8, out); break;
    case 6: kv_decode_kernel<6><<<grid, 256, 0, stream>>>(q, sz, n8, out); break;
    default: kv_decode_kernel<8><<<grid, 256, 0, stream>>>(q, sz, n8, out); break;
  }
  return check_launch("moe_kv_decode");
}
