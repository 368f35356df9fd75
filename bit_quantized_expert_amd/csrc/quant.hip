// Group quantisation of fp32 weights into the packed format, and the unpack
// test entry that runs the decode kernels' in-register unpacking.
#include "format.h"
#include "quant_group.h"

using namespace moeq;

// HQQ's zero-point refinement (Badri & Shaji, "Half-Quadratic Quantization
// of Large Machine Learning Models", the half-quadratic solver with the
// scale held): parameters of the lp penalty, the coupling weight and its
// growth, and the number of rounds (0: plain min-max quantisation).
struct HqqParams {
  float lp, beta, kappa;
  int iters;
};

// Sum of one double per lane over the wavefront (every lane gets it).  The
// order of the additions is the butterfly's; in fp64 it moves the sum of a
// group's 64 values by a few ulps at most, far below an fp16 step.
MOEQ_DEV double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// fp64 -> fp16 bits, round to nearest even, in one rounding (no stop in
// fp32 on the way), for finite |x| < 65520.
MOEQ_DEV uint32_t f64_to_f16_bits(double x) {
  const uint32_t sign = __builtin_signbit(x) ? 0x8000u : 0u;
  const double a = fabs(x);
  if (a < 0x1p-14) return sign | (uint32_t)rint(a * 0x1p24);   // subnormal (1024 is the smallest normal)
  int e;
  frexp(a, &e);                                 // a in [2^(e-1), 2^e)
  double m = rint(ldexp(a, 11 - e));            // 11 significant bits: [1024, 2048]
  int E = e - 1;
  if (m == 2048.0) {
    m = 1024.0;
    ++E;
  }
  return sign | ((uint32_t)(E + 15) << 10) | ((uint32_t)m - 1024u);
}

// One round per iteration, for the group in this wavefront (lane l holds
// value v of the group, sf its scale, z its current zero, an fp16 value):
// the codes for z (fp32, as the quantiser) and the exact residual r (fp64);
// the group stops when its mean absolute error is not below its best; else
// z is kept as the best and replaced by the zero sub-problem's solution for
// the shrunk residual, formed in fp64 and rounded once to fp16.  The shrink
// is 0 wherever |r| is clearly below the round's threshold
// beta^(-1/(2 - lp)) (there |r| - |r|^(lp - 1)/beta < 0), so the power is
// only evaluated where it can matter.
MOEQ_DEV float hqq_zero(float v, float sf, float z, float qmax, const HqqParams& hp) {
#pragma clang fp contract(off)
  double best = INFINITY, beta = (double)hp.beta;
  float zb = z;
  const double pm1 = (double)hp.lp - 1.0, vd = (double)v, sd = (double)sf;
  for (int it = 0; it < hp.iters; ++it) {
    const float qv = fminf(fmaxf(rintf(v / sf + z), 0.0f), qmax);
    const double r = vd - ((double)qv - (double)z) * sd;             // exact in fp64
    const double a = fabs(r);
    const double E = wave_sum_f64(a) / 64.0;
    if (!(E < best)) break;                                           // the same value in every lane
    best = E;
    zb = z;
    const double tau = pow(beta, -1.0 / (1.0 - pm1));                 // threshold of the shrink
    double e = 0.0;
    if (a >= tau * (1.0 - 1e-9)) e = copysign(fmax(a - pow(a, pm1) / beta, 0.0), r);
    const double zn = wave_sum_f64((double)qv - (vd - e) / sd) / 64.0;
    z = f16_bits_to_f32(f64_to_f16_bits(zn));
    beta = beta * (double)hp.kappa;
  }
  return zb;
}

// One wavefront per 64-value group: lane l holds value l of the group.
// Min and max come from wave reductions (then the zero is refined if
// hp.iters > 0); the code of every lane is packed into the tiled field order
// (format.h) by shuffles.  fp32 arithmetic with IEEE division and rint (ties
// to even) so the codes equal any other IEEE fp32 evaluation of the same
// formula bit for bit.
template <int BITS>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, long ngroups, int gpr,
                                                       HqqParams hp, uint8_t* __restrict__ q,
                                                       uint32_t* __restrict__ sz) {
  using F = Fmt<BITS>;
  const int lane = threadIdx.x & 63;
  const long stride = (long)gridDim.x * 4;
  const int cpr = gpr * F::CHUNKS_PER_GROUP;
  for (long g = (long)blockIdx.x * 4 + (threadIdx.x >> 6); g < ngroups; g += stride) {
    const float v = w[g * 64 + lane];
    const GroupQuant gq = minmax_group<BITS>(v);
    const uint32_t s16 = gq.s16;
    uint32_t z16 = gq.z16;
    float zf = gq.zf;
    if (!gq.degenerate && hp.iters > 0) {
      zf = hqq_zero(v, gq.sf, zf, gq.qmax, hp);
      z16 = f32_to_f16_bits(zf);                     // exact: zf is an fp16 value
    }
    const uint32_t code = group_code(gq, v, zf);
    const long row = g / gpr;
    const int gi = (int)(g % gpr);
    if constexpr (BITS == 4) {
      // lanes 0..31: byte b of chunk k (32 codes) holds fields 2b, 2b+1
      const int k = (lane >> 4) & 1, b = lane & 15;
      const uint32_t lo = __shfl(code, 32 * k + field_code<4>(2 * b));
      const uint32_t hi = __shfl(code, 32 * k + field_code<4>(2 * b + 1));
      if (lane < 32) q[chunk_offset<4>(row, 2 * gi + k, cpr) + b] = (uint8_t)(lo | (hi << 4));
    } else if constexpr (BITS == 6) {
      // lanes 0..15: 24-bit word i of chunk k holds fields 4i..4i+3
      const int k = (lane >> 2) & 3, i = lane & 3;
      uint32_t word = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) word |= __shfl(code, 16 * k + field_code<6>(4 * i + m)) << (6 * m);
      if (lane < 16) {
        uint8_t* dst = q + chunk_offset<6>(row, 4 * gi + k, cpr) + 3 * i;
        dst[0] = (uint8_t)(word & 0xFF);
        dst[1] = (uint8_t)((word >> 8) & 0xFF);
        dst[2] = (uint8_t)((word >> 16) & 0xFF);
      }
    } else {
      q[chunk_offset<8>(row, 4 * gi + (lane >> 4), cpr) + (lane & 15)] = (uint8_t)code;
    }
    if (lane == 0) sz[sz_index(row, gi, gpr)] = s16 | (z16 << 16);
  }
}

// One thread per chunk (in memory order): load, turn into bf16 pairs exactly
// as the decode kernels do, and write the codes back in natural order.
template <int BITS>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ q, long nchunks, int cpr, int K,
                                                     uint8_t* __restrict__ codes) {
  using F = Fmt<BITS>;
  for (long m = (long)blockIdx.x * blockDim.x + threadIdx.x; m < nchunks; m += (long)gridDim.x * blockDim.x) {
    const long tile = m / (64L * cpr), rem = m % (64L * cpr);
    const long row = tile * 64 + rem % 64;
    const long c = rem / 64;
    uint32_t d[F::DW];
    load_chunk<BITS>(q + m * F::BYTES, d);
    uint32_t P[F::PAIRS];
    chunk_pairs<BITS>(d, P);
    uint8_t* out = codes + row * K + c * F::CODES;
#pragma unroll
    for (int p = 0; p < F::PAIRS; ++p) {
      out[pair_code<BITS>(p, 0)] = (uint8_t)(bf16_bits_to_f32(P[p] & 0xFFFFu) - F::OFFSET);
      out[pair_code<BITS>(p, 1)] = (uint8_t)(bf16_bits_to_f32(P[p] >> 16) - F::OFFSET);
    }
  }
}

static int grid_for(long work, int per_block) {
  long b = (work + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > 65536) b = 65536;
  return (int)b;
}

static int quantize_impl(const float* w, long rows, int K, int bits, HqqParams hp, uint8_t* q, uint32_t* sz,
                         hipStream_t stream) {
  if (!w || !q || !sz) return set_error(MOEQ_ERR_INVALID_ARG, "moe_quantize: NULL pointer");
  if (rows < 0 || K <= 0) return set_error(MOEQ_ERR_INVALID_ARG, "moe_quantize: rows=%ld K=%d", rows, K);
  if (!bits_ok(bits)) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_quantize: bits=%d not in {4,6,8}", bits);
  if (K % MOEQ_GROUP) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_quantize: K=%d not a multiple of 64", K);
  if (rows % 64) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_quantize: rows=%ld not a multiple of 64", rows);
  if (!aligned16(w) || !aligned16(q)) return set_error(MOEQ_ERR_MISALIGNED, "moe_quantize: w and q must be 16-byte aligned");
  if (((uintptr_t)sz & 3u) != 0) return set_error(MOEQ_ERR_MISALIGNED, "moe_quantize: sz must be 4-byte aligned");
  const long ngroups = rows * (K / MOEQ_GROUP);
  if (ngroups == 0) return MOEQ_OK;
  const int grid = grid_for(ngroups, 4);
  switch (bits) {
    case 4: quantize_kernel<4><<<grid, 256, 0, stream>>>(w, ngroups, K / 64, hp, q, sz); break;
    case 6: quantize_kernel<6><<<grid, 256, 0, stream>>>(w, ngroups, K / 64, hp, q, sz); break;
    default: quantize_kernel<8><<<grid, 256, 0, stream>>>(w, ngroups, K / 64, hp, q, sz); break;
  }
  return check_launch("moe_quantize");
}

extern "C" int moe_quantize(const float* w, long rows, int K, int bits, uint8_t* q, uint32_t* sz,
                            hipStream_t stream) {
  return quantize_impl(w, rows, K, bits, HqqParams{1.0f, 1.0f, 1.0f, 0}, q, sz, stream);
}

extern "C" int moe_quantize_hqq(const float* w, long rows, int K, int bits, float lp, float beta, float kappa,
                                int iters, uint8_t* q, uint32_t* sz, hipStream_t stream) {
  if (!(lp > 0.0f && lp <= 1.0f) || !(beta > 0.0f && beta < INFINITY) || !(kappa >= 1.0f && kappa < INFINITY) ||
      iters < 0 || iters > 1000)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_quantize_hqq: lp=%g beta=%g kappa=%g iters=%d", (double)lp,
                     (double)beta, (double)kappa, iters);
  return quantize_impl(w, rows, K, bits, HqqParams{lp, beta, kappa, iters}, q, sz, stream);
}

extern "C" int moe_unpack(const uint8_t* q, long rows, int K, int bits, uint8_t* codes, hipStream_t stream) {
  if (!q || !codes) return set_error(MOEQ_ERR_INVALID_ARG, "moe_unpack: NULL pointer");
  if (rows < 0 || K <= 0) return set_error(MOEQ_ERR_INVALID_ARG, "moe_unpack: rows=%ld K=%d", rows, K);
  if (!bits_ok(bits)) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_unpack: bits=%d not in {4,6,8}", bits);
  if (K % MOEQ_GROUP) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_unpack: K=%d not a multiple of 64", K);
  if (rows % 64) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_unpack: rows=%ld not a multiple of 64", rows);
  if (!aligned16(q)) return set_error(MOEQ_ERR_MISALIGNED, "moe_unpack: q must be 16-byte aligned");
  const long ncodes = rows * (long)K;
  if (ncodes == 0) return MOEQ_OK;
  switch (bits) {
    case 4: unpack_kernel<4><<<grid_for(ncodes / 32, 256), 256, 0, stream>>>(q, ncodes / 32, K / 32, K, codes); break;
    case 6: unpack_kernel<6><<<grid_for(ncodes / 16, 256), 256, 0, stream>>>(q, ncodes / 16, K / 16, K, codes); break;
    default: unpack_kernel<8><<<grid_for(ncodes / 16, 256), 256, 0, stream>>>(q, ncodes / 16, K / 16, K, codes); break;
  }
  return check_launch("moe_unpack");
}
