// Routing-weighted combine of the expert outputs, optional residual add,
// and the RMSNorm used between stacked blocks.
#include "common.h"

using namespace moeq;

namespace {

// One thread per 8 consecutive outputs of one token; slots summed in
// ascending order in fp32.
template <bool F32>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ yv, const float* __restrict__ w,
                                                      const uint16_t* __restrict__ residual, int T, int k, int S,
                                                      int H, uint16_t* __restrict__ out) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int per_tok = H / 8;
  if (i >= (long)T * per_tok) return;
  const int t = (int)(i / per_tok), n = (int)(i % per_tok) * 8;
  const int kS = k + S;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  for (int j = 0; j < kS; ++j) {
    const float wt = j < k ? w[(size_t)t * k + j] : 1.0f;
    const size_t row = (size_t)t * kS + j;
    float v[8];
    if constexpr (F32) {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(yv) + row * H + n);
      const float4 a = p[0], b = p[1];
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
      const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(yv) + row * H + n);
      const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        v[2 * c] = bf16_bits_to_f32(d[c] & 0xFFFFu);
        v[2 * c + 1] = bf16_bits_to_f32(d[c] >> 16);
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = fmaf(wt, v[c], acc[c]);
  }
  uint32_t o[4];
  if (residual) {
    const uint4 r = *reinterpret_cast<const uint4*>(residual + (size_t)t * H + n);
    const uint32_t rd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float lo = bf16_bits_to_f32(rd[c] & 0xFFFFu) + bf16_bits_to_f32(f32_to_bf16_bits(acc[2 * c]));
      const float hi = bf16_bits_to_f32(rd[c] >> 16) + bf16_bits_to_f32(f32_to_bf16_bits(acc[2 * c + 1]));
      o[c] = f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = f32_to_bf16_bits(acc[2 * c]) | (f32_to_bf16_bits(acc[2 * c + 1]) << 16);
  }
  *reinterpret_cast<uint4*>(out + (size_t)t * H + n) = make_uint4(o[0], o[1], o[2], o[3]);
}

// One block per row.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ g,
                                                      int H, float eps, uint16_t* __restrict__ out) {
  __shared__ float part[4];
  const uint16_t* xr = x + (size_t)blockIdx.x * H;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < H; i += 256) {
    const float v = bf16_bits_to_f32(xr[i]);
    ss = fmaf(v, v, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += 256) {
    float v = bf16_bits_to_f32(xr[i]) * r;
    if (g) v *= bf16_bits_to_f32(g[i]);
    out[(size_t)blockIdx.x * H + i] = (uint16_t)f32_to_bf16_bits(v);
  }
}

}  // namespace

extern "C" int moe_combine(const void* y, int y_dtype, const float* topk_w, const uint16_t* residual, int T, int k,
                           int S, int H, uint16_t* out, hipStream_t stream) {
  if (T < 0 || k <= 0 || S < 0 || H <= 0) return set_error(MOEQ_ERR_INVALID_ARG, "moe_combine: T=%d k=%d S=%d H=%d", T, k, S, H);
  if (H % 8) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_combine: H=%d not a multiple of 8", H);
  if (y_dtype != MOEQ_Y_F32 && y_dtype != MOEQ_Y_BF16) return set_error(MOEQ_ERR_INVALID_ARG, "moe_combine: y_dtype=%d", y_dtype);
  if (T == 0) return MOEQ_OK;
  if (!y || !topk_w || !out) return set_error(MOEQ_ERR_INVALID_ARG, "moe_combine: NULL pointer");
  if (!aligned16(y) || !aligned16(out) || (residual && !aligned16(residual)))
    return set_error(MOEQ_ERR_MISALIGNED, "moe_combine: y, residual and out must be 16-byte aligned");
  const long n = (long)T * (H / 8);
  const int grid = (int)((n + 255) / 256);
  if (y_dtype == MOEQ_Y_F32) combine_kernel<true><<<grid, 256, 0, stream>>>(y, topk_w, residual, T, k, S, H, out);
  else combine_kernel<false><<<grid, 256, 0, stream>>>(y, topk_w, residual, T, k, S, H, out);
  return check_launch("moe_combine");
}

extern "C" int moe_rmsnorm(const uint16_t* x, const uint16_t* gamma, int T, int H, float eps, uint16_t* out,
                           hipStream_t stream) {
  if (T < 0 || H <= 0 || !(eps >= 0.0f)) return set_error(MOEQ_ERR_INVALID_ARG, "moe_rmsnorm: T=%d H=%d eps=%g", T, H, (double)eps);
  if (T == 0) return MOEQ_OK;
  if (!x || !out) return set_error(MOEQ_ERR_INVALID_ARG, "moe_rmsnorm: NULL pointer");
  if (x == out) return set_error(MOEQ_ERR_INVALID_ARG, "moe_rmsnorm: x and out may not alias");
  rmsnorm_kernel<<<T, 256, 0, stream>>>(x, gamma, H, eps, out);
  return check_launch("moe_rmsnorm");
}
