// Router logits and top-k routing.
//
// Small batches (decode): a GEMV-style kernel; each wave owns expert rows of
// the router weight and streams them once, the token activations are staged
// in LDS one K-slice at a time and shared by the block's waves.
// Large batches (prefill): the bf16 matrix-core GEMM of gemm_bf16.h.
// Then one wavefront per token selects the top k (value desc, index asc) and
// computes the renormalised softmax weights.
#include "format.h"
#include "gemm_bf16.h"

using namespace moeq;

namespace {

constexpr int kRouterRowsPerWave = 2;
constexpr int kRouterWaves = 4;
constexpr int kRouterRows = kRouterRowsPerWave * kRouterWaves;   // expert rows per block
constexpr int kRouterSlice = 1024;                               // H columns per LDS slice
constexpr int kRouterTok = 8;                                    // tokens per pass

// logits[t][e] = sum_h x[t][h] * wr[e][h] (+ bias[e]); fp32 accumulation.
__global__ __launch_bounds__(256) void router_gemv_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          const float* __restrict__ bias, int T, int H,
                                                          int E, float* __restrict__ logits) {
  __shared__ uint32_t xs[kRouterTok][kRouterSlice / 2];   // bf16 pairs, 16 KB
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row0 = blockIdx.x * kRouterRows + wave * kRouterRowsPerWave;
  for (int t0 = 0; t0 < T; t0 += kRouterTok) {
    const int nt = min(kRouterTok, T - t0);
    float acc[kRouterRowsPerWave][kRouterTok];
#pragma unroll
    for (int r = 0; r < kRouterRowsPerWave; ++r)
#pragma unroll
      for (int t = 0; t < kRouterTok; ++t) acc[r][t] = 0.0f;
    for (int h0 = 0; h0 < H; h0 += kRouterSlice) {
      const int hs = min(kRouterSlice, H - h0);       // multiple of 64
      __syncthreads();
      // stage x[t0..t0+nt)[h0..h0+hs) as uint32 pairs
      for (int i = threadIdx.x; i < nt * (hs / 2); i += blockDim.x) {
        const int t = i / (hs / 2), c = i % (hs / 2);
        xs[t][c] = reinterpret_cast<const uint32_t*>(x + (size_t)(t0 + t) * H + h0)[c];
      }
      __syncthreads();
      // each lane takes 8 columns (16 bytes) per step
      for (int c = lane * 8; c < hs; c += 512) {
#pragma unroll
        for (int r = 0; r < kRouterRowsPerWave; ++r) {
          const int e = row0 + r;
          if (e >= E) continue;
          const moeq_u32x4 w4 = *reinterpret_cast<const moeq_u32x4*>(wr + (size_t)e * H + h0 + c);
#pragma unroll
          for (int t = 0; t < kRouterTok; ++t) {
            if (t < nt) {
              const uint32_t* xp = &xs[t][c / 2];
              float a = acc[r][t];
              a = dot2_bf16(w4.x, xp[0], a);
              a = dot2_bf16(w4.y, xp[1], a);
              a = dot2_bf16(w4.z, xp[2], a);
              a = dot2_bf16(w4.w, xp[3], a);
              acc[r][t] = a;
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kRouterRowsPerWave; ++r) {
      const int e = row0 + r;
#pragma unroll
      for (int t = 0; t < kRouterTok; ++t) {
        const float s = group_sum_last<64>(acc[r][t]);
        if (lane == 63 && e < E && t < nt) logits[(size_t)(t0 + t) * E + e] = s + (bias ? bias[e] : 0.0f);
      }
    }
  }
}

// (value, index) ordering of the selection: larger value first, then lower index.
constexpr int kMaxSlots = 64;   // E <= 64 * 64 candidates per wave

// One wavefront per token.  Lane l holds experts l, l+64, ...; k rounds of a
// wave arg-max, the owner lane then drops the winner from its candidates.
template <int NS>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                   int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* L = logits + (size_t)t * E;
  float v[NS];
  uint64_t taken = 0;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? L[e] : -INFINITY;
    if (e >= E) taken |= 1ull << i;
  }
  float top0 = 0.0f;
  float wsum = 0.0f;
  int32_t* idx_row = idx_out + (size_t)t * k;
  float* w_row = w_out + (size_t)t * k;
  for (int j = 0; j < k; ++j) {
    float bv;
    const int be = wave_topk_next<NS>(v, taken, bv);   // the same on every lane
    if (j == 0) top0 = bv;
    const float ex = expf(bv - top0);
    wsum += ex;
    if (lane == (j & 63)) { idx_row[j] = be; w_row[j] = ex; }   // normalised below
  }
  for (int j = lane; j < k; j += 64) w_row[j] = w_row[j] / wsum;   // entries this lane wrote
}

// The same selection with lane l holding experts NS l .. NS l + NS - 1
// (select_token: one ballot a round instead of one a slot), for k <= 64 and
// E <= 1024; the same choices, and the weights formed the same way (expf,
// summed in choice order, one division each).
template <int NS>
__global__ __launch_bounds__(256) void topk_keys_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                        int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int idx;
  float w;
  select_token<NS, true>(logits + (size_t)t * E, E, k, k, idx, w);
  if (lane < k) {
    idx_out[(size_t)t * k + lane] = idx;
    w_out[(size_t)t * k + lane] = w;
  }
}

}  // namespace

extern "C" int moe_route_topk(const uint16_t* x, const uint16_t* w_router, const float* bias, int T, int H,
                              int E, int k, float* logits, int32_t* topk_idx, float* topk_w, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (T < 0 || E <= 0 || k <= 0) return set_error(MOEQ_ERR_INVALID_ARG, "moe_route_topk: T=%d E=%d k=%d", T, E, k);
  if (k > E) return set_error(MOEQ_ERR_INVALID_ARG, "moe_route_topk: k=%d > E=%d", k, E);
  if (E > 64 * kMaxSlots) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_route_topk: E=%d > %d", E, 64 * kMaxSlots);
  if (!w_router && bias) return set_error(MOEQ_ERR_INVALID_ARG, "moe_route_topk: bias given without router weights");
  if (w_router && (H <= 0 || H % 64))
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_route_topk: H=%d not a positive multiple of 64", H);
  if (T == 0) return MOEQ_OK;
  if (!logits || !topk_idx || !topk_w) return set_error(MOEQ_ERR_INVALID_ARG, "moe_route_topk: NULL output");
  if (w_router) {
    if (!x) return set_error(MOEQ_ERR_INVALID_ARG, "moe_route_topk: x is NULL");
    if (H <= 0 || H % 64) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_route_topk: H=%d not a positive multiple of 64", H);
    if (!aligned16(x) || !aligned16(w_router))
      return set_error(MOEQ_ERR_MISALIGNED, "moe_route_topk: x and w_router must be 16-byte aligned");
  }
  if (w_router) {
    if (T >= kGemmMinTokens) {
      int rc = gemm_bf16_nt(x, w_router, bias, T, E, H, logits, stream);
      if (rc != MOEQ_OK) return rc;
    } else {
      const int grid = (E + kRouterRows - 1) / kRouterRows;
      router_gemv_kernel<<<grid, 256, 0, stream>>>(x, w_router, bias, T, H, E, logits);
      int rc = check_launch("moe_route_topk (router)");
      if (rc != MOEQ_OK) return rc;
    }
  }
  const unsigned grid = (unsigned)((T + 3) / 4);
  const int ns = (E + 63) / 64;
  if (k <= 64 && ns <= 16) {
    if (ns <= 1) topk_keys_kernel<1><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
    else if (ns <= 2) topk_keys_kernel<2><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
    else if (ns <= 4) topk_keys_kernel<4><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
    else if (ns <= 8) topk_keys_kernel<8><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
    else topk_keys_kernel<16><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
    return check_launch("moe_route_topk (top-k)");
  }
  if (ns <= 1) topk_kernel<1><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  else if (ns <= 2) topk_kernel<2><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  else if (ns <= 4) topk_kernel<4><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  else if (ns <= 8) topk_kernel<8><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  else if (ns <= 16) topk_kernel<16><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  else if (ns <= 32) topk_kernel<32><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  else topk_kernel<64><<<grid, 256, 0, stream>>>(logits, T, E, k, topk_idx, topk_w);
  return check_launch("moe_route_topk (top-k)");
}
