// One router row's logits for a decode batch, computed by one wavefront:
// logits[t][e] = sum_h x[t][h] Wr[e][h] (+ bias[e]) in fp32 (dot2 of bf16
// pairs, DPP reduction).  The row (H = 512 NCH bf16) is loaded once into
// registers; the tokens come straight from global memory (they stay in L2)
// in groups whose loads are all issued before the first use.
#pragma once
#include "format.h"

namespace moeq {

// tokens whose activations are loaded together (at most 128 registers of
// them; TG overrides it where fewer registers are free)
constexpr int router_tok_group(int nch) { return nch <= 4 ? 8 : 4; }

template <int NCH, int TG = router_tok_group(NCH)>
MOEQ_DEV void router_row(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                         const float* __restrict__ bias, int T, int E, int e, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  constexpr int H = NCH * 512;
  moeq_u32x4 w4[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) w4[i] = *reinterpret_cast<const moeq_u32x4*>(wr + (size_t)e * H + 8 * (lane + 64 * i));
  const float be = bias ? bias[e] : 0.0f;
  constexpr int kTokGroup = TG;
  for (int t0 = 0; t0 < T; t0 += kTokGroup) {
    moeq_u32x4 xv[kTokGroup][NCH];
#pragma unroll
    for (int u = 0; u < kTokGroup; ++u) {
      const int t = min(t0 + u, T - 1);   // past the end: repeat the last token, never stored
#pragma unroll
      for (int i = 0; i < NCH; ++i)
        xv[u][i] = *reinterpret_cast<const moeq_u32x4*>(x + (size_t)t * H + 8 * (lane + 64 * i));
    }
#pragma unroll
    for (int u = 0; u < kTokGroup; ++u) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        a = dot2_bf16(w4[i].x, xv[u][i].x, a);
        a = dot2_bf16(w4[i].y, xv[u][i].y, a);
        a = dot2_bf16(w4[i].z, xv[u][i].z, a);
        a = dot2_bf16(w4[i].w, xv[u][i].w, a);
      }
      a = group_sum_last<64>(a);
      if (lane == 63 && t0 + u < T) logits[(size_t)(t0 + u) * E + e] = a + be;
    }
  }
}

}  // namespace moeq
