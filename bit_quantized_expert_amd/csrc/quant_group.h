// Min-max affine quantisation of one 64-value group held by one wavefront
// (lane l holds value l), shared by the weight quantiser and the KV-cache
// codec.  fp32 with IEEE division and rint (ties to even):
//   s16 = fp16(fp32(max - min) / (2^bits - 1)),  z16 = fp16(-min / s16),
//   q   = clamp(rint(w / s16 + z16), 0, 2^bits - 1);
// a group whose s16 is zero stores s16 = 1, z16 = fp16(-min), q = 0.
#pragma once
#include "common.h"

namespace moeq {

struct GroupQuant {
  uint32_t s16, z16;   // fp16 bits
  float sf, zf;        // their values
  float qmax;
  bool degenerate;
};

// From the group's minimum and maximum.
template <int BITS>
MOEQ_DEV GroupQuant minmax_from(float mn, float mx) {
  GroupQuant g;
  g.qmax = (float)((1 << BITS) - 1);
  const float s = (mx - mn) / g.qmax;
  g.s16 = f32_to_f16_bits(s);
  g.degenerate = (g.s16 & 0x7FFFu) == 0;
  if (g.degenerate) g.s16 = 0x3C00u;   // fp16 1.0
  g.sf = f16_bits_to_f32(g.s16);
  g.z16 = f32_to_f16_bits(-mn / g.sf);
  g.zf = f16_bits_to_f32(g.z16);
  return g;
}

template <int BITS>
MOEQ_DEV GroupQuant minmax_group(float v) {
  return minmax_from<BITS>(wave_min(v), wave_max(v));
}

// The code of value v for zero z (an fp16 value) of group g.
MOEQ_DEV uint32_t group_code(const GroupQuant& g, float v, float z) {
  const float r = fminf(fmaxf(rintf(v / g.sf + z), 0.0f), g.qmax);
  return g.degenerate ? 0u : (uint32_t)r;
}

}  // namespace moeq
