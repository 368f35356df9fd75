// Decode kernels instantiated for 8-bit weights (see decode_impl.h and
// decode_fused.h).
#include "decode_fused.h"

// one launch per (W, CW) shape that covers whole groups at this width
#define MOEQ_LAUNCH_GU(W_, CW_)                                                                        \
  if constexpr (CW_ % Fmt<8>::CHUNKS_PER_GROUP == 0 && CW_ / Fmt<8>::CHUNKS_PER_GROUP <= 8)           \
  if (W == W_ && CW == CW_) {                                                                          \
    decode_detail::gateup_rows_kernel<8, W_, CW_><<<grid, 64 * W_, 0, s>>>(                          \
        L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, dg, offsets, sorted, active, hh);     \
    launched = true;                                                                                   \
  }
#define MOEQ_LAUNCH_DN(W_, CW_)                                                                        \
  if constexpr (CW_ % Fmt<8>::CHUNKS_PER_GROUP == 0 && CW_ / Fmt<8>::CHUNKS_PER_GROUP <= 8)           \
  if (W == W_ && CW == CW_) {                                                                          \
    decode_detail::down_rows_kernel<8, W_, CW_><<<grid, 64 * W_, 0, s>>>(                            \
        L->down.q, L->down.sz, hh, L->H, L->I, dg, offsets, sorted, active, y);                        \
    launched = true;                                                                                   \
  }
#define MOEQ_LAUNCH_GU_LIST(W_, CW_)                                                                   \
  if constexpr (CW_ % Fmt<8>::CHUNKS_PER_GROUP == 0 && CW_ / Fmt<8>::CHUNKS_PER_GROUP <= 8)           \
  if (W == W_ && CW == CW_) {                                                                          \
    decode_detail::gateup_list_kernel<8, W_, CW_><<<grid, 64 * W_, 0, s>>>(                          \
        L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, dg, offsets, sorted, active, hh);     \
    launched = true;                                                                                   \
  }
#define MOEQ_LAUNCH_DN_LIST(W_, CW_)                                                                   \
  if constexpr (CW_ % Fmt<8>::CHUNKS_PER_GROUP == 0 && CW_ / Fmt<8>::CHUNKS_PER_GROUP <= 8)           \
  if (W == W_ && CW == CW_) {                                                                          \
    decode_detail::down_list_kernel<8, W_, CW_><<<grid, 64 * W_, 0, s>>>(                            \
        L->down.q, L->down.sz, hh, L->H, L->I, dg, offsets, sorted, active, y);                        \
    launched = true;                                                                                   \
  }
namespace moeq {
MOEQ_DEFINE_DECODE(8)
MOEQ_DEFINE_DECODE_FUSED(8)
}  // namespace moeq
