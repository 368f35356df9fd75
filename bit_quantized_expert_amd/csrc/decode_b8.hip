// Decode kernels instantiated for 8-bit weights (see decode_impl.h).
#include "decode_impl.h"

#define MOEQ_GATEUP_CALL(IT, LP)                                                                          \
  switch (L->down.bits) {                                                                                 \
    case 4: decode_detail::gateup_gemv_kernel<8, 4, IT, LP><<<grid, 256, 0, s>>>(GATEUP_ARGS); break;     \
    case 6: decode_detail::gateup_gemv_kernel<8, 6, IT, LP><<<grid, 256, 0, s>>>(GATEUP_ARGS); break;     \
    default: decode_detail::gateup_gemv_kernel<8, 8, IT, LP><<<grid, 256, 0, s>>>(GATEUP_ARGS); break;    \
  }
#define GATEUP_ARGS \
  L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, L->k + L->S, offsets, sorted, active, tiles, hh
#define MOEQ_DOWN_CALL(IT, LP)                                                                            \
  decode_detail::down_gemv_kernel<8, IT, LP><<<grid, 256, 0, s>>>(L->down.q, L->down.sz, hh, L->H,  \
                                                                   L->I, offsets, sorted, active, tiles, y)

namespace moeq {
MOEQ_DEFINE_DECODE(8)
}  // namespace moeq
