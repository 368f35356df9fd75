// Decode kernels instantiated for 8-bit weights (see decode_impl.h).
#include "decode_impl.h"

namespace moeq {
MOEQ_DEFINE_DECODE(8)
}  // namespace moeq
