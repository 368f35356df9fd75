// Decode kernels instantiated for 6-bit weights (see decode_impl.h).
#include "decode_impl.h"

namespace moeq {
MOEQ_DEFINE_DECODE(6)
}  // namespace moeq
