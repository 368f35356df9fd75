// Decode kernels instantiated for 4-bit weights (see decode_impl.h).
#include "decode_impl.h"

namespace moeq {
MOEQ_DEFINE_DECODE(4)
}  // namespace moeq
