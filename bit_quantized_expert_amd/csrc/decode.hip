// Host side of the decode path (moe_qgemv_decode): argument checks, lane
// geometry and grid sizing.  The kernels are in decode_impl.h, instantiated
// per bit width in decode_b{4,6,8}.hip.
#include "decode_impl.h"

using namespace moeq;

namespace {

// Lane geometry for K inputs at `bits`: chunks per row CPR = K / codes-per-
// chunk; LPR = largest power of two <= 64 dividing CPR; ITER = CPR / LPR
// must be 1..4 (K up to 8192 at 4-bit, 4096 at 6/8-bit).
bool geometry(int K, int bits, int& lpr, int& iter) {
  const int codes = bits == 4 ? 32 : 16;
  if (K % codes) return false;
  const int cpr = K / codes;
  lpr = 1;
  while (lpr < 64 && cpr % (lpr * 2) == 0) lpr *= 2;
  iter = cpr / lpr;
  return iter >= 1 && iter <= 4;
}

// Rows per wave: CH chunks per lane and matrix held in registers cover
// CH / iter row steps of 64 / lpr rows (CH as in decode_impl.h).
int rows_per_wave(int lpr, int iter, bool gateup) {
  const int ch = gateup ? decode_detail::gateup_ch(iter) : decode_detail::down_ch(iter);
  return (ch / iter) * (64 / lpr);
}

}  // namespace

extern "C" int moe_qgemv_decode(const moe_layer_desc* L, const uint16_t* x, int T, const int32_t* offsets,
                                const int32_t* sorted, const int32_t* active, float* y, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  int rc = validate_layer(L);
  if (rc != MOEQ_OK) return rc;
  if (T < 0) return set_error(MOEQ_ERR_INVALID_ARG, "moe_qgemv_decode: T=%d", T);
  if (T == 0) return MOEQ_OK;
  if (!x || !offsets || !sorted || !active || !y)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_qgemv_decode: NULL pointer");
  if (!aligned16(x) || !aligned16(y))
    return set_error(MOEQ_ERR_MISALIGNED, "moe_qgemv_decode: x and y must be 16-byte aligned");
  if (L->gate.bits != L->up.bits)
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_qgemv_decode: gate and up must share a bit width");
  int lpr1, it1, lpr2, it2;
  if (!geometry(L->H, L->gate.bits, lpr1, it1) || !geometry(L->I, L->down.bits, lpr2, it2))
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_qgemv_decode: no kernel for H=%d/I=%d at these bit widths", L->H,
                     L->I);
  const WsLayout wl = ws_layout(L->H, L->I, L->E, L->S, L->k, T);
  if (!ws || ws_bytes < wl.total)
    return set_error(MOEQ_ERR_WORKSPACE, "moe_qgemv_decode: workspace of %zu bytes, need %zu", ws_bytes, wl.total);
  // h: bf16 [A][I] in the down kernel's pair order
  uint16_t* hh = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + wl.h);
  const long A = (long)T * (L->k + L->S);
  const int slots = (int)(A < L->E + L->S ? A : L->E + L->S);   // upper bound on active experts
  const int rpw1 = rows_per_wave(lpr1, it1, true);
  const int rpw2 = rows_per_wave(lpr2, it2, false);
  switch (L->gate.bits) {
    case 4: rc = decode_gateup_b4(L, x, offsets, sorted, active, slots, rpw1, lpr1, it1, hh, stream); break;
    case 6: rc = decode_gateup_b6(L, x, offsets, sorted, active, slots, rpw1, lpr1, it1, hh, stream); break;
    default: rc = decode_gateup_b8(L, x, offsets, sorted, active, slots, rpw1, lpr1, it1, hh, stream); break;
  }
  if (rc != MOEQ_OK) return rc;
  switch (L->down.bits) {
    case 4: rc = decode_down_b4(L, hh, offsets, sorted, active, slots, rpw2, lpr2, it2, y, stream); break;
    case 6: rc = decode_down_b6(L, hh, offsets, sorted, active, slots, rpw2, lpr2, it2, y, stream); break;
    default: rc = decode_down_b8(L, hh, offsets, sorted, active, slots, rpw2, lpr2, it2, y, stream); break;
  }
  return rc;
}
