// Host side of the decode path (moe_qgemv_decode, moe_decode_forward):
// argument checks, block shape and grid sizing.  The kernels are in
// decode_impl.h and decode_fused.h, instantiated per bit width in
// decode_b{4,6,8}.hip.
#include "decode_fused.h"

#include <mutex>

using namespace moeq;

// Scratch of moe_decode_forward_noalloc: a fixed array in device memory that
// every GPU holds one copy of from the time the library's code is loaded on
// it until the process ends.  Host code never passes the array's name to a
// kernel (in host code it only names the symbol): it passes the device
// address hipGetSymbolAddress returns for the current device, kept below.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

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
  int w1, cw1, w2, cw2;
  if (!pick_shape(L->H, L->gate.bits, MOEQ_GATEUP_RUN, w1, cw1) ||
      !pick_shape(L->I, L->down.bits, MOEQ_DOWN_RUN, w2, cw2))
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_qgemv_decode: no kernel for H=%d/I=%d at these bit widths", L->H,
                     L->I);
  const WsLayout wl = ws_layout(L->H, L->I, L->E, L->S, L->k, T);
  if (!ws || ws_bytes < wl.total)
    return set_error(MOEQ_ERR_WORKSPACE, "moe_qgemv_decode: workspace of %zu bytes, need %zu", ws_bytes, wl.total);
  // h: bf16 [A][I], rows in sorted order
  uint16_t* hh = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + wl.h);
  switch (L->gate.bits) {
    case 4: rc = decode_gateup_b4(L, x, offsets, sorted, active, T, w1, cw1, hh, stream); break;
    case 6: rc = decode_gateup_b6(L, x, offsets, sorted, active, T, w1, cw1, hh, stream); break;
    default: rc = decode_gateup_b8(L, x, offsets, sorted, active, T, w1, cw1, hh, stream); break;
  }
  if (rc != MOEQ_OK) return rc;
  switch (L->down.bits) {
    case 4: rc = decode_down_b4(L, hh, offsets, sorted, active, T, w2, cw2, y, stream); break;
    case 6: rc = decode_down_b6(L, hh, offsets, sorted, active, T, w2, cw2, y, stream); break;
    default: rc = decode_down_b8(L, hh, offsets, sorted, active, T, w2, cw2, y, stream); break;
  }
  return rc;
}

namespace {

// moe_decode_forward's body; norm.xraw != nullptr for moe_decode_block
// (then x is where launch 1 stores the normalised rows).
int decode_forward_impl(const char* fn, const moe_layer_desc* L, const uint16_t* x, const uint16_t* w_router,
                        const float* bias, int T, const uint16_t* residual, float* logits, int32_t* topk_idx,
                        float* topk_w, uint16_t* out, void* ws, size_t ws_bytes, decode_detail::NormArgs norm,
                        hipStream_t stream) {
  using namespace decode_detail;
  int rc = validate_layer(L);
  if (rc != MOEQ_OK) return rc;
  if (T < 0) return set_error(MOEQ_ERR_INVALID_ARG, "%s: T=%d", fn, T);
  if (T == 0) return MOEQ_OK;
  const int H = L->H, I = L->I, E = L->E, S = L->S, k = L->k;
  if (T > kFusedMaxT || E > kFusedMaxE || k + S > kFusedMaxSlots)
    return set_error(MOEQ_ERR_UNSUPPORTED, "%s: needs T <= %d, E <= %d and k+S <= %d (T=%d E=%d k=%d S=%d)", fn,
                     kFusedMaxT, kFusedMaxE, kFusedMaxSlots, T, E, k, S);
  if (H != 512 && H != 1024 && H != 2048 && H != 4096)
    return set_error(MOEQ_ERR_UNSUPPORTED, "%s: H=%d must be 512, 1024, 2048 or 4096", fn, H);
  if (I != 256 && I != 512 && I != 768 && I != 1024)
    return set_error(MOEQ_ERR_UNSUPPORTED, "%s: I=%d must be 256, 512, 768 or 1024", fn, I);
  if (L->gate.bits != L->up.bits)
    return set_error(MOEQ_ERR_UNSUPPORTED, "%s: gate and up must share a bit width", fn);
  if (!(norm.xraw || x) || !w_router || !logits || !topk_idx || !topk_w || !out)
    return set_error(MOEQ_ERR_INVALID_ARG, "%s: NULL pointer", fn);
  if (!aligned16(norm.xraw ? norm.xraw : x) || !aligned16(w_router))
    return set_error(MOEQ_ERR_MISALIGNED, "%s: x and w_router must be 16-byte aligned", fn);
  const WsLayout wl = ws_layout(H, I, E, S, k, T);
  if (!ws || ws_bytes < wl.total)
    return set_error(MOEQ_ERR_WORKSPACE, "%s: workspace of %zu bytes, need %zu", fn, ws_bytes, wl.total);
  // h: bf16 [T (k+S)][I], rows in assignment order
  uint16_t* hh = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + wl.h);
  float* spart = reinterpret_cast<float*>(static_cast<char*>(ws) + wl.shared_part);
  if (norm.xraw) {
    norm.nout = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + wl.norm);
    x = norm.nout;
  }
  const bool nm = norm.xraw != nullptr;
  switch (L->gate.bits) {
    case 4: rc = decode_router_shared_b4(L, x, w_router, bias, T, logits, spart, norm, stream); break;
    case 6: rc = decode_router_shared_b6(L, x, w_router, bias, T, logits, spart, norm, stream); break;
    default: rc = decode_router_shared_b8(L, x, w_router, bias, T, logits, spart, norm, stream); break;
  }
  if (rc != MOEQ_OK) return rc;
  switch (L->gate.bits) {
    case 4: rc = decode_gateup_routed_b4(L, x, logits, spart, T, topk_idx, topk_w, hh, nm, stream); break;
    case 6: rc = decode_gateup_routed_b6(L, x, logits, spart, T, topk_idx, topk_w, hh, nm, stream); break;
    default: rc = decode_gateup_routed_b8(L, x, logits, spart, T, topk_idx, topk_w, hh, nm, stream); break;
  }
  if (rc != MOEQ_OK) return rc;
  switch (L->down.bits) {
    case 4: rc = decode_down_combine_b4(L, hh, T, topk_idx, topk_w, residual, out, stream); break;
    case 6: rc = decode_down_combine_b6(L, hh, T, topk_idx, topk_w, residual, out, stream); break;
    default: rc = decode_down_combine_b8(L, hh, T, topk_idx, topk_w, residual, out, stream); break;
  }
  return rc;
}

}  // namespace

extern "C" int moe_decode_forward(const moe_layer_desc* L, const uint16_t* x, const uint16_t* w_router,
                                  const float* bias, int T, const uint16_t* residual, float* logits,
                                  int32_t* topk_idx, float* topk_w, uint16_t* out, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  return decode_forward_impl("moe_decode_forward", L, x, w_router, bias, T, residual, logits, topk_idx, topk_w, out,
                             ws, ws_bytes, decode_detail::NormArgs{nullptr, 0.0f, nullptr}, stream);
}

extern "C" int moe_decode_block(const moe_layer_desc* L, uint16_t* x, const uint16_t* w_router, const float* bias,
                                int T, float eps, float* logits, int32_t* topk_idx, float* topk_w, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
  if (!x) return set_error(MOEQ_ERR_INVALID_ARG, "moe_decode_block: NULL pointer");
  if (!(eps >= 0.0f)) return set_error(MOEQ_ERR_INVALID_ARG, "moe_decode_block: eps=%g", (double)eps);
  return decode_forward_impl("moe_decode_block", L, nullptr, w_router, bias, T, x, logits, topk_idx, topk_w, x, ws,
                             ws_bytes, decode_detail::NormArgs{x, eps, nullptr}, stream);
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];   // scratch's device address, per device

// The current device's address of `scratch`, looked up once per device with
// that device current.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(MOEQ_ERR_HIP, "moe_decode_forward_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_decode_forward_noalloc: device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(MOEQ_ERR_HIP, "moe_decode_forward_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOEQ_OK;
}

}  // namespace

extern "C" size_t moe_decode_forward_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

extern "C" int moe_decode_forward_noalloc(const moe_layer_desc* L, const uint16_t* x, const uint16_t* w_router,
                                          const float* bias, int T, const uint16_t* residual, float* logits,
                                          int32_t* topk_idx, float* topk_w, uint16_t* out, hipStream_t stream) {
  int rc = validate_layer(L);
  if (rc != MOEQ_OK) return rc;
  if (T < 0 || T > decode_detail::kFusedMaxT)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_decode_forward_noalloc: T=%d (0 <= T <= %d)", T, decode_detail::kFusedMaxT);
  const size_t need = ws_layout(L->H, L->I, L->E, L->S, L->k, T).total;
  if (need > kNoAllocScratchBytes)
    return set_error(MOEQ_ERR_WORKSPACE,
                     "moe_decode_forward_noalloc: this layer at T=%d needs %zu bytes of scratch; the static scratch "
                     "holds %zu (use moe_decode_forward with a workspace)", T, need, kNoAllocScratchBytes);
  if (T == 0) return MOEQ_OK;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws)) != MOEQ_OK) return rc;
  return decode_forward_impl("moe_decode_forward_noalloc", L, x, w_router, bias, T, residual, logits, topk_idx, topk_w,
                             out, ws, kNoAllocScratchBytes, decode_detail::NormArgs{nullptr, 0.0f, nullptr}, stream);
}
