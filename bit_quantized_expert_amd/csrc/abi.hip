// Host-side plumbing of the C ABI: thread-local last error, workspace layout
// and sizing, layer validation, status read-back.
#include "common.h"

#include <string.h>

namespace moeq {

static thread_local char g_err[512] = "";

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(MOEQ_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return MOEQ_OK;
}

int perm_blocks(long A) { return (int)((A + kPermBlock - 1) / kPermBlock); }

long prefill_max_tiles(long A, int nexp) {
  // sum_e ceil(c_e / BM) <= A / BM + number of experts
  return A / kPrefillBM + nexp + 1;
}

WsLayout ws_layout(int H, int I, int E, int S, int k, int T_max) {
  WsLayout w{};
  long A = (long)T_max * (k + S);
  int nexp = E + S;
  size_t off = 0;
  w.status = off;
  off += 256;
  w.perm_hist = off;
  off = align_up(off + (size_t)perm_blocks(A) * nexp * sizeof(int32_t), 256);
  w.sched = off;
  off = align_up(off + (size_t)(prefill_max_tiles(A, nexp) + 4) * 2 * sizeof(int32_t), 256);
  w.h = off;
  off = align_up(off + (size_t)A * I * sizeof(float), 256);   // fp32 covers bf16 too
  w.shared_part = off;   // [S][T][slice][gate, up][I]
  const long Tf = T_max < kFusedMaxTokens ? T_max : kFusedMaxTokens;
  off = align_up(off + (size_t)S * Tf * kSharedMaxSplit * 2 * I * sizeof(float), 256);
  w.norm = off;          // [T][H] bf16, decode batches
  off = align_up(off + (size_t)Tf * H * sizeof(uint16_t), 256);
  w.gemv = off;
  off = align_up(off + (size_t)(nexp + 1) * sizeof(int32_t), 256);
  w.total = off;
  return w;
}

int validate_layer(const moe_layer_desc* L) {
  if (!L) return set_error(MOEQ_ERR_INVALID_ARG, "layer descriptor is NULL");
  if (L->H <= 0 || L->I <= 0 || L->E <= 0 || L->S < 0 || L->k <= 0)
    return set_error(MOEQ_ERR_INVALID_ARG, "layer sizes must be positive (H=%d I=%d E=%d S=%d k=%d)",
                     L->H, L->I, L->E, L->S, L->k);
  if (L->k > L->E) return set_error(MOEQ_ERR_INVALID_ARG, "k=%d exceeds E=%d", L->k, L->E);
  if (L->E + L->S > 4096) return set_error(MOEQ_ERR_UNSUPPORTED, "E+S=%d exceeds 4096", L->E + L->S);
  if (L->H % MOEQ_GROUP || L->I % MOEQ_GROUP)
    return set_error(MOEQ_ERR_UNSUPPORTED, "H=%d and I=%d must be multiples of %d", L->H, L->I, MOEQ_GROUP);
  // kernels address one expert's matrix with 32-bit byte offsets
  if ((long long)L->H * L->I >= (1LL << 31))
    return set_error(MOEQ_ERR_UNSUPPORTED, "H*I=%lld: one expert matrix must stay below 2^31 weights",
                     (long long)L->H * L->I);
  const moe_qweight* ws[3] = {&L->gate, &L->up, &L->down};
  const char* nm[3] = {"gate", "up", "down"};
  for (int i = 0; i < 3; ++i) {
    if (!ws[i]->q || !ws[i]->sz) return set_error(MOEQ_ERR_INVALID_ARG, "%s weights are NULL", nm[i]);
    if (!bits_ok(ws[i]->bits))
      return set_error(MOEQ_ERR_UNSUPPORTED, "%s bits=%d not in {4,6,8}", nm[i], ws[i]->bits);
    if (!aligned16(ws[i]->q) || !aligned16(ws[i]->sz))
      return set_error(MOEQ_ERR_MISALIGNED, "%s weights must be 16-byte aligned", nm[i]);
  }
  return MOEQ_OK;
}

}  // namespace moeq

using namespace moeq;

extern "C" size_t moe_workspace_bytes(const moe_layer_desc* L, int T_max) {
  if (validate_layer(L) != MOEQ_OK || T_max < 0) return 0;
  return ws_layout(L->H, L->I, L->E, L->S, L->k, T_max).total;
}

extern "C" const char* moe_last_error(void) { return g_err; }

extern "C" int moe_workspace_h(const moe_layer_desc* L, int T_max, size_t* offset) {
  int rc = validate_layer(L);
  if (rc != MOEQ_OK) return rc;
  if (T_max < 0 || !offset) return set_error(MOEQ_ERR_INVALID_ARG, "moe_workspace_h: T_max=%d or NULL offset", T_max);
  *offset = ws_layout(L->H, L->I, L->E, L->S, L->k, T_max).h;
  return MOEQ_OK;
}

extern "C" int moe_read_status(const void* ws, size_t ws_bytes, int* n_bad_ids, hipStream_t stream) {
  if (!ws || !n_bad_ids) return set_error(MOEQ_ERR_INVALID_ARG, "NULL workspace or output");
  if (ws_bytes < 256) return set_error(MOEQ_ERR_WORKSPACE, "workspace smaller than its status block");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return set_error(MOEQ_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
  int v = 0;
  e = hipMemcpy(&v, ws, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return set_error(MOEQ_ERR_HIP, "hipMemcpy: %s", hipGetErrorString(e));
  *n_bad_ids = v;
  return MOEQ_OK;
}
