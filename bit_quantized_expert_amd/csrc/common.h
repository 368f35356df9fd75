// Internal helpers shared by the libmoeq translation units: error reporting,
// workspace layout and small device functions (bf16/fp16 conversion, wave
// reductions).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <stdarg.h>
#include <stdio.h>
#include <limits.h>

#include "moeq.h"

// --------------------------------------------------------------------------
// host side: error reporting and validation
// --------------------------------------------------------------------------
namespace moeq {

int set_error(int code, const char* fmt, ...);
int check_launch(const char* what);   // hipGetLastError after a launch

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool bits_ok(int b) { return b == 4 || b == 6 || b == 8; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// bytes of one packed row of K codes
__host__ __device__ inline size_t row_bytes(int K, int bits) { return (size_t)K * bits / 8; }

// Workspace layout for a layer and a maximum batch.  All regions are
// 256-byte aligned; `total` is what moe_workspace_bytes reports.
struct WsLayout {
  size_t status;     // int32 status words (n_bad ids ...)
  size_t perm_hist;  // int32 [perm_blocks][E+S] block histograms
  size_t h;          // decode: fp32 [A][I]; prefill: bf16 [A][I]
  size_t sched;      // prefill: int32 tile schedule
  size_t shared_part;   // moe_decode_forward: fp32 partial gate/up sums of the shared experts
  size_t norm;          // moe_decode_block: the normalised token rows, bf16
  size_t gemv;          // prefill: int32 [1 + E + S] experts taking the GEMV path (count, ids)
  size_t total;
};
constexpr int kPermBlock = 1024;          // assignments per permute block
constexpr int kPrefillBM = 128;           // prefill token tile
constexpr int kFusedMaxTokens = 64;       // moe_decode_forward batches
constexpr int kSharedMaxSplit = 16;       // moe_decode_forward: K slices of a shared-expert row
#ifndef MOEQ_PREFILL_GEMV_MAX
#define MOEQ_PREFILL_GEMV_MAX 2
#endif
#ifndef MOEQ_PREFILL_GEMV_MIN
#define MOEQ_PREFILL_GEMV_MIN 64
#endif
constexpr int kPrefillGemvMax = MOEQ_PREFILL_GEMV_MAX;   // prefill: experts with at most this many assignments take the GEMV path,
constexpr int kPrefillGemvMin = MOEQ_PREFILL_GEMV_MIN;   // when a batch has at least this many of them
int perm_blocks(long A);
long prefill_max_tiles(long A, int nexp);
WsLayout ws_layout(int H, int I, int E, int S, int k, int T_max);
int validate_layer(const moe_layer_desc* L);
// Router logits of a decode batch, one wavefront per router row (H in
// {512, 1024, 2048, 4096}, checked by the caller).
int launch_router_rows(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H, int E,
                       float* logits, hipStream_t stream);

}  // namespace moeq

// --------------------------------------------------------------------------
// device side
// --------------------------------------------------------------------------
#define MOEQ_DEV __device__ __forceinline__
#define MOEQ_HD __host__ __device__ __forceinline__

MOEQ_DEV float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs)
MOEQ_DEV uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

MOEQ_DEV float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

MOEQ_DEV uint32_t f32_to_f16_bits(float f) {   // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int CTRL>
MOEQ_DEV float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of `span` lanes (span in {1,2,4,...,64}); every lane
// of a group ends with the group's sum.  DPP within a row of 16 lanes,
// ds_swizzle / bpermute across rows.
MOEQ_DEV float group_sum(float v, int span) {
  if (span >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  if (span >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  if (span >= 8) v += dpp_f<0x141>(v);   // row_half_mirror
  if (span >= 16) v += dpp_f<0x140>(v);  // row_mirror
  if (span >= 32) v += __shfl_xor(v, 16);
  if (span >= 64) v += __shfl_xor(v, 32);
  return v;
}

MOEQ_DEV float wave_sum(float v) { return group_sum(v, 64); }

template <int CTRL, int ROW_MASK>
MOEQ_DEV float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                                  0xF, false));
}

// Sum over aligned groups of SPAN lanes (SPAN a power of two <= 64) with DPP
// only -- no branches, no LDS permutes.  The group's sum is valid in the
// group's last lane (lane % SPAN == SPAN - 1); other lanes hold partials.
template <int SPAN>
MOEQ_DEV float group_sum_last(float v) {
  if constexpr (SPAN >= 2) v = dpp_add<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  if constexpr (SPAN >= 4) v = dpp_add<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  if constexpr (SPAN >= 8) v = dpp_add<0x141, 0xF>(v);   // row_half_mirror
  if constexpr (SPAN >= 16) v = dpp_add<0x140, 0xF>(v);  // row_mirror: whole row of 16
  if constexpr (SPAN >= 32) v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  if constexpr (SPAN >= 64) v = dpp_add<0x143, 0x8>(v);  // row_bcast:31 into row 3
  return v;
}

MOEQ_DEV float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
MOEQ_DEV float wave_min(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}

template <int CTRL, int ROW_MASK>
MOEQ_DEV float dpp_max(float v) {
  const int ninf = __builtin_bit_cast(int, -INFINITY);   // rows the mask leaves out contribute -inf
  return fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(ninf, __builtin_bit_cast(int, v), CTRL,
                                                                       ROW_MASK, 0xF, false)));
}

// Wave maximum with DPP (NaN-ignoring like fmaxf), returned on every lane.
MOEQ_DEV float wave_max_dpp(float v) {
  v = dpp_max<0xB1, 0xF>(v);
  v = dpp_max<0x4E, 0xF>(v);
  v = dpp_max<0x141, 0xF>(v);
  v = dpp_max<0x140, 0xF>(v);
  v = dpp_max<0x142, 0xA>(v);
  v = dpp_max<0x143, 0x8>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// One round of top-k selection over the candidates a wave holds: lane l,
// slot i holds expert 64 i + l with value v[i]; bit i of `taken` marks slots
// already chosen or past the last expert.  Returns the next expert in the
// routing order (larger value first, ties to the lower index; NaN after every
// number, in index order), the same on every lane, marks it taken on its
// lane, and sets `best` to its value.  Branch-free apart from uniform scalar
// tests: a DPP maximum, then one ballot per slot finds the lowest index that
// holds it.
template <int NS>
MOEQ_DEV int wave_topk_next(const float (&v)[NS], uint64_t& taken, float& best) {
  static_assert(NS <= 64, "at most 64 slots per lane");
  const int lane = threadIdx.x & 63;
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < NS; ++i) m = ((taken >> i) & 1u) ? m : fmaxf(m, v[i]);
  m = wave_max_dpp(m);
  int slot = -1;
  uint64_t hit = 0;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const uint64_t b = __ballot(!((taken >> i) & 1u) && v[i] == m);
    if (slot < 0 && b) { slot = i; hit = b; }
  }
  best = m;
  if (slot < 0) {   // only NaN left
    best = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const uint64_t b = __ballot(!((taken >> i) & 1u));
      if (slot < 0 && b) { slot = i; hit = b; }
    }
  }
  const int l = __builtin_ctzll(hit);
  if (lane == l) taken |= 1ull << slot;
  return 64 * slot + l;
}

// Selection keys: a signed integer per logit whose order is the routing
// order of the values (larger first); -0 counts as +0, NaN below every
// number, and kKeyGone (padding, already chosen) below NaN.
constexpr int kKeyGone = INT_MIN;
constexpr int kKeyNaN = INT_MIN + 1;
MOEQ_DEV int logit_key(float f) {
  if (f != f) return kKeyNaN;
  const int b = __float_as_int(f + 0.0f);   // -0 + 0 = +0
  return b >= 0 ? b : b ^ 0x7FFFFFFF;
}
MOEQ_DEV float key_value(int key) {
  if (key == kKeyNaN) return __builtin_nanf("");
  return __int_as_float(key >= 0 ? key : key ^ 0x7FFFFFFF);
}

template <int CTRL, int ROW_MASK>
MOEQ_DEV int dpp_max_i32(int v) {
  return max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, CTRL, ROW_MASK, 0xF, false));
}

// Wave maximum of an int with DPP, returned (uniform) from lane 63.
MOEQ_DEV int wave_max_i32(int v) {
  v = dpp_max_i32<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  v = dpp_max_i32<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  v = dpp_max_i32<0x141, 0xF>(v);   // row_half_mirror
  v = dpp_max_i32<0x140, 0xF>(v);   // row_mirror
  v = dpp_max_i32<0x142, 0xA>(v);   // row_bcast:15
  v = dpp_max_i32<0x143, 0x8>(v);   // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// The top k of one token's E logits, by one wavefront, and their softmax
// weights renormalised over the k chosen: w_j = e^(l_j - l_0) /
// sum_i e^(l_i - l_0), l_0 the largest.  Lane l holds experts NS l ..
// NS l + NS - 1, so among equal values the lowest index is on the lowest
// lane holding the maximum, in its lowest slot: each of the k rounds is a
// lane maximum, a DPP wave maximum and one ballot.  Order: larger value
// first, ties to the lower index, NaN after every number (in index order).
// On return lane j < k holds choice j in idx and its weight in w (other
// lanes: -1 and 0).  Needs k <= min(E, 64).  With rounds < k only the
// first `rounds` choices are made (lanes j < rounds), and w is not valid.
// EXACT_EXP: the weights' exponentials by expf instead of the hardware
// exp2 (moe_route_topk's weights).
template <int NS, bool EXACT_EXP = false>
MOEQ_DEV void select_token(const float* __restrict__ L, int E, int k, int rounds, int& idx, float& w) {
  const int lane = threadIdx.x & 63;
  int key[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = NS * lane + i;
    key[i] = e < E ? logit_key(L[e]) : kKeyGone;
  }
  float top0 = 0.0f, wsum = 0.0f, myw = 0.0f;
  idx = -1;
  for (int j = 0; j < rounds; ++j) {
    int m = key[0];
#pragma unroll
    for (int i = 1; i < NS; ++i) m = max(m, key[i]);
    const int M = wave_max_i32(m);
    const int wl = __builtin_ctzll(__ballot(m == M));   // lowest lane holding the maximum
    int slot = NS - 1;
#pragma unroll
    for (int i = NS - 2; i >= 0; --i) slot = key[i] == M ? i : slot;
    const int ws = __builtin_amdgcn_readlane(slot, wl);
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i < NS; ++i) key[i] = i == ws ? kKeyGone : key[i];
    }
    const float bv = key_value(M);
    if (j == 0) top0 = bv;
    const float ex = EXACT_EXP ? expf(bv - top0) : __expf(bv - top0);
    wsum += ex;
    if (lane == j) {
      myw = ex;
      idx = NS * wl + ws;
    }
  }
  w = lane < k ? myw / wsum : 0.0f;
}

// silu(g) = g / (1 + e^-g) with the hardware exp2 and reciprocal (about
// 1 ulp each); -g*log2(e) overflowing to +inf gives rcp(inf) = 0, i.e. 0.
MOEQ_DEV float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}
