// The decode layer in three launches (moe_decode_forward):
//
//  1. router logits (one wavefront per router row, route_decode.hip);
//  2. selection + gate/up: one block per (routed assignment t k + j, 64-row
//     tile of I); its first wavefront makes the first j + 1 choices of token
//     t from the logits (select_token), then the block streams that
//     expert's gate and up rows for token t as gateup_rows_kernel does.  No
//     launch sits between the router and the expert GEMV, and no block
//     needs the selection of any other token.  h goes to the workspace in
//     assignment order (row t (k+S) + j);
//  3. down + combine: one block per (token, 64-row tile of H), one wavefront
//     per expert slot of the token; each wavefront streams its expert's down
//     rows over the whole of I, and the block adds the k+S results with the
//     routing weights in ascending slot order, as moe_combine does.  The
//     expert outputs never leave the chip.
//
// Removing the dependent small launches between routing, expert GEMVs and
// combine is the decode lever the pages report (Raon-1-mini on an RTX
// 5070 Ti, optimisation table).  The price: an expert that several tokens
// of the batch chose is streamed once per token, by blocks of one row tile
// that share an XCD (so mostly from its L2 after the first).
#pragma once
#include "decode_impl.h"

namespace moeq {
namespace decode_detail {

constexpr int kFusedMaxT = 64;       // tokens per batch
constexpr int kFusedMaxE = 1024;     // routed experts (select_token holds 16 per lane)
constexpr int kFusedMaxSlots = 16;   // k + S: one wavefront per slot in the down + combine block

struct FusedGrid {
  int E, S, k, T;
  int kS;              // k + S
  int tiles;           // 64-row tiles of I
  int shared_blocks;   // as DecodeGrid: S * tiles rounded up to 8, times ceil(T / 2)
  int groups;          // token pairs: ceil(T / 2)
};

MOEQ_DEV void select_token_any(const float* L, int E, int k, int rounds, int& idx, float& w) {
  const int ns = (E + 63) / 64;
  if (ns <= 1) select_token<1>(L, E, k, rounds, idx, w);
  else if (ns <= 2) select_token<2>(L, E, k, rounds, idx, w);
  else if (ns <= 4) select_token<4>(L, E, k, rounds, idx, w);
  else if (ns <= 8) select_token<8>(L, E, k, rounds, idx, w);
  else select_token<16>(L, E, k, rounds, idx, w);
}

// -------------------------------------------------------------------------
// selection + gate/up.  Grid: the shared-expert part of DecodeGrid, then one
// block per (routed assignment, row tile), T k tiles of them.  h[a][i] =
// bf16(silu(Wg x_t)[i] * (Wu x_t)[i]) for assignment a = t (k+S) + j.
// -------------------------------------------------------------------------
template <int BITS, int W, int CW>
__global__ __launch_bounds__(64 * W, 4) void gateup_routed_kernel(const uint8_t* __restrict__ gq,
                                                                  const uint32_t* __restrict__ gsz,
                                                                  const uint8_t* __restrict__ uq,
                                                                  const uint32_t* __restrict__ usz,
                                                                  const uint16_t* __restrict__ x, int H, int I,
                                                                  FusedGrid fg, const float* __restrict__ logits,
                                                                  int32_t* __restrict__ topk_idx,
                                                                  float* __restrict__ topk_w,
                                                                  uint16_t* __restrict__ hh) {
  using F = Fmt<BITS>;
  constexpr int D = CW < kDepth ? CW : kDepth;
  __shared__ Partials<W, 2> part;
  __shared__ int chosen;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = (int)blockIdx.x;
  Stream<BITS, 2> st;
  ChunkBuf<BITS, 2> buf[D];
  // weights of expert e, row tile `tile`: the first D chunk loads go out at once
  auto start = [&](int e, int tile) {
    const size_t ebytes = (size_t)I * row_bytes(H, BITS), ewords = (size_t)I * (H / 64);
    const uint8_t* const qe[2] = {gq + e * ebytes, uq + e * ebytes};
    const uint32_t* const sze[2] = {gsz + e * ewords, usz + e * ewords};
    st.init(qe, sze, H / F::CODES, H / 64, tile, wave * CW);
#pragma unroll
    for (int c = 0; c < D; ++c) st.load(c, buf[c]);
    stage_fence();
  };
  int tile, t0, t1, nt, a0, a1;
  if (b < fg.shared_blocks) {
    const int span = 8 * fg.groups;
    const int l = (b / span) * 8 + (b % 8);   // (shared expert, row tile)
    if (l >= fg.S * fg.tiles) return;
    const int pair = (b % span) / 8;
    const int s = l / fg.tiles;
    tile = l % fg.tiles;
    start(fg.E + s, tile);
    t0 = 2 * pair;
    nt = min(2, fg.T - t0);
    t1 = nt > 1 ? t0 + 1 : t0;
    a0 = t0 * fg.kS + fg.k + s;
    a1 = t1 * fg.kS + fg.k + s;
  } else {
    // wavefront 0 makes the first j + 1 choices of token t (all k, and the
    // weights, in the block that stores them for the down + combine kernel)
    const int r = b - fg.shared_blocks;
    const int a = r / fg.tiles, t = a / fg.k, j = a % fg.k;
    tile = r % fg.tiles;
    const bool writer = j == 0 && tile == 0;
    if (wave == 0) {
      int bi;
      float w;
      select_token_any(logits + (size_t)t * fg.E, fg.E, fg.k, writer ? fg.k : j + 1, bi, w);
      if (writer && lane < fg.k) {
        topk_idx[(size_t)t * fg.k + lane] = bi;
        topk_w[(size_t)t * fg.k + lane] = w;
      }
      if (lane == 0) chosen = __builtin_amdgcn_readlane(bi, j);
    }
    __syncthreads();
    start(uniform(chosen), tile);
    t0 = t1 = t;
    nt = 1;
    a0 = a1 = t * fg.kS + j;
  }
  tile = uniform(tile);
  t0 = uniform(t0);
  t1 = uniform(t1);
  nt = uniform(nt);
  const uint16_t* const xr[kMaxNT] = {x + (size_t)t0 * H, x + (size_t)t1 * H};
  float tot[2];
  block_pass<BITS, 2, W, CW>(st, buf, xr, nt, part, tot);
  if (wave < nt)
    hh[(size_t)(wave == 0 ? a0 : a1) * I + tile * 64 + lane] = (uint16_t)f32_to_bf16_bits(silu_f32(tot[0]) * tot[1]);
}

// -------------------------------------------------------------------------
// down + combine: block (token t, 64-row tile of H); wavefront j < k+S
// streams the down rows of the expert in slot j (topk_idx, or shared expert
// E + j - k) against h[t (k+S) + j] over all NG groups of I, then
// out[t][n] = bf16(sum_j w_j y_j[n]) (w_j = 1 for shared slots), summed in
// fp32 in ascending j, with the residual added as moe_combine does.
// -------------------------------------------------------------------------
template <int BITS, int NG>
__global__ __launch_bounds__(64 * kFusedMaxSlots) void down_combine_kernel(const uint8_t* __restrict__ dq,
                                                                          const uint32_t* __restrict__ dsz,
                                                                          const uint16_t* __restrict__ hh, int H,
                                                                          int I, FusedGrid fg,
                                                                          const int32_t* __restrict__ topk_idx,
                                                                          const float* __restrict__ topk_w,
                                                                          const uint16_t* __restrict__ residual,
                                                                          uint16_t* __restrict__ out) {
  using F = Fmt<BITS>;
  constexpr int CPR = NG * F::CHUNKS_PER_GROUP;
  constexpr int D = CPR < 8 ? CPR : 8;
  __shared__ float ys[kFusedMaxSlots][64];
  __shared__ float wsl[kFusedMaxSlots];
  const int lane = threadIdx.x & 63, j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // block -> (token, tile): the T blocks of one tile land on one XCD (blocks
  // are dealt to the 8 XCDs round-robin), so a weight tile that several of
  // the batch's tokens use is read from that XCD's L2 after the first
  const int tiles = H / 64, b = (int)blockIdx.x;
  int t, tile;
  if (tiles % 8 == 0) {
    const int slot = b / 8;
    tile = (slot / fg.T) * 8 + b % 8;
    t = slot % fg.T;
  } else {
    tile = b / fg.T;
    t = b % fg.T;
  }
  // the h row's loads first: its group sums need nothing else, and the
  // expert id comes meanwhile (a scalar load)
  const uint16_t* hrow = hh + (size_t)(t * fg.kS + j) * I;
  GroupX<NG> gx;
  gx.load(hrow, 0);
  const int e = uniform(j < fg.k ? topk_idx[(size_t)t * fg.k + j] : fg.E + (j - fg.k));
  Stream<BITS, 1> st;
  {
    const uint8_t* const qe[1] = {dq + e * ((size_t)H * row_bytes(I, BITS))};
    const uint32_t* const sze[1] = {dsz + e * ((size_t)H * (I / 64))};
    st.init(qe, sze, CPR, NG, tile, 0);
  }
  ChunkBuf<BITS, 1> buf[D];
#pragma unroll
  for (int c = 0; c < D; ++c) st.load(c, buf[c]);
  stage_fence();
  const float wj = j < fg.k ? topk_w[(size_t)t * fg.k + j] : 1.0f;
  const uint16_t* const xr[kMaxNT] = {hrow, hrow};
  float xs[kMaxNT] = {gx.sum(), 0.0f};
  stage_fence();
  float y[1][kMaxNT];
  stream_rows<BITS, 1, 1, CPR, D>(st, buf, xr, xs, y);
  ys[j][lane] = y[0][0];
  if (lane == 0) wsl[j] = wj;
  __syncthreads();
  if (j == 0) {
    float acc = 0.0f;
    for (int s = 0; s < fg.kS; ++s) acc = fmaf(wsl[s], ys[s][lane], acc);
    const size_t o = (size_t)t * H + tile * 64 + lane;
    uint32_t ob = f32_to_bf16_bits(acc);
    if (residual) ob = f32_to_bf16_bits(bf16_bits_to_f32(residual[o]) + bf16_bits_to_f32(ob));
    out[o] = (uint16_t)ob;
  }
}

}  // namespace decode_detail

// Launchers per bit width (decode_b{4,6,8}.hip).
#define MOEQ_DECODE_FUSED_LAUNCHERS(B)                                                                     \
  int decode_gateup_routed_b##B(const moe_layer_desc* L, const uint16_t* x, const float* logits, int T,     \
                                int W, int CW, int32_t* topk_idx, float* topk_w, uint16_t* hh,             \
                                hipStream_t s);                                                            \
  int decode_down_combine_b##B(const moe_layer_desc* L, const uint16_t* hh, int T, const int32_t* topk_idx, \
                               const float* topk_w, const uint16_t* residual, uint16_t* out, hipStream_t s)

MOEQ_DECODE_FUSED_LAUNCHERS(4);
MOEQ_DECODE_FUSED_LAUNCHERS(6);
MOEQ_DECODE_FUSED_LAUNCHERS(8);

inline decode_detail::FusedGrid fused_grid(const moe_layer_desc* L, int T) {
  decode_detail::FusedGrid fg;
  fg.E = L->E;
  fg.S = L->S;
  fg.k = L->k;
  fg.T = T;
  fg.kS = L->k + L->S;
  fg.tiles = L->I / 64;
  fg.groups = (T + 1) / 2;
  fg.shared_blocks = L->S > 0 ? (L->S * fg.tiles + 7) / 8 * 8 * fg.groups : 0;
  return fg;
}

// One down + combine launch: I / 64 groups in {4, 8, 12}, and 16 at 4 bits
// (the 6- and 8-bit rows of I = 1024 would not fit the registers of a
// 1024-thread block without spilling).
template <int B>
int launch_down_combine(const moe_layer_desc* L, const uint16_t* hh, int T, const int32_t* topk_idx,
                        const float* topk_w, const uint16_t* residual, uint16_t* out, hipStream_t s) {
  const decode_detail::FusedGrid fg = fused_grid(L, T);
  const int grid = T * (L->H / 64), threads = 64 * fg.kS;
  auto go = [&](auto ng) {
    decode_detail::down_combine_kernel<B, decltype(ng)::value><<<grid, threads, 0, s>>>(
        L->down.q, L->down.sz, hh, L->H, L->I, fg, topk_idx, topk_w, residual, out);
  };
  switch (L->I / 64) {
    case 4: go(std::integral_constant<int, 4>()); break;
    case 8: go(std::integral_constant<int, 8>()); break;
    case 12: go(std::integral_constant<int, 12>()); break;
    case 16:
      if constexpr (B == 4) {
        go(std::integral_constant<int, 16>());
        break;
      }
      [[fallthrough]];
    default:
      return set_error(MOEQ_ERR_UNSUPPORTED, "moe_decode_forward: I=%d at %d bits not supported", L->I, B);
  }
  return check_launch("moe_decode_forward (down + combine)");
}

#define MOEQ_DEFINE_DECODE_FUSED(B)                                                                        \
  int decode_gateup_routed_b##B(const moe_layer_desc* L, const uint16_t* x, const float* logits, int T,     \
                                int W, int CW, int32_t* topk_idx, float* topk_w, uint16_t* hh,             \
                                hipStream_t s) {                                                           \
    const decode_detail::FusedGrid fg = fused_grid(L, T);                                                  \
    const int grid = fg.shared_blocks + T * L->k * fg.tiles;                                               \
    bool launched = false;                                                                                 \
    MOEQ_DECODE_SHAPES(MOEQ_LAUNCH_GUR)                                                                    \
    if (!launched) return set_error(MOEQ_ERR_UNSUPPORTED, "decode: no gate/up kernel for W=%d CW=%d", W, CW); \
    return check_launch("moe_decode_forward (routing + gate/up)");                                         \
  }                                                                                                        \
  int decode_down_combine_b##B(const moe_layer_desc* L, const uint16_t* hh, int T, const int32_t* topk_idx, \
                               const float* topk_w, const uint16_t* residual, uint16_t* out, hipStream_t s) { \
    return launch_down_combine<B>(L, hh, T, topk_idx, topk_w, residual, out, s);                           \
  }

}  // namespace moeq
