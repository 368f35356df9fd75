// The decode layer in three launches (moe_decode_forward):
//
//  1. router + shared experts: blocks of four wavefronts, one router row per
//     wavefront (router_row), and the shared experts' gate/up rows, which
//     every token uses and so need no routing: one block per (shared
//     expert, 64-row tile, K slice, pair of tokens) writes partial sums;
//  2. selection + routed gate/up: one block per (routed assignment
//     t k + j, 64-row tile of I); its first wavefront makes the first j + 1
//     choices of token t from the logits (select_token), then the block
//     streams that expert's gate and up rows for token t as
//     gateup_rows_kernel does.  Meanwhile the blocks of slot 0 add up the
//     shared experts' slices for their token and tile into h.  No launch
//     sits between the router and the expert GEMV, no block needs the
//     selection of any other token, and every block carries the same work,
//     T k tiles of them (shared-expert tiles here would leave some CUs one
//     block more than the rest, and the launch waiting on those);
//  3. down + combine: one block per (token, 64-row tile of H), one wavefront
//     per expert slot of the token; each wavefront streams its expert's down
//     rows over the whole of I, and the block adds the k+S results with the
//     routing weights in ascending slot order, as moe_combine does.  The
//     expert outputs never leave the chip.
// h goes through the workspace in assignment order (row t (k+S) + j).
//
// Removing the dependent small launches between routing, expert GEMVs and
// combine is the decode lever the pages report (Raon-1-mini on an RTX
// 5070 Ti, optimisation table).  The price: an expert that several tokens
// of the batch chose is streamed once per token, by blocks of one row tile
// that share an XCD (so mostly from its L2 after the first).
#pragma once
#include "decode_impl.h"
#include "router.h"
#include "rows8.h"

namespace moeq {
namespace decode_detail {

constexpr int kFusedMaxT = kFusedMaxTokens;   // tokens per batch
constexpr int kFusedMaxE = 1024;     // routed experts (select_token holds 16 per lane)
constexpr int kFusedMaxSlots = 16;   // k + S: one wavefront per slot in the down + combine block

constexpr int cmax_i(int a, int b) { return a > b ? a : b; }

// Gate/up block shape of the fused path for rows of H codes: W wavefronts
// of CW chunks each; 16-chunk runs (8 at H = 512, 4-bit), so that blocks are
// short in wavefronts and several share a CU.
template <int BITS, int NCH>
struct FusedShape {
  static constexpr int CPR = NCH * 512 / Fmt<BITS>::CODES;
#ifndef MOEQ_FUSED_RUN
#define MOEQ_FUSED_RUN 16
#endif
  static constexpr int CW = CPR >= 2 * MOEQ_FUSED_RUN ? cmax_i(MOEQ_FUSED_RUN, CPR / 16) : CPR / 2;
  static constexpr int W = CPR / CW;
  static_assert(W * CW == CPR && W <= 16 && CW % Fmt<BITS>::CHUNKS_PER_GROUP == 0, "shape");
};

// Shared-expert gate/up in launch 1: blocks of four wavefronts of CW = 4
// chunks each, so a block covers one K slice of 16 chunks; Q slices per row.
template <int BITS, int NCH>
struct SharedShape {
  static constexpr int W = 4, CW = 4;
  static constexpr int Q = NCH * 512 / Fmt<BITS>::CODES / (W * CW);
  static_assert(Q >= 1 && Q <= kSharedMaxSplit && CW % Fmt<BITS>::CHUNKS_PER_GROUP == 0, "shape");
};

struct FusedGrid {
  int E, S, k, T;
  int kS;              // k + S
  int tiles;           // 64-row tiles of I
  int router_blocks;   // launch 1: blocks of four router rows (a multiple of 8)
  int shared_blocks;   // launch 1: S tiles Q slices rounded up to 8, times ceil(T / 2)
  int shared_late;     // shared experts in launch 2 instead (whole rows, as extra blocks)
  int late_blocks;     // launch 2: S tiles rounded up to 8, times ceil(T / 2), if shared_late
  int Q;               // K slices of a shared-expert row
  int groups;          // token pairs: ceil(T / 2)
};

// RMSNorm of the raw residual rows inside launch 1 (moe_decode_block): every
// router block normalises the token rows itself, block 0 also stores them
// for the later launches.  xraw == nullptr: the input is already normalised.
struct NormArgs {
  const uint16_t* xraw;   // [T][H] bf16
  float eps;
  uint16_t* nout;         // [T][H] bf16
};

MOEQ_DEV void select_token_any(const float* L, int E, int k, int rounds, int& idx, float& w) {
  const int ns = (E + 63) / 64;
  if (ns <= 1) select_token<1>(L, E, k, rounds, idx, w);
  else if (ns <= 2) select_token<2>(L, E, k, rounds, idx, w);
  else if (ns <= 4) select_token<4>(L, E, k, rounds, idx, w);
  else if (ns <= 8) select_token<8>(L, E, k, rounds, idx, w);
  else select_token<16>(L, E, k, rounds, idx, w);
}

// One block's gate/up tile: rows tile*64 .. +63 of expert e's gate and up
// matrices for up to two tokens, h = bf16(silu(g) u) stored to h rows a0
// (and a1).  start() issues the first loads; finish() streams the rest.
template <int BITS, int W, int CW>
struct GateupTile {
  using F = Fmt<BITS>;
  static constexpr int D = CW < kDepth ? CW : kDepth;
  Stream<BITS, 2> st;
  ChunkBuf<BITS, 2> buf[D];
  int tile;
  MOEQ_DEV void start(const uint8_t* gq, const uint32_t* gsz, const uint8_t* uq, const uint32_t* usz, int H, int I,
                      int e, int tile_) {
    tile = tile_;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t ebytes = (size_t)I * row_bytes(H, BITS), ewords = (size_t)I * (H / 64);
    const uint8_t* const qe[2] = {gq + e * ebytes, uq + e * ebytes};
    const uint32_t* const sze[2] = {gsz + e * ewords, usz + e * ewords};
    st.init(qe, sze, H / F::CODES, H / 64, tile, wave * CW);
#pragma unroll
    for (int c = 0; c < D; ++c) st.load(c, buf[c]);
    stage_fence();
  }
  MOEQ_DEV void finish(const uint16_t* x, int H, int I, int t0, int t1, int nt, int a0, int a1,
                       Partials<W, 2>& part, uint16_t* hh) {
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    t0 = uniform(t0);
    t1 = uniform(t1);
    nt = uniform(nt);
    const uint16_t* const xr[kMaxNT] = {x + (size_t)t0 * H, x + (size_t)t1 * H};
    float tot[2];
    block_pass<BITS, 2, W, CW>(st, buf, xr, nt, part, tot);
    if (wave < nt)
      hh[(size_t)(wave == 0 ? a0 : a1) * I + tile * 64 + lane] = (uint16_t)f32_to_bf16_bits(silu_f32(tot[0]) * tot[1]);
  }
};

// -------------------------------------------------------------------------
// launch 1: router rows, then the shared experts' gate/up slices: block
// (shared expert s, row tile, K slice q, token pair) writes, for each of
// its tokens t, the slice's sums part[s][t][q][gate, up][row] (fp32).  The
// pairs of one (s, tile, q) land on one XCD a few dispatches apart, so the
// weights they all read come from its L2 after the first.
// -------------------------------------------------------------------------
template <int BITS, int NCH>
__global__ __launch_bounds__(256) void router_shared_kernel(const uint16_t* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            const uint8_t* __restrict__ gq,
                                                            const uint32_t* __restrict__ gsz,
                                                            const uint8_t* __restrict__ uq,
                                                            const uint32_t* __restrict__ usz,
                                                            const uint16_t* __restrict__ x, int I, FusedGrid fg,
                                                            float* __restrict__ logits, float* __restrict__ spart,
                                                            NormArgs norm) {
  using Sh = SharedShape<BITS, NCH>;
  constexpr int H = NCH * 512;
  __shared__ Partials<Sh::W, 2> part;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = (int)blockIdx.x;
  if (b < fg.router_blocks) {
    const int e = b * 4 + wave;
    if (norm.xraw) {
      // token by token: n = bf16(x / sqrt(mean(x^2) + eps)) as moe_rmsnorm
      // forms it (the same sums in the same order), then the router rows
      __shared__ __attribute__((aligned(16))) uint16_t nrow[H];
      __shared__ float red[4];
      for (int t = 0; t < fg.T; ++t) {
        const uint16_t* xr = norm.xraw + (size_t)t * H;
        float ss = 0.0f;
        for (int i = threadIdx.x; i < H; i += 256) {
          const float v = bf16_bits_to_f32(xr[i]);
          ss = fmaf(v, v, ss);
        }
        ss = wave_sum(ss);
        if (lane == 0) red[wave] = ss;
        __syncthreads();
        const float tot = (red[0] + red[1]) + (red[2] + red[3]);
        const float r = 1.0f / sqrtf(tot / (float)H + norm.eps);
        for (int i = threadIdx.x; i < H; i += 256) {
          const uint16_t n = (uint16_t)f32_to_bf16_bits(bf16_bits_to_f32(xr[i]) * r);
          nrow[i] = n;
          if (b == 0) norm.nout[(size_t)t * H + i] = n;
        }
        __syncthreads();
        if (e < fg.E) router_row<NCH, 1>(nrow, wr, bias, 1, fg.E, e, logits + (size_t)t * fg.E);
        __syncthreads();   // nrow and red are rewritten for the next token
      }
      return;
    }
    if (e < fg.E) router_row<NCH>(x, wr, bias, fg.T, fg.E, e, logits);
    return;
  }
  const int bs = b - fg.router_blocks;
  const int span = 8 * fg.groups;
  const int l = (bs / span) * 8 + (bs % 8);   // (shared expert, row tile, slice)
  if (l >= fg.S * fg.tiles * Sh::Q) return;
  const int pair = (bs % span) / 8;
  const int s = l / (fg.tiles * Sh::Q), tile = (l / Sh::Q) % fg.tiles, q = l % Sh::Q;
  Stream<BITS, 2> st;
  ChunkBuf<BITS, 2> buf[Sh::CW];
  {
    const size_t ebytes = (size_t)I * row_bytes(H, BITS), ewords = (size_t)I * (H / 64);
    const int e = fg.E + s;
    const uint8_t* const qe[2] = {gq + e * ebytes, uq + e * ebytes};
    const uint32_t* const sze[2] = {gsz + e * ewords, usz + e * ewords};
    st.init(qe, sze, H / Fmt<BITS>::CODES, H / 64, tile, (q * Sh::W + wave) * Sh::CW);
#pragma unroll
    for (int c = 0; c < Sh::CW; ++c) st.load(c, buf[c]);
    stage_fence();
  }
  const int t0 = 2 * pair, nt = uniform(min(2, fg.T - t0)), t1 = nt > 1 ? t0 + 1 : t0;
  const uint16_t* const xr[kMaxNT] = {x + (size_t)t0 * H, x + (size_t)t1 * H};
  float tot[2];
  block_pass<BITS, 2, Sh::W, Sh::CW>(st, buf, xr, nt, part, tot);
  if (wave < nt) {
    float* p = spart + ((((size_t)s * fg.T + t0 + wave) * Sh::Q + q) * 2) * I + tile * 64 + lane;
    p[0] = tot[0];
    p[I] = tot[1];
  }
}

// -------------------------------------------------------------------------
// launch 2: selection + routed gate/up, one block per (routed assignment,
// row tile), T k tiles of them.  h[a][i] = bf16(silu(Wg x_t)[i] *
// (Wu x_t)[i]) for assignment a = t (k+S) + j.  The blocks of slot 0 also
// finish the shared experts' h rows of their token and tile from launch 1's
// slices (summed in slice order).
// -------------------------------------------------------------------------
template <int BITS, int NCH>
__global__ __launch_bounds__((64 * FusedShape<BITS, NCH>::W), 4) void gateup_routed_kernel(
    const uint8_t* __restrict__ gq, const uint32_t* __restrict__ gsz, const uint8_t* __restrict__ uq,
    const uint32_t* __restrict__ usz, const uint16_t* __restrict__ x, int I, FusedGrid fg,
    const float* __restrict__ logits, const float* __restrict__ spart, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, uint16_t* __restrict__ hh) {
  using Sh = FusedShape<BITS, NCH>;
  static_assert(Sh::W >= 2, "a second wavefront finishes the shared rows");
  constexpr int H = NCH * 512;
  __shared__ Partials<Sh::W, 2> part;
  __shared__ int chosen;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = (int)blockIdx.x;
  GateupTile<BITS, Sh::W, Sh::CW> gt;
  const int routed = fg.T * fg.k * fg.tiles;
  if (b >= routed) {
    // a shared expert's tile for a pair of tokens, whole rows (small
    // batches: the launch has CUs to spare); the pairs of one tile on one
    // XCD a few dispatches apart
    const int bs = b - routed, span = 8 * fg.groups;
    const int l = (bs / span) * 8 + (bs % 8);
    if (l >= fg.S * fg.tiles) return;
    const int pair = (bs % span) / 8, s = l / fg.tiles;
    gt.start(gq, gsz, uq, usz, H, I, fg.E + s, l % fg.tiles);
    const int t0 = 2 * pair, nt = min(2, fg.T - t0), t1 = nt > 1 ? t0 + 1 : t0;
    gt.finish(x, H, I, t0, t1, nt, t0 * fg.kS + fg.k + s, t1 * fg.kS + fg.k + s, part, hh);
    return;
  }
  const int a = b / fg.tiles, t = a / fg.k, j = a % fg.k, tile = b % fg.tiles;
  // wavefront 0 makes the first j + 1 choices of token t (all k, and the
  // weights, in the block that stores them for the down + combine kernel)
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
  } else if (wave == 1 && j == 0 && !fg.shared_late) {
    for (int s = 0; s < fg.S; ++s) {
      const float* p = spart + (((size_t)s * fg.T + t) * fg.Q * 2) * I + tile * 64 + lane;
      float g = 0.0f, u = 0.0f;
      for (int q = 0; q < fg.Q; ++q) {
        g += p[(size_t)q * 2 * I];
        u += p[(size_t)q * 2 * I + I];
      }
      hh[(size_t)(t * fg.kS + fg.k + s) * I + tile * 64 + lane] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
    }
  }
  __syncthreads();
  gt.start(gq, gsz, uq, usz, H, I, uniform(chosen), tile);
  gt.finish(x, H, I, t, t, 1, t * fg.kS + j, t * fg.kS + j, part, hh);
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

// -------------------------------------------------------------------------
// Small batches (T <= kRows8MaxT): launches 2 and 3 as whole-row units of
// eight rows (rows8.h), so that one token's work spreads over every CU
// instead of one block per 64-row tile streaming whole rows of H or I.
//  2'. block (token t, slot j, eight rows of I): wavefront 0 makes the first
//      j + 1 choices of token t (shared slots j >= k: expert E + j - k), the
//      block computes the eight rows' gate and up sums over all of H and
//      stores h = bf16(silu(g) u) of them;
//  3'. block (token t, eight rows of H): every (slot, 64-group of I) item of
//      the eight rows, times its slot's routing weight (1 for shared slots),
//      summed over the block in a fixed order; out = bf16(y), with the
//      residual added as moe_combine adds it.
// The shared experts are slots of launch 2' (launch 1 is the router only).
// -------------------------------------------------------------------------
#ifndef MOEQ_ROWS8_MAX_T
#define MOEQ_ROWS8_MAX_T 2
#endif
constexpr int kRows8MaxT = MOEQ_ROWS8_MAX_T;

// n bf16 values from src into LDS dst (8 per thread and pass) with their
// 64-group sums into gsum (8 threads per group), n a multiple of 64.
MOEQ_DEV void stage_rows(const uint16_t* __restrict__ src, int n, uint16_t* dst, float* gsum) {
  for (int i0 = 0; i0 < n; i0 += 256 * 8) {
    const int i = i0 + (int)threadIdx.x * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (i < n) v = *reinterpret_cast<const uint4*>(src + i);
    float s = 0.0f;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) s += bf16_bits_to_f32(w[c] & 0xFFFFu) + bf16_bits_to_f32(w[c] >> 16);
    s = group_sum(s, 8);
    if (i < n) {
      *reinterpret_cast<uint4*>(dst + i) = v;
      if ((threadIdx.x & 7) == 0) gsum[i / 64] = s;
    }
  }
}

// stage_rows split in two for n <= 2048 N: issue() loads this thread's
// values, finish() sums and stores them (work can go between the two)
template <int N>
struct RowStage {
  uint4 v[N];
  MOEQ_DEV void issue(const uint16_t* __restrict__ src, int n) {
#pragma unroll
    for (int p = 0; p < N; ++p) {
      const int i = p * 2048 + (int)threadIdx.x * 8;
      v[p] = i < n ? *reinterpret_cast<const uint4*>(src + i) : make_uint4(0, 0, 0, 0);
    }
  }
  MOEQ_DEV void finish(int n, uint16_t* dst, float* gsum) const {
#pragma unroll
    for (int p = 0; p < N; ++p) {
      const int i = p * 2048 + (int)threadIdx.x * 8;
      const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
      float s = 0.0f;
#pragma unroll
      for (int c = 0; c < 4; ++c) s += bf16_bits_to_f32(w[c] & 0xFFFFu) + bf16_bits_to_f32(w[c] >> 16);
      s = group_sum(s, 8);
      if (i < n) {
        *reinterpret_cast<uint4*>(dst + i) = v[p];
        if ((threadIdx.x & 7) == 0) gsum[i / 64] = s;
      }
    }
  }
};

template <int BITS, int NCH>
__global__ __launch_bounds__(256, 2) void gateup_rows8_kernel(const uint8_t* __restrict__ gq,
                                                             const uint32_t* __restrict__ gsz,
                                                             const uint8_t* __restrict__ uq,
                                                             const uint32_t* __restrict__ usz,
                                                             const uint16_t* __restrict__ x, int I, FusedGrid fg,
                                                             const float* __restrict__ logits,
                                                             int32_t* __restrict__ topk_idx,
                                                             float* __restrict__ topk_w, uint16_t* __restrict__ hh) {
  constexpr int H = NCH * 512, NG = H / 64, NGL = (NG + 31) / 32;
  __shared__ __attribute__((aligned(16))) uint16_t xs[H];
  __shared__ float xsum[NG];
  __shared__ float rsum[64];
  __shared__ int chosen;
  const int lane = threadIdx.x & 63, wave = uniform((int)threadIdx.x >> 6);
  const int r8 = lane & 7, ql = (lane >> 3) + 8 * wave;
  const int per = I / 8;
  const int u = xcd_unit((int)blockIdx.x, fg.T * fg.kS * per);
  const int a = u / per, t = a / fg.kS, j = a % fg.kS, r0 = (u % per) * 8;
  // the token's row is loaded while wavefront 0 selects
  RowStage<(H + 2047) / 2048> xst;
  xst.issue(x + (size_t)t * H, H);
  if (j < fg.k) {
    if (wave == 0) {
      const bool writer = j == 0 && r0 == 0;
      int bi;
      float w;
      select_token_any(logits + (size_t)t * fg.E, fg.E, fg.k, writer ? fg.k : j + 1, bi, w);
      if (writer && lane < fg.k) {
        topk_idx[(size_t)t * fg.k + lane] = bi;
        topk_w[(size_t)t * fg.k + lane] = w;
      }
      if (lane == 0) chosen = __builtin_amdgcn_readlane(bi, j);
    }
  } else if (threadIdx.x == 0) {
    chosen = fg.E + (j - fg.k);
  }
  xst.finish(H, xs, xsum);
  __syncthreads();
  const size_t row = (size_t)uniform(chosen) * I + r0 + r8;
  Grp G[NGL][2];
#pragma unroll
  for (int i = 0; i < NGL; ++i) {
    const int g = ql + 32 * i;
    grp_load<BITS>(G[i][0], gq, gsz, row, H, g, g < NG);
    grp_load<BITS>(G[i][1], uq, usz, row, H, g, g < NG);
  }
  float ag = 0.0f, au = 0.0f;
#pragma unroll
  for (int i = 0; i < NGL; ++i) {
    const int g = ql + 32 * i;
    if (g < NG) {
      ag += grp_dot<BITS>(G[i][0], xs + g * 64, xsum[g]);
      au += grp_dot<BITS>(G[i][1], xs + g * 64, xsum[g]);
    }
  }
  ag = sum_stride8(ag);
  au = sum_stride8(au);
  if (lane < 8) {
    rsum[wave * 16 + lane] = ag;
    rsum[wave * 16 + 8 + lane] = au;
  }
  __syncthreads();
  if (wave == 0 && lane < 8) {
    const float gs = ((rsum[lane] + rsum[16 + lane]) + rsum[32 + lane]) + rsum[48 + lane];
    const float us = ((rsum[8 + lane] + rsum[24 + lane]) + rsum[40 + lane]) + rsum[56 + lane];
    hh[(size_t)a * I + r0 + lane] = (uint16_t)f32_to_bf16_bits(silu_f32(gs) * us);
  }
}

// NGI: 64-groups of I
template <int BITS, int NGI>
__global__ __launch_bounds__(256, 2) void down_rows8_kernel(const uint8_t* __restrict__ dq,
                                                           const uint32_t* __restrict__ dsz,
                                                           const uint16_t* __restrict__ hh, int H, FusedGrid fg,
                                                           const int32_t* __restrict__ topk_idx,
                                                           const float* __restrict__ topk_w,
                                                           const uint16_t* __restrict__ residual,
                                                           uint16_t* __restrict__ out) {
  constexpr int I = NGI * 64;
  constexpr int NIL = (kFusedMaxSlots * NGI + 31) / 32;   // items per lane at most
  __shared__ __attribute__((aligned(16))) uint16_t hs[kFusedMaxSlots * I];
  __shared__ float hsum[kFusedMaxSlots * NGI];
  __shared__ float rsum[32];
  const int lane = threadIdx.x & 63, wave = uniform((int)threadIdx.x >> 6);
  const int r8 = lane & 7, ql = (lane >> 3) + 8 * wave;
  const int per = H / 8;
  const int u = xcd_unit((int)blockIdx.x, fg.T * per);
  const int t = u / per, r0 = (u % per) * 8;
  const int nIt = fg.kS * NGI;
  // the items' experts and weights, then their weights' codes; the token's
  // h rows meanwhile
  int ej[NIL];
  float wj[NIL];
#pragma unroll
  for (int i = 0; i < NIL; ++i) {
    const int idx = ql + 32 * i, j = idx / NGI;
    const bool on = idx < nIt;
    ej[i] = !on ? 0 : j < fg.k ? topk_idx[(size_t)t * fg.k + j] : fg.E + (j - fg.k);
    wj[i] = !on ? 0.0f : j < fg.k ? topk_w[(size_t)t * fg.k + j] : 1.0f;
  }
  constexpr int B = NIL < 4 ? NIL : 4;   // items in registers at once
  Grp D[B];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const int idx = ql + 32 * i;
    grp_load<BITS>(D[i], dq, dsz, (size_t)ej[i] * H + r0 + r8, I, idx % NGI, idx < nIt);
  }
  stage_rows(hh + (size_t)t * fg.kS * I, fg.kS * I, hs, hsum);
  __syncthreads();
  float acc = 0.0f;
#pragma unroll
  for (int i0 = 0; i0 < NIL; i0 += B) {
    if (i0 > 0) {
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const int idx = ql + 32 * (i0 + i);
        if (i0 + i < NIL)
          grp_load<BITS>(D[i], dq, dsz, (size_t)ej[min(i0 + i, NIL - 1)] * H + r0 + r8, I, idx % NGI, idx < nIt);
      }
    }
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const int idx = ql + 32 * (i0 + i);
      if (i0 + i < NIL && idx < nIt) {
        const int j = idx / NGI, g = idx % NGI;
        acc = fmaf(wj[min(i0 + i, NIL - 1)], grp_dot<BITS>(D[i], hs + j * I + g * 64, hsum[j * NGI + g]), acc);
      }
    }
  }
  acc = sum_stride8(acc);
  if (lane < 8) rsum[wave * 8 + lane] = acc;
  __syncthreads();
  if (wave == 0 && lane < 8) {
    const float y = ((rsum[lane] + rsum[8 + lane]) + rsum[16 + lane]) + rsum[24 + lane];
    const size_t o = (size_t)t * H + r0 + lane;
    uint32_t ob = f32_to_bf16_bits(y);
    if (residual) ob = f32_to_bf16_bits(bf16_bits_to_f32(residual[o]) + bf16_bits_to_f32(ob));
    out[o] = (uint16_t)ob;
  }
}

}  // namespace decode_detail

// Launchers per bit width (decode_b{4,6,8}.hip).
#define MOEQ_DECODE_FUSED_LAUNCHERS(B)                                                                     \
  int decode_router_shared_b##B(const moe_layer_desc* L, const uint16_t* x, const uint16_t* wr,           \
                                const float* bias, int T, float* logits, float* spart,                     \
                                decode_detail::NormArgs norm, hipStream_t s);                              \
  int decode_gateup_routed_b##B(const moe_layer_desc* L, const uint16_t* x, const float* logits,          \
                                const float* spart, int T, int32_t* topk_idx, float* topk_w, uint16_t* hh, \
                                bool norm, hipStream_t s);                                                 \
  int decode_down_combine_b##B(const moe_layer_desc* L, const uint16_t* hh, int T, const int32_t* topk_idx, \
                               const float* topk_w, const uint16_t* residual, uint16_t* out, hipStream_t s)

MOEQ_DECODE_FUSED_LAUNCHERS(4);
MOEQ_DECODE_FUSED_LAUNCHERS(6);
MOEQ_DECODE_FUSED_LAUNCHERS(8);

#ifndef MOEQ_SHARED_LATE_BLOCKS
#define MOEQ_SHARED_LATE_BLOCKS 256
#endif

// norm: moe_decode_block's launch 1 normalises the rows itself, so the
// shared experts run as whole rows in launch 2 (reading the stored rows)
template <int B, int NCH>
decode_detail::FusedGrid fused_grid(const moe_layer_desc* L, int T, bool norm = false) {
  decode_detail::FusedGrid fg;
  fg.E = L->E;
  fg.S = L->S;
  fg.k = L->k;
  fg.T = T;
  fg.kS = L->k + L->S;
  fg.tiles = L->I / 64;
  fg.groups = (T + 1) / 2;
  fg.Q = decode_detail::SharedShape<B, NCH>::Q;
  fg.router_blocks = ((L->E + 3) / 4 + 7) / 8 * 8;
  // shared experts: beside the router as K slices, unless the routed launch
  // leaves CUs idle anyway (small batches), where whole rows there are cheaper
  fg.shared_late = L->S > 0 && (norm || T <= decode_detail::kRows8MaxT || T * L->k * fg.tiles < MOEQ_SHARED_LATE_BLOCKS);
  fg.shared_blocks = L->S > 0 && !fg.shared_late ? (L->S * fg.tiles * fg.Q + 7) / 8 * 8 * fg.groups : 0;
  fg.late_blocks = fg.shared_late ? (L->S * fg.tiles + 7) / 8 * 8 * fg.groups : 0;
  return fg;
}

// Runs fn(std::integral_constant<int, NCH>) for H = 512 NCH, NCH in {1, 2, 4, 8}.
template <class Fn>
int with_nch(int H, Fn&& fn) {
  switch (H) {
    case 512: return fn(std::integral_constant<int, 1>());
    case 1024: return fn(std::integral_constant<int, 2>());
    case 2048: return fn(std::integral_constant<int, 4>());
    case 4096: return fn(std::integral_constant<int, 8>());
    default: return set_error(MOEQ_ERR_UNSUPPORTED, "moe_decode_forward: H=%d not in {512, 1024, 2048, 4096}", H);
  }
}

template <int B>
int launch_router_shared(const moe_layer_desc* L, const uint16_t* x, const uint16_t* wr, const float* bias, int T,
                         float* logits, float* spart, decode_detail::NormArgs norm, hipStream_t s) {
  return with_nch(L->H, [&](auto nch) {
    constexpr int NCH = decltype(nch)::value;
    const decode_detail::FusedGrid fg = fused_grid<B, NCH>(L, T, norm.xraw != nullptr);
    decode_detail::router_shared_kernel<B, NCH><<<fg.router_blocks + fg.shared_blocks, 256, 0, s>>>(
        wr, bias, L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->I, fg, logits, spart, norm);
    return check_launch("moe_decode_forward (router + shared gate/up)");
  });
}

template <int B>
int launch_gateup_routed(const moe_layer_desc* L, const uint16_t* x, const float* logits, const float* spart, int T,
                         int32_t* topk_idx, float* topk_w, uint16_t* hh, bool norm, hipStream_t s) {
  return with_nch(L->H, [&](auto nch) {
    constexpr int NCH = decltype(nch)::value;
    const decode_detail::FusedGrid fg = fused_grid<B, NCH>(L, T, norm);
    if (T <= decode_detail::kRows8MaxT) {
      decode_detail::gateup_rows8_kernel<B, NCH><<<T * fg.kS * (L->I / 8), 256, 0, s>>>(
          L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->I, fg, logits, topk_idx, topk_w, hh);
      return check_launch("moe_decode_forward (selection + gate/up rows)");
    }
    decode_detail::gateup_routed_kernel<B, NCH><<<T * L->k * fg.tiles + fg.late_blocks, 64 * decode_detail::FusedShape<B, NCH>::W,
                                                 0, s>>>(L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->I, fg,
                                                         logits, spart, topk_idx, topk_w, hh);
    return check_launch("moe_decode_forward (selection + routed gate/up)");
  });
}

// One down + combine launch: I / 64 groups in {4, 8, 12}, and 16 at 4 bits
// (the 6- and 8-bit rows of I = 1024 would not fit the registers of a
// 1024-thread block without spilling).
template <int B>
int launch_down_combine(const moe_layer_desc* L, const uint16_t* hh, int T, const int32_t* topk_idx,
                        const float* topk_w, const uint16_t* residual, uint16_t* out, hipStream_t s) {
  const decode_detail::FusedGrid fg = fused_grid<B, 1>(L, T);
  const int grid = T * (L->H / 64), threads = 64 * fg.kS;
  const bool rows8 = T <= decode_detail::kRows8MaxT;
  auto go = [&](auto ng) {
    if (rows8)
      decode_detail::down_rows8_kernel<B, decltype(ng)::value><<<T * (L->H / 8), 256, 0, s>>>(
          L->down.q, L->down.sz, hh, L->H, fg, topk_idx, topk_w, residual, out);
    else
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
  int decode_router_shared_b##B(const moe_layer_desc* L, const uint16_t* x, const uint16_t* wr,           \
                                const float* bias, int T, float* logits, float* spart,                     \
                                decode_detail::NormArgs norm, hipStream_t s) {                             \
    return launch_router_shared<B>(L, x, wr, bias, T, logits, spart, norm, s);                             \
  }                                                                                                        \
  int decode_gateup_routed_b##B(const moe_layer_desc* L, const uint16_t* x, const float* logits,          \
                                const float* spart, int T, int32_t* topk_idx, float* topk_w, uint16_t* hh, \
                                bool norm, hipStream_t s) {                                                \
    return launch_gateup_routed<B>(L, x, logits, spart, T, topk_idx, topk_w, hh, norm, s);                 \
  }                                                                                                        \
  int decode_down_combine_b##B(const moe_layer_desc* L, const uint16_t* hh, int T, const int32_t* topk_idx, \
                               const float* topk_w, const uint16_t* residual, uint16_t* out, hipStream_t s) { \
    return launch_down_combine<B>(L, hh, T, topk_idx, topk_w, residual, out, s);                           \
  }

}  // namespace moeq
