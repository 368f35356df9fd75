// Decode path kernels: grouped GEMV over the routed experts only.
//
// Weight streaming is the whole cost at decode (Raon-1-mini on an RTX
// 5070 Ti: the finished runtime streams weights at about two thirds of the
// card's bandwidth), so the kernels read each routed expert's packed rows
// exactly once, with full-width coalesced loads, and spend as few vector
// instructions per byte as possible:
//
//   * one lane owns one output row: a wavefront covers a tile of 64 rows and
//     walks its share of the K chunks; the tiled weight layout (format.h)
//     makes each chunk load of the wavefront one contiguous block, and no
//     cross-lane reduction is needed per row;
//   * the activations of a chunk are the same for all 64 rows, so they are
//     read with scalar loads into SGPRs (the dot products take them as their
//     scalar operand): no vector registers or vector memory traffic for x;
//   * codes become bf16 (128 + q, or q for 8-bit) with one AND-OR per two
//     codes and are multiplied by v_dot2_f32_bf16 with fp32 accumulation: the
//     products are exact, and the group's scale and zero enter once per
//     group in fp32:
//         sum_i (q_i - z) s x_i = s * (sum_i (128+q_i) x_i - (z+128) sum_i x_i);
//     the group sums of x come from one cooperative load per wavefront;
//   * gate and up rows that share the input are read in the same pass and
//     combined into h = silu(g) u (Raon-1-mini optimisation table:
//     projections sharing an input run together);
//   * the W wavefronts of a block split K; each keeps the loads of DEPTH
//     chunks in flight while it computes one (a software pipeline), and their
//     partial sums meet in LDS, added in a fixed order.
// h goes to the down projection in bf16, as on the prefill path.
//
// Grid: see DecodeGrid.  Blocks whose expert is not active exit at once, so
// the host never needs the routing result.
#pragma once
#include "format.h"

namespace moeq {
namespace decode_detail {

#ifndef MOEQ_DEPTH
#define MOEQ_DEPTH 4
#endif
constexpr int kDepth = MOEQ_DEPTH;   // chunks whose loads are in flight per wavefront
constexpr int kMaxNT = 2;   // tokens per pass

// Block -> work mapping shared by both kernels.  The grid has two parts:
//  * shared experts (every token uses them, so the host knows their load):
//    one block per (shared expert, row tile, pair of tokens), laid out so
//    that the blocks of one row tile land on the same XCD (blocks are dealt
//    to the 8 XCDs round-robin) a few dispatches apart, so the weights they
//    all read come from that XCD's L2 after the first;
//  * routed experts: one block per (active routed expert, row tile), the
//    expert's tokens taken in passes of up to two.
struct DecodeGrid {
  int E, S;            // routed and shared expert counts
  int kS;              // assignments per token (k + S)
  int tiles;           // 64-row tiles per expert
  int shared_blocks;   // blocks in the shared part (a multiple of 8 * groups)
  int groups;          // token pairs of a shared expert: ceil(T / 2)
};

// Decodes blockIdx.x.  Returns false for a block without work; otherwise
// sets the expert, the row tile and, for a shared-expert block, its token
// pair (-1 for a routed block: all of the expert's tokens).
MOEQ_DEV bool block_work(int b, const DecodeGrid& dg, const int32_t* __restrict__ active, int& e, int& tile,
                         int& pair) {
  if (b < dg.shared_blocks) {
    const int span = 8 * dg.groups;
    const int l = (b / span) * 8 + (b % 8);   // (shared expert, row tile)
    if (l >= dg.S * dg.tiles) return false;
    pair = (b % span) / 8;
    e = dg.E + l / dg.tiles;
    tile = l % dg.tiles;
    return true;
  }
  const int r = b - dg.shared_blocks;
  const int j = r / dg.tiles;
  tile = r % dg.tiles;
  pair = -1;
  if (j >= active[0] - dg.S) return false;   // active: routed ids first, then the S shared ones
  e = active[1 + j];
  return e < dg.E;
}

template <int BITS>
MOEQ_DEV void load_chunk_g(gbytes p, uint32_t (&d)[Fmt<BITS>::DW]) {
  typedef const __attribute__((address_space(1))) moeq_u32x4* g4;
  if constexpr (Fmt<BITS>::DW == 4) {
    const moeq_u32x4 v = *reinterpret_cast<g4>(p);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  } else {
    typedef const __attribute__((address_space(1))) moeq_u32x3* g3;
    const moeq_u32x3 v = *reinterpret_cast<g3>(p);
    d[0] = v.x; d[1] = v.y; d[2] = v.z;
  }
}

// Loads in flight for one chunk of NM matrices: the chunk's codes and, on
// the first chunk of a group, the group's scale/zero words.
template <int BITS, int NM>
struct ChunkBuf {
  uint32_t q[NM][Fmt<BITS>::DW];
  uint32_t sz[NM];
};

// One wavefront's work: rows tile*64 + lane of one expert's matrices,
// chunks [c0, c0 + CW) of K.  Each load address is a scalar base (this
// wavefront's first chunk) plus a 32-bit lane offset (the global_load
// "saddr" form), so no per-chunk address occupies registers.
template <int BITS, int NM>
struct Stream {
  using F = Fmt<BITS>;
  gbytes q[NM];    // codes of chunk c0 of the tile (uniform)
  gbytes sz[NM];   // scale/zero word of group c0 / CPG of the tile (uniform)
  int c0;
  // qe, sze: the expert's codes and scale/zero words; cpr, gpr: chunks and
  // groups per row
  MOEQ_DEV void init(const uint8_t* const (&qe)[NM], const uint32_t* const (&sze)[NM], int cpr, int gpr, int tile,
                     int first) {
    c0 = first;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      q[m] = uniform_ptr(qe[m] + ((size_t)tile * cpr + (size_t)c0) * (64 * F::BYTES));
      sz[m] = uniform_ptr(reinterpret_cast<const uint8_t*>(
          sze[m] + ((size_t)tile * gpr + (size_t)(c0 / F::CHUNKS_PER_GROUP)) * 64));
    }
  }
  MOEQ_DEV void load(int c, ChunkBuf<BITS, NM>& b) const {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t off = lane * (uint32_t)F::BYTES + (uint32_t)c * (64u * F::BYTES);
#pragma unroll
    for (int m = 0; m < NM; ++m) load_chunk_g<BITS>(q[m] + off, b.q[m]);
    if (c % F::CHUNKS_PER_GROUP == 0) {   // c0 is a multiple of the group's chunks
      const uint32_t so = lane * 4u + (uint32_t)(c / F::CHUNKS_PER_GROUP) * 256u;
#pragma unroll
      for (int m = 0; m < NM; ++m) b.sz[m] = load_word_g(sz[m] + so);
    }
  }
};

// keeps the compiler from moving instructions across a pipeline stage
MOEQ_DEV void stage_fence() { __builtin_amdgcn_sched_barrier(0); }

// Sums of x over the wavefront's NG groups [g0, g0 + NG) for up to two token
// rows, computed cooperatively: for NG <= 8 lane 8 g + j adds x values
// 8 j .. 8 j + 7 of group g, for NG <= 16 lane 4 g + j adds values
// 16 j .. 16 j + 15; the sum of group g ends in lane xs_lane<NG>(g).
template <int NG>
constexpr int xs_lane(int g) { return NG <= 8 ? 8 * g + 7 : 4 * g + 3; }

// The two halves of one row's group sums, so that the loads can be issued
// early: GroupX<NG>::load, then GroupX<NG>::sum.
template <int NG>
struct GroupX {
  static_assert(NG >= 1 && NG <= 16, "at most 16 groups per wavefront");
  static constexpr int PER = NG <= 8 ? 8 : 16;   // values per lane
  moeq_u32x4 v[PER / 8];
  MOEQ_DEV void load(const uint16_t* xr, int g0) {
    const int lane = threadIdx.x & 63;
    const int off = g0 * 64 + PER * (lane < 64 / PER * NG ? lane : 0);
#pragma unroll
    for (int h = 0; h < PER / 8; ++h) v[h] = *reinterpret_cast<const moeq_u32x4*>(xr + off + 8 * h);
  }
  MOEQ_DEV float sum() const {
    const uint32_t ones = 0x3F803F80u;   // bf16 (1, 1): dot2 with it sums a pair
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < PER / 8; ++h) {
      s = dot2_bf16(v[h].x, ones, s);
      s = dot2_bf16(v[h].y, ones, s);
      s = dot2_bf16(v[h].z, ones, s);
      s = dot2_bf16(v[h].w, ones, s);
    }
    return group_sum_last<64 / PER>(s);
  }
};

template <int NG>
MOEQ_DEV void group_sums(const uint16_t* const (&xr)[kMaxNT], int nt, int g0, float (&xs)[kMaxNT]) {
#pragma unroll
  for (int t = 0; t < kMaxNT; ++t) {
    GroupX<NG> gx;
    if (t < nt) gx.load(xr[t], g0);
    xs[t] = t < nt ? gx.sum() : 0.0f;
  }
}

MOEQ_DEV float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Largest divisor of cw that is at most lim (at least 1).
constexpr int x_group(int cw, int lim) {
  int g = 1;
  for (int d = 1; d <= cw && d <= lim; ++d)
    if (cw % d == 0) g = d;
  return g;
}

// The wavefront's part of the dot products of its 64 rows with NT token rows
// xr[t] (bf16, read as scalars), for NM matrices: out[m][t].  The loads of
// chunks [0, D) are already in buf.
template <int BITS, int NM, int NT, int CW, int D>
MOEQ_DEV void stream_rows(const Stream<BITS, NM>& st, ChunkBuf<BITS, NM> (&buf)[D],
                          const uint16_t* const (&xr)[kMaxNT], const float (&xs)[kMaxNT], float (&out)[NM][kMaxNT]) {
  using F = Fmt<BITS>;
  constexpr int CPG = F::CHUNKS_PER_GROUP;
  static_assert(CW % CPG == 0, "a wavefront covers whole groups");
  float acc[NM][NT][2];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
#pragma unroll
    for (int t = 0; t < kMaxNT; ++t) out[m][t] = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) { acc[m][t][0] = 0.0f; acc[m][t][1] = 0.0f; }
  }
  float s[NM], zc[NM];
  // Activations: the same for every lane, read with scalar loads into
  // SGPRs, XG chunks at a time (64 SGPRs), so one load latency covers XG
  // chunks.
  constexpr int XG = x_group(CW, 64 / F::PAIRS / NT);   // chunks per x load group
  uint32_t X[XG][NT][F::PAIRS];
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    ChunkBuf<BITS, NM>& b = buf[c % D];
    if (c % XG == 0) {
#pragma unroll
      for (int g = 0; g < XG; ++g)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint32_t* xp = reinterpret_cast<const uint32_t*>(xr[t] + (size_t)(st.c0 + c + g) * F::CODES);
#pragma unroll
          for (int p = 0; p < F::PAIRS; ++p) X[g][t][p] = xp[p];
        }
    }
    if (c % CPG == 0) {
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        s[m] = f16_bits_to_f32(b.sz[m] & 0xFFFFu);
        zc[m] = f16_bits_to_f32(b.sz[m] >> 16) + F::OFFSET;
      }
    }
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      // the chunk's codes are taken here, where they are needed: nothing
      // derived from them is computed (and kept live) earlier
#pragma unroll
      for (int j = 0; j < F::DW; ++j) asm volatile("" : "+v"(b.q[m][j]));
      uint32_t P[F::PAIRS];
      chunk_pairs<BITS>(b.q[m], P);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int p = 0; p < F::PAIRS; ++p) acc[m][t][p & 1] = dot2_bf16(P[p], X[c % XG][t][p], acc[m][t][p & 1]);
      stage_fence();   // one matrix's unpacked pairs live at a time
    }
    if (c + D < CW) st.load(c + D, b);
    if (c % CPG == CPG - 1) {   // group complete: apply its scale and zero
      const int gl = c / CPG;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float x_sum = lane_value(xs[t], xs_lane<CW / CPG>(gl));
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          out[m][t] = fmaf(s[m], (acc[m][t][0] + acc[m][t][1]) - zc[m] * x_sum, out[m][t]);
          acc[m][t][0] = 0.0f;
          acc[m][t][1] = 0.0f;
        }
      }
    }
    stage_fence();
  }
}

// Partial sums of the block's W wavefronts: v[w][m][t][row].
template <int W, int NM>
struct Partials {
  float v[W][NM][kMaxNT][64];
};

// One pass over the block's rows for the tokens of rows xr (nt of them):
// every wavefront streams its chunks, then the partials are added in
// wavefront order; wavefront t < nt ends with the sums of token t for its
// lane's row in tot[m].
template <int BITS, int NM, int W, int CW>
MOEQ_DEV void block_pass(const Stream<BITS, NM>& st, ChunkBuf<BITS, NM> (&buf)[CW < kDepth ? CW : kDepth],
                         const uint16_t* const (&xr)[kMaxNT], int nt, Partials<W, NM>& part, float (&tot)[NM]) {
  constexpr int CPG = Fmt<BITS>::CHUNKS_PER_GROUP;
  constexpr int D = CW < kDepth ? CW : kDepth;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index is uniform
  float xs[kMaxNT];
  group_sums<CW / CPG>(xr, nt, st.c0 / CPG, xs);
  stage_fence();
  float out[NM][kMaxNT];
  if (nt == 2) stream_rows<BITS, NM, 2, CW, D>(st, buf, xr, xs, out);
  else stream_rows<BITS, NM, 1, CW, D>(st, buf, xr, xs, out);
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int t = 0; t < kMaxNT; ++t) part.v[wave][m][t][lane] = out[m][t];
  __syncthreads();
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    float v = 0.0f;
    if (wave < nt)
#pragma unroll
      for (int w = 0; w < W; ++w) v += part.v[w][m][wave][lane];
    tot[m] = v;
  }
}

// -------------------------------------------------------------------------
// gate/up: h[p][i] = bf16(silu(Wg x_t)[i] * (Wu x_t)[i]) for the expert's
// sorted positions p (token t = sorted[p] / (k+S)); h is [A][I] bf16.
// -------------------------------------------------------------------------
template <int BITS, int W, int CW>
MOEQ_DEV void gateup_rows_unit(int b, Partials<W, 2>& part, const uint8_t* __restrict__ gq,
                               const uint32_t* __restrict__ gsz, const uint8_t* __restrict__ uq,
                               const uint32_t* __restrict__ usz, const uint16_t* __restrict__ x, int H, int I,
                               const DecodeGrid& dg, const int32_t* __restrict__ offsets,
                               const int32_t* __restrict__ sorted, const int32_t* __restrict__ active,
                               uint16_t* __restrict__ hh) {
  using F = Fmt<BITS>;
  constexpr int D = CW < kDepth ? CW : kDepth;
  int e, tile, pair;
  if (!block_work(b, dg, active, e, tile, pair)) return;
  e = uniform(e);
  tile = uniform(tile);
  pair = uniform(pair);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index is uniform
  Stream<BITS, 2> st;
  {
    const size_t ebytes = (size_t)I * row_bytes(H, BITS), ewords = (size_t)I * (H / 64);
    const uint8_t* const qe[2] = {gq + e * ebytes, uq + e * ebytes};
    const uint32_t* const sze[2] = {gsz + e * ewords, usz + e * ewords};
    st.init(qe, sze, H / F::CODES, H / 64, tile, wave * CW);
  }
  ChunkBuf<BITS, 2> buf[D];
#pragma unroll
  for (int c = 0; c < D; ++c) st.load(c, buf[c]);   // before the token lookups
  stage_fence();
  int pb = uniform(offsets[e]), pe = uniform(offsets[e + 1]);
  if (pair >= 0) {
    pb += 2 * pair;
    pe = min(pe, pb + 2);
  }
  const int row = tile * 64 + lane;
  // The first pass uses the loads issued above; later passes (experts with
  // more than two tokens) reload into buffers of their own, so no buffer is
  // carried around the loop (that would force a wait for every load in
  // flight before the loop).
  auto pass = [&](int p0, ChunkBuf<BITS, 2> (&b)[D]) {
    const int nt = min(kMaxNT, pe - p0);
    const int t0 = uniform(sorted[p0] / dg.kS);
    const int t1 = nt > 1 ? uniform(sorted[p0 + 1] / dg.kS) : t0;
    const uint16_t* const xr[kMaxNT] = {x + (size_t)t0 * H, x + (size_t)t1 * H};
    float tot[2];
    block_pass<BITS, 2, W, CW>(st, b, xr, nt, part, tot);
    if (wave < nt) hh[(size_t)(p0 + wave) * I + row] = (uint16_t)f32_to_bf16_bits(silu_f32(tot[0]) * tot[1]);
  };
  if (pb >= pe) return;
  pass(pb, buf);
  for (int p0 = pb + kMaxNT; p0 < pe; p0 += kMaxNT) {
    __syncthreads();   // the previous pass's partials have been read
    ChunkBuf<BITS, 2> lb[D];
#pragma unroll
    for (int c = 0; c < D; ++c) st.load(c, lb[c]);
    stage_fence();
    pass(p0, lb);
  }
}

// One block per unit (decode batches).
template <int BITS, int W, int CW>
__global__ __launch_bounds__(64 * W, 4) void gateup_rows_kernel(const uint8_t* __restrict__ gq,
                                                                const uint32_t* __restrict__ gsz,
                                                                const uint8_t* __restrict__ uq,
                                                                const uint32_t* __restrict__ usz,
                                                                const uint16_t* __restrict__ x, int H, int I,
                                                                DecodeGrid dg, const int32_t* __restrict__ offsets,
                                                                const int32_t* __restrict__ sorted,
                                                                const int32_t* __restrict__ active,
                                                                uint16_t* __restrict__ hh) {
  __shared__ Partials<W, 2> part;
  gateup_rows_unit<BITS, W, CW>((int)blockIdx.x, part, gq, gsz, uq, usz, x, H, I, dg, offsets, sorted, active, hh);
}

// A grid smaller than the list: each block takes units blockIdx.x,
// blockIdx.x + gridDim.x, ... up to the list's active[0] * tiles (routed
// experts only), so an empty or short list costs one read per block.
template <int BITS, int W, int CW>
__global__ __launch_bounds__(64 * W, 4) void gateup_list_kernel(const uint8_t* __restrict__ gq,
                                                                const uint32_t* __restrict__ gsz,
                                                                const uint8_t* __restrict__ uq,
                                                                const uint32_t* __restrict__ usz,
                                                                const uint16_t* __restrict__ x, int H, int I,
                                                                DecodeGrid dg, const int32_t* __restrict__ offsets,
                                                                const int32_t* __restrict__ sorted,
                                                                const int32_t* __restrict__ active,
                                                                uint16_t* __restrict__ hh) {
  __shared__ Partials<W, 2> part;
  const int units = uniform(active[0]) * dg.tiles;
  for (int b = (int)blockIdx.x; b < units; b += (int)gridDim.x) {
    __syncthreads();   // the previous unit's partials have been read
    gateup_rows_unit<BITS, W, CW>(b, part, gq, gsz, uq, usz, x, H, I, dg, offsets, sorted, active, hh);
  }
}

MOEQ_DEV float y_value(float v, float*) { return v; }
MOEQ_DEV uint16_t y_value(float v, uint16_t*) { return (uint16_t)f32_to_bf16_bits(v); }

// -------------------------------------------------------------------------
// down: y[a][n] = (Wd h_p)[n] for the expert's sorted positions p and their
// assignments a = sorted[p]; y is [A][H], fp32 (YT = float) or bf16 (YT =
// uint16_t, rounded to nearest even).
// -------------------------------------------------------------------------
template <int BITS, int W, int CW, typename YT>
MOEQ_DEV void down_rows_unit(int b, Partials<W, 1>& part, const uint8_t* __restrict__ dq,
                             const uint32_t* __restrict__ dsz, const uint16_t* __restrict__ hh, int H, int I,
                             const DecodeGrid& dg, const int32_t* __restrict__ offsets,
                             const int32_t* __restrict__ sorted, const int32_t* __restrict__ active,
                             YT* __restrict__ y) {
  using F = Fmt<BITS>;
  constexpr int D = CW < kDepth ? CW : kDepth;
  int e, tile, pair;
  if (!block_work(b, dg, active, e, tile, pair)) return;
  e = uniform(e);
  tile = uniform(tile);
  pair = uniform(pair);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave index is uniform
  Stream<BITS, 1> st;
  {
    const uint8_t* const qe[1] = {dq + e * ((size_t)H * row_bytes(I, BITS))};
    const uint32_t* const sze[1] = {dsz + e * ((size_t)H * (I / 64))};
    st.init(qe, sze, I / F::CODES, I / 64, tile, wave * CW);
  }
  ChunkBuf<BITS, 1> buf[D];
#pragma unroll
  for (int c = 0; c < D; ++c) st.load(c, buf[c]);   // before the token lookups
  stage_fence();
  int pb = uniform(offsets[e]), pe = uniform(offsets[e + 1]);
  if (pair >= 0) {
    pb += 2 * pair;
    pe = min(pe, pb + 2);
  }
  const int row = tile * 64 + lane;
  auto pass = [&](int p0, ChunkBuf<BITS, 1> (&b)[D]) {   // as in the gate/up kernel
    const int nt = min(kMaxNT, pe - p0);
    const uint16_t* const xr[kMaxNT] = {hh + (size_t)p0 * I, hh + (size_t)(p0 + (nt > 1 ? 1 : 0)) * I};
    float tot[1];
    block_pass<BITS, 1, W, CW>(st, b, xr, nt, part, tot);
    if (wave < nt) y[(size_t)sorted[p0 + wave] * H + row] = y_value(tot[0], y);
  };
  if (pb >= pe) return;
  pass(pb, buf);
  for (int p0 = pb + kMaxNT; p0 < pe; p0 += kMaxNT) {
    __syncthreads();
    ChunkBuf<BITS, 1> lb[D];
#pragma unroll
    for (int c = 0; c < D; ++c) st.load(c, lb[c]);
    stage_fence();
    pass(p0, lb);
  }
}

template <int BITS, int W, int CW, typename YT>
__global__ __launch_bounds__(64 * W, 4) void down_rows_kernel(const uint8_t* __restrict__ dq,
                                                              const uint32_t* __restrict__ dsz,
                                                              const uint16_t* __restrict__ hh, int H, int I,
                                                              DecodeGrid dg, const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ sorted,
                                                              const int32_t* __restrict__ active,
                                                              YT* __restrict__ y) {
  __shared__ Partials<W, 1> part;
  down_rows_unit<BITS, W, CW, YT>((int)blockIdx.x, part, dq, dsz, hh, H, I, dg, offsets, sorted, active, y);
}

template <int BITS, int W, int CW, typename YT>
__global__ __launch_bounds__(64 * W, 4) void down_list_kernel(const uint8_t* __restrict__ dq,
                                                              const uint32_t* __restrict__ dsz,
                                                              const uint16_t* __restrict__ hh, int H, int I,
                                                              DecodeGrid dg, const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ sorted,
                                                              const int32_t* __restrict__ active,
                                                              YT* __restrict__ y) {
  __shared__ Partials<W, 1> part;
  const int units = uniform(active[0]) * dg.tiles;
  for (int b = (int)blockIdx.x; b < units; b += (int)gridDim.x) {
    __syncthreads();
    down_rows_unit<BITS, W, CW, YT>(b, part, dq, dsz, hh, H, I, dg, offsets, sorted, active, y);
  }
}

// (W, CW) shapes with a kernel: W wavefronts per block, CW chunks each.
#define MOEQ_DECODE_SHAPES(X)                                                                            \
  X(2, 2) X(2, 4) X(2, 8) X(2, 16) X(4, 2) X(4, 4) X(4, 6) X(4, 8) X(4, 12) X(4, 16) X(8, 2) X(8, 4)      \
  X(8, 8) X(8, 16) X(16, 4) X(16, 8) X(16, 16)
constexpr int kShapes[][2] = {{2, 2}, {2, 4}, {2, 8}, {2, 16}, {4, 2}, {4, 4}, {4, 6}, {4, 8}, {4, 12},
                              {4, 16}, {8, 2}, {8, 4}, {8, 8}, {8, 16}, {16, 4}, {16, 8}, {16, 16}};

}  // namespace decode_detail

// Block shape for K inputs at `bits`: W wavefronts split the CPR = K / codes
// chunks of a row, CW = CPR / W each, a whole number of groups (at most 8).
// The wavefront's run of CW chunks is a software pipeline whose register
// footprint grows with CW, so the shape with the run closest to `want`
// chunks (and not shorter than one group) is taken.
inline bool pick_shape(int K, int bits, int want, int& W, int& CW) {
  const int codes = bits == 4 ? 32 : 16, cpg = 64 / codes;
  if (K % codes) return false;
  const int cpr = K / codes;
  bool found = false;
  int best = 0;
  for (const auto& s : decode_detail::kShapes) {
    const int w = s[0], cw = s[1];
    if (w * cw != cpr || cw % cpg || cw / cpg > 8) continue;
    const int score = cw >= want ? cw - want : 2 * (want - cw);   // shorter runs cost more
    if (!found || score < best) {
      W = w;
      CW = cw;
      best = score;
      found = true;
    }
  }
  return found;
}

#ifndef MOEQ_GATEUP_RUN
#define MOEQ_GATEUP_RUN 8
#endif
#ifndef MOEQ_DOWN_RUN
#define MOEQ_DOWN_RUN 8
#endif
// run lengths and grid size of the prefill's GEMV list (cold experts)
#ifndef MOEQ_LIST_GATEUP_RUN
#define MOEQ_LIST_GATEUP_RUN MOEQ_GATEUP_RUN
#endif
#ifndef MOEQ_LIST_DOWN_RUN
#define MOEQ_LIST_DOWN_RUN MOEQ_DOWN_RUN
#endif
#ifndef MOEQ_LIST_GRID
#define MOEQ_LIST_GRID 1024
#endif

// Grid of the decode kernels for N output rows per expert (see
// decode_detail::DecodeGrid); returns the block count.
inline int decode_grid(const moe_layer_desc* L, int T, int N, decode_detail::DecodeGrid& dg) {
  dg.E = L->E;
  dg.S = L->S;
  dg.kS = L->k + L->S;
  dg.tiles = N / 64;
  dg.groups = (T + 1) / 2;
  dg.shared_blocks = L->S > 0 ? (L->S * dg.tiles + 7) / 8 * 8 * dg.groups : 0;
  const long routed = (long)T * L->k < L->E ? (long)T * L->k : L->E;   // upper bound on active routed experts
  return dg.shared_blocks + (int)routed * dg.tiles;
}

// Grid of the list kernels over routed experts only (no shared blocks):
// up to max_experts of them, N output rows each, at most 1024 blocks.
inline int decode_list_grid(const moe_layer_desc* L, int max_experts, int N, decode_detail::DecodeGrid& dg) {
  dg.E = L->E;
  dg.S = 0;
  dg.kS = L->k + L->S;
  dg.tiles = N / 64;
  dg.groups = 1;
  dg.shared_blocks = 0;
  const int units = max_experts * dg.tiles;
  return units < MOEQ_LIST_GRID ? units : MOEQ_LIST_GRID;
}

// Per-bit-width launchers (one translation unit each, decode_b{4,6,8}.hip).
#define MOEQ_DECODE_LAUNCHERS(B)                                                                          \
  int decode_gateup_b##B(const moe_layer_desc* L, const uint16_t* x, const int32_t* offsets,              \
                         const int32_t* sorted, const int32_t* active, int T, int W, int CW, uint16_t* hh,  \
                         hipStream_t s);                                                                  \
  int decode_down_b##B(const moe_layer_desc* L, const uint16_t* hh, const int32_t* offsets,               \
                       const int32_t* sorted, const int32_t* active, int T, int W, int CW, float* y,      \
                       hipStream_t s);                                                                    \
  int list_gateup_b##B(const moe_layer_desc* L, const uint16_t* x, const int32_t* offsets,                \
                       const int32_t* sorted, const int32_t* list, int W, int CW, uint16_t* hh,           \
                       hipStream_t s);                                                                    \
  int list_down_b##B(const moe_layer_desc* L, const uint16_t* hh, const int32_t* offsets,                 \
                     const int32_t* sorted, const int32_t* list, int W, int CW, uint16_t* y, hipStream_t s)

MOEQ_DECODE_LAUNCHERS(4);
MOEQ_DECODE_LAUNCHERS(6);
MOEQ_DECODE_LAUNCHERS(8);

#define MOEQ_DEFINE_DECODE(B)                                                                             \
  int decode_gateup_b##B(const moe_layer_desc* L, const uint16_t* x, const int32_t* offsets,              \
                         const int32_t* sorted, const int32_t* active, int T, int W, int CW, uint16_t* hh,  \
                         hipStream_t s) {                                                                 \
    decode_detail::DecodeGrid dg;                                                                         \
    const int grid = decode_grid(L, T, L->I, dg);                                                         \
    if (grid == 0) return MOEQ_OK;                                                                        \
    bool launched = false;                                                                                \
    MOEQ_DECODE_SHAPES(MOEQ_LAUNCH_GU)                                                                    \
    if (!launched) return set_error(MOEQ_ERR_UNSUPPORTED, "decode: no gate/up kernel for W=%d CW=%d", W, CW); \
    return check_launch("moe_qgemv_decode (gate/up)");                                                    \
  }                                                                                                       \
  int decode_down_b##B(const moe_layer_desc* L, const uint16_t* hh, const int32_t* offsets,               \
                       const int32_t* sorted, const int32_t* active, int T, int W, int CW, float* y,      \
                       hipStream_t s) {                                                                   \
    decode_detail::DecodeGrid dg;                                                                         \
    const int grid = decode_grid(L, T, L->H, dg);                                                         \
    if (grid == 0) return MOEQ_OK;                                                                        \
    bool launched = false;                                                                                \
    MOEQ_DECODE_SHAPES(MOEQ_LAUNCH_DN)                                                                    \
    if (!launched) return set_error(MOEQ_ERR_UNSUPPORTED, "decode: no down kernel for W=%d CW=%d", W, CW); \
    return check_launch("moe_qgemv_decode (down)");                                                       \
  }                                                                                                       \
  int list_gateup_b##B(const moe_layer_desc* L, const uint16_t* x, const int32_t* offsets,                \
                       const int32_t* sorted, const int32_t* active, int W, int CW, uint16_t* hh,         \
                       hipStream_t s) {                                                                   \
    decode_detail::DecodeGrid dg;                                                                         \
    const int grid = decode_list_grid(L, L->E, L->I, dg);                                                 \
    bool launched = false;                                                                                \
    MOEQ_DECODE_SHAPES(MOEQ_LAUNCH_GU_LIST)                                                               \
    if (!launched) return set_error(MOEQ_ERR_UNSUPPORTED, "expert list: no gate/up kernel for W=%d CW=%d", W, CW); \
    return check_launch("moe_qgemm_prefill (gate/up of the GEMV list)");                                  \
  }                                                                                                       \
  int list_down_b##B(const moe_layer_desc* L, const uint16_t* hh, const int32_t* offsets,                 \
                     const int32_t* sorted, const int32_t* active, int W, int CW, uint16_t* y,            \
                     hipStream_t s) {                                                                     \
    decode_detail::DecodeGrid dg;                                                                         \
    const int grid = decode_list_grid(L, L->E, L->H, dg);                                                 \
    bool launched = false;                                                                                \
    MOEQ_DECODE_SHAPES(MOEQ_LAUNCH_DN_LIST)                                                               \
    if (!launched) return set_error(MOEQ_ERR_UNSUPPORTED, "expert list: no down kernel for W=%d CW=%d", W, CW); \
    return check_launch("moe_qgemm_prefill (down of the GEMV list)");                                     \
  }

}  // namespace moeq
