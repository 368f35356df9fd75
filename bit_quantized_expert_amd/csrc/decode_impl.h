// Decode path kernels: grouped GEMV over the routed experts only.
//
// Weight streaming is the whole cost at decode (Raon-1-mini on an RTX
// 5070 Ti: the finished runtime streams weights at about two thirds of the
// card's bandwidth), so the kernels are built around reading each routed
// expert's packed rows exactly once, with full-width vector loads:
//
//   * a lane owns fixed "chunks" of a row (16 B for 4/8-bit, 12 B for 6-bit);
//     LPR lanes cover ITER chunks of a row each, so the lane's slice of the
//     activation vector is fixed for a pass and lives in registers as bf16
//     pairs;
//   * codes become bf16 (128 + q, or q for 8-bit) with one AND-OR per two
//     codes and are multiplied by v_dot2_f32_bf16 with fp32 accumulation: the
//     products are exact, and the group's scale and zero enter once per chunk
//     in fp32:
//         sum_i (q_i - z) s x_i = s * (sum_i (128+q_i) x_i - (z+128) sum_i x_i);
//   * gate and up rows that share the input are read in the same pass and
//     combined into h = silu(g) u (Raon-1-mini optimisation table:
//     projections sharing an input run together);
//   * a wave loads all of its weight chunks (CH per lane, CH/ITER row steps)
//     into registers before anything else, so every weight load of the wave
//     is in flight at once; token passes (up to two tokens each) then reuse
//     those registers, so an expert's weights are read from HBM once however
//     many of the batch's tokens it serves;
//   * rows are reduced across their LPR lanes with DPP.
// The intermediate h = silu(g) u goes to the down projection in bf16, as on
// the prefill path.
//
// Grid: (expert slot, row tile).  Slots index the active-expert list built by
// moe_permute, walked from its end (shared experts, which serve every token,
// come first, so the longest blocks start first); blocks whose slot is past
// the list's end exit at once, so the host never needs the routing result.
// A wave holds few rows so that several waves share each SIMD: while some
// wait for their weights, others compute.
#pragma once
#include "format.h"

namespace moeq {
namespace decode_detail {

constexpr int kMaxNT = 2;        // tokens per pass over the weights

// NT tokens' activation slices (bf16 rows of `ld` elements) for chunk `cpos`
// as dot2 pairs in the format's pair order, with their fp32 sums.  Tokens
// t >= nt get zeros.
template <int BITS, int NT>
MOEQ_DEV void load_x_bf16(const uint16_t* __restrict__ x, const int (&rowidx)[NT], int nt, int cpos,
                          uint32_t (&X)[NT][Fmt<BITS>::PAIRS], float (&XS)[NT], int ld) {
  using F = Fmt<BITS>;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    uint32_t v[F::CODES / 2];
    if (t < nt) {
      const uint16_t* src = x + (size_t)rowidx[t] * ld + (size_t)cpos * F::CODES;
#pragma unroll
      for (int i = 0; i < F::CODES / 8; ++i) {
        const moeq_u32x4 q = *reinterpret_cast<const moeq_u32x4*>(src + 8 * i);
        v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < F::CODES / 2; ++i) v[i] = 0u;
    }
    float s = 0.0f;
    const uint32_t ones = 0x3F803F80u;   // bf16 (1, 1): dot2 with it sums a pair
#pragma unroll
    for (int p = 0; p < F::PAIRS; ++p) {
      const int c0 = pair_code<BITS>(p, 0), c1 = pair_code<BITS>(p, 1);
      const uint32_t lo = (v[c0 >> 1] >> (16 * (c0 & 1))) & 0xFFFFu;
      const uint32_t hi = (v[c1 >> 1] >> (16 * (c1 & 1))) & 0xFFFFu;
      X[t][p] = lo | (hi << 16);
      s = dot2_bf16(X[t][p], ones, s);
    }
    XS[t] = s;
  }
}

// The intermediate h of the down projection comes from the gate/up kernel
// as bf16, stored in the down kernel's pair order (h_store_pos), so a
// chunk's pairs load directly.  XS is the fp32 sum of the chunk's h values.
template <int BITS, int NT>
MOEQ_DEV void load_h_pairs(const uint16_t* __restrict__ hh, int row0, int nt, int cpos,
                           uint32_t (&XH)[NT][Fmt<BITS>::PAIRS], float (&XS)[NT], int ld) {
  using F = Fmt<BITS>;
  const uint32_t ones = 0x3F803F80u;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < nt) {
      const size_t off = (size_t)(row0 + t) * ld + (size_t)cpos * F::CODES;
#pragma unroll
      for (int i = 0; i < F::PAIRS / 4; ++i) {
        const moeq_u32x4 a = *reinterpret_cast<const moeq_u32x4*>(hh + off + 8 * i);
        XH[t][4 * i] = a.x; XH[t][4 * i + 1] = a.y; XH[t][4 * i + 2] = a.z; XH[t][4 * i + 3] = a.w;
      }
    } else {
#pragma unroll
      for (int p = 0; p < F::PAIRS; ++p) XH[t][p] = 0u;
    }
    float s = 0.0f;
#pragma unroll
    for (int p = 0; p < F::PAIRS; ++p) s = dot2_bf16(XH[t][p], ones, s);
    XS[t] = s;
  }
}

// Where natural index i of a K = I row of h is stored for a down projection
// at DBITS: chunk-major, and inside a chunk pair p's two halves at 2p, 2p+1
// (the inverse of pair_code).  4-bit: code 8q + r sits in pair 4q + (r & 3),
// half r >> 2.  8-bit: pairs are natural.  6-bit: a 16-entry nibble table.
template <int DBITS>
MOEQ_DEV int h_store_pos(int i) {
  using F = Fmt<DBITS>;
  const int c = i / F::CODES, j = i % F::CODES;
  int pos;
  if constexpr (DBITS == 4) {
    pos = (j & ~7) + 2 * (j & 3) + ((j >> 2) & 1);
  } else if constexpr (DBITS == 8) {
    pos = j;
  } else {
    // position of code j: codes (0,3)->(0,1), (1,4)->(2,3), (5,8)->(4,5),
    // (6,9)->(6,7), (10,13)->(8,9), (11,14)->(10,11), (2,7)->(12,13),
    // (12,15)->(14,15)
    constexpr uint64_t kPos = 0xFB9EA875D6431C20ull;   // nibble j = position of code j
    pos = (int)((kPos >> (4 * j)) & 0xF);
  }
  return c * F::CODES + pos;
}

// Partial dot products of one row chunk against NT tokens with the group's
// scale/zero applied: out[t] += s * (sum (off+q) x - (z+off) * sum x).
template <int BITS, int NT>
MOEQ_DEV void chunk_dot(const uint32_t (&d)[Fmt<BITS>::DW], uint32_t szw, const uint32_t (&X0)[NT][Fmt<BITS>::PAIRS],
                        const float (&XS)[NT], float (&out)[NT]) {
  using F = Fmt<BITS>;
  uint32_t P[F::PAIRS];
  chunk_pairs<BITS>(d, P);
  const float s = f16_bits_to_f32(szw & 0xFFFFu);
  const float zc = f16_bits_to_f32(szw >> 16) + F::OFFSET;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    // four independent accumulation chains: the dot2 results are not
    // waited on one after another
    float a[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < F::PAIRS; ++p) {
      a[p & 3] = dot2_bf16(P[p], X0[t][p], a[p & 3]);
    }
    const float acc = (a[0] + a[1]) + (a[2] + a[3]);
    out[t] = fmaf(s, acc - zc * XS[t], out[t]);
  }
}

// Empty register-only barrier (no instruction is emitted): makes the packed
// weights look modified at the start of each token pass, so the compiler
// re-derives the bf16 pairs per pass instead of keeping all of them live.
template <int CH, int DW>
MOEQ_DEV void opaque(uint32_t (&d)[CH][DW]) {
#pragma unroll
  for (int s = 0; s < CH; ++s)
#pragma unroll
    for (int j = 0; j < DW; ++j) asm volatile("" : "+v"(d[s][j]));
}

template <int ITER, int LPR>
struct Geo {
  static constexpr int iter = ITER;      // chunks per lane per row
  static constexpr int lpr = LPR;        // lanes per row
  static constexpr int rpw = 64 / LPR;   // rows per wave step
  int rg, cl;           // this lane's row within a step and its chunk column
  MOEQ_DEV Geo() {
    const int lane = threadIdx.x & 63;
    rg = lane / LPR;
    cl = lane % LPR;
  }
  MOEQ_DEV bool writer() const { return cl == LPR - 1; }   // holds the row sum
  // chunk s of this lane: row step s / iter, chunk column cl + lpr * (s % iter)
  MOEQ_DEV int row_of(int s) const { return (s / ITER) * rpw + rg; }
  MOEQ_DEV int cpos_of(int s) const { return cl + lpr * (s % ITER); }
};

#ifndef MOEQ_GU_CH1
#define MOEQ_GU_CH1 2
#endif
#ifndef MOEQ_DN_CH1
#define MOEQ_DN_CH1 4
#endif
#ifndef MOEQ_NT2_MAX_ITER
#define MOEQ_NT2_MAX_ITER 1
#endif
#ifndef MOEQ_GU_WAVES
#define MOEQ_GU_WAVES 4
#endif
#ifndef MOEQ_DN_WAVES
#define MOEQ_DN_WAVES 4
#endif
// chunks per lane and matrix held in registers (a multiple of iter)
constexpr int gateup_ch(int iter) { return iter == 1 ? MOEQ_GU_CH1 : iter; }
constexpr int down_ch(int iter) { return iter == 1 ? MOEQ_DN_CH1 : (iter == 3 ? 3 : 4); }
constexpr int kGateupWaves = MOEQ_GU_WAVES;   // minimum waves per SIMD the register budget allows
constexpr int kDownWaves = MOEQ_DN_WAVES;

// -------------------------------------------------------------------------
// gate/up: h[p][i] = silu(Wg x_t)[i] * (Wu x_t)[i]
// A wave owns CH/ITER row steps (CH chunks of gate and of up per lane).  All
// of its weight chunks are loaded into registers first; then every pass over
// up to kMaxNT of the expert's tokens reuses them, one chunk column (ITER)
// of activations at a time.
// -------------------------------------------------------------------------
template <int BITS, int DBITS, int ITER, int LPR, int CH, int NT>
MOEQ_DEV void gateup_pass(uint32_t (&dg)[CH][Fmt<BITS>::DW], uint32_t (&du)[CH][Fmt<BITS>::DW],
                          const uint32_t (&sg)[CH], const uint32_t (&su)[CH], const uint16_t* __restrict__ x,
                          int H, int I, int kS, const int32_t* __restrict__ sorted, int p0, int nt, int row0,
                          int I_end, const Geo<ITER, LPR>& g, uint16_t* __restrict__ hh) {
  using F = Fmt<BITS>;
  opaque(dg);
  opaque(du);
  int tok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) tok[t] = t < nt ? sorted[p0 + t] / kS : 0;
  float ag[CH][NT], au[CH][NT];
#pragma unroll
  for (int s = 0; s < CH; ++s)
#pragma unroll
    for (int t = 0; t < NT; ++t) { ag[s][t] = 0.0f; au[s][t] = 0.0f; }
#pragma unroll 1
  for (int it = 0; it < ITER; ++it) {
    uint32_t X[NT][F::PAIRS];
    float XS[NT];
    load_x_bf16<BITS, NT>(x, tok, nt, g.cl + g.lpr * it, X, XS, H);
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      if (s % ITER == it) {
        chunk_dot<BITS, NT>(dg[s], sg[s], X, XS, ag[s]);
        chunk_dot<BITS, NT>(du[s], su[s], X, XS, au[s]);
      }
    }
  }
  // rows: chunks s = step*iter .. step*iter+iter-1 belong to row step `step`
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    if (s % ITER != 0) continue;
    float gs[NT], us[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) { gs[t] = ag[s][t]; us[t] = au[s][t]; }
#pragma unroll
    for (int q = 1; q < CH; ++q)
      if (q < ITER && s + q < CH) {
#pragma unroll
        for (int t = 0; t < NT; ++t) { gs[t] += ag[s + q][t]; us[t] += au[s + q][t]; }
      }
    const int row = row0 + g.row_of(s);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float gv = group_sum_last<LPR>(gs[t]);
      const float uv = group_sum_last<LPR>(us[t]);
      if (g.writer() && t < nt && row < I_end) {
        const float hv = silu_f32(gv) * uv;
        hh[(size_t)(p0 + t) * I + h_store_pos<DBITS>(row)] = (uint16_t)f32_to_bf16_bits(hv);
      }
    }
  }
}

template <int BITS, int DBITS, int ITER, int LPR>
__global__ __launch_bounds__(256, ITER <= 2 ? kGateupWaves : 2) void gateup_gemv_kernel(const uint8_t* __restrict__ gq, const uint32_t* __restrict__ gsz,
                                                          const uint8_t* __restrict__ uq, const uint32_t* __restrict__ usz,
                                                          const uint16_t* __restrict__ x, int H, int I, int kS,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted,
                                                          const int32_t* __restrict__ active, int tiles,
                                                          uint16_t* __restrict__ hh) {
  using F = Fmt<BITS>;
  constexpr int CH = gateup_ch(ITER);
  const int n_active = min(active[0], (int)(gridDim.x / tiles));   // the grid has a block row per possible slot
  const int slot = n_active - 1 - (int)(blockIdx.x / tiles), tile = blockIdx.x % tiles;
  if (slot < 0) return;
  const int e = active[1 + slot];
  const Geo<ITER, LPR> g;
  const int wave = threadIdx.x >> 6;
  const int rows_w = (CH / ITER) * g.rpw;
  const int row0 = (tile * 4 + wave) * rows_w;
  if (row0 >= I) return;
  const int I_end = min(I, row0 + rows_w);
  const size_t rb = row_bytes(H, BITS), gpr = H / 64;
  // all weight chunks of this wave first
  uint32_t dg[CH][F::DW], du[CH][F::DW], sg[CH], su[CH];
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    const int row = min(row0 + g.row_of(s), I - 1);   // rows past I repeat the last row, never stored
    const int cpos = g.cpos_of(s);
    const size_t grow = (size_t)e * I + row;
    load_chunk<BITS>(gq + grow * rb + (size_t)cpos * F::BYTES, dg[s]);
    load_chunk<BITS>(uq + grow * rb + (size_t)cpos * F::BYTES, du[s]);
    sg[s] = gsz[grow * gpr + cpos / F::CHUNKS_PER_GROUP];
    su[s] = usz[grow * gpr + cpos / F::CHUNKS_PER_GROUP];
  }
  const int pb = offsets[e], pe = offsets[e + 1];
  constexpr bool NT2 = ITER <= MOEQ_NT2_MAX_ITER;
  for (int p0 = pb; p0 < pe;) {
    if (NT2 && pe - p0 >= 2) {
      gateup_pass<BITS, DBITS, ITER, LPR, CH, 2>(dg, du, sg, su, x, H, I, kS, sorted, p0, 2, row0, I_end, g, hh);
      p0 += 2;
    } else {
      gateup_pass<BITS, DBITS, ITER, LPR, CH, 1>(dg, du, sg, su, x, H, I, kS, sorted, p0, 1, row0, I_end, g, hh);
      p0 += 1;
    }
  }
}

// -------------------------------------------------------------------------
// down: y[a][n] = (Wd h_p)[n] for the expert's assignments a = sorted[p]
// -------------------------------------------------------------------------
template <int BITS, int ITER, int LPR, int CH, int NT>
MOEQ_DEV void down_pass(uint32_t (&d)[CH][Fmt<BITS>::DW], const uint32_t (&sw)[CH], const uint16_t* __restrict__ hh,
                        int H, int I, const int32_t* __restrict__ sorted, int p0, int nt, int row0, int H_end,
                        const Geo<ITER, LPR>& g, float* __restrict__ y) {
  using F = Fmt<BITS>;
  opaque(d);
  int arow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) arow[t] = t < nt ? sorted[p0 + t] : 0;
  float ac[CH][NT];
#pragma unroll
  for (int s = 0; s < CH; ++s)
#pragma unroll
    for (int t = 0; t < NT; ++t) ac[s][t] = 0.0f;
#pragma unroll 1
  for (int it = 0; it < ITER; ++it) {
    uint32_t XH[NT][F::PAIRS];
    float XS[NT];
    load_h_pairs<BITS, NT>(hh, p0, nt, g.cl + g.lpr * it, XH, XS, I);
#pragma unroll
    for (int s = 0; s < CH; ++s)
      if (s % ITER == it) chunk_dot<BITS, NT>(d[s], sw[s], XH, XS, ac[s]);
  }
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    if (s % ITER != 0) continue;
    float cs[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) cs[t] = ac[s][t];
#pragma unroll
    for (int q = 1; q < CH; ++q)
      if (q < ITER && s + q < CH) {
#pragma unroll
        for (int t = 0; t < NT; ++t) cs[t] += ac[s + q][t];
      }
    const int row = row0 + g.row_of(s);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float v = group_sum_last<LPR>(cs[t]);
      if (g.writer() && t < nt && row < H_end) y[(size_t)arow[t] * H + row] = v;
    }
  }
}

template <int BITS, int ITER, int LPR>
__global__ __launch_bounds__(256, ITER <= 2 ? kDownWaves : 2) void down_gemv_kernel(const uint8_t* __restrict__ dq, const uint32_t* __restrict__ dsz,
                                                        const uint16_t* __restrict__ hh, int H, int I,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ sorted,
                                                        const int32_t* __restrict__ active, int tiles,
                                                        float* __restrict__ y) {
  using F = Fmt<BITS>;
  constexpr int CH = down_ch(ITER);
  const int n_active = min(active[0], (int)(gridDim.x / tiles));   // the grid has a block row per possible slot
  const int slot = n_active - 1 - (int)(blockIdx.x / tiles), tile = blockIdx.x % tiles;
  if (slot < 0) return;
  const int e = active[1 + slot];
  const Geo<ITER, LPR> g;
  const int wave = threadIdx.x >> 6;
  const int rows_w = (CH / ITER) * g.rpw;
  const int row0 = (tile * 4 + wave) * rows_w;
  if (row0 >= H) return;
  const int H_end = min(H, row0 + rows_w);
  const size_t rb = row_bytes(I, BITS), gpr = I / 64;
  uint32_t d[CH][F::DW], sw[CH];
#pragma unroll
  for (int s = 0; s < CH; ++s) {
    const int row = min(row0 + g.row_of(s), H - 1);
    const int cpos = g.cpos_of(s);
    const size_t grow = (size_t)e * H + row;
    load_chunk<BITS>(dq + grow * rb + (size_t)cpos * F::BYTES, d[s]);
    sw[s] = dsz[grow * gpr + cpos / F::CHUNKS_PER_GROUP];
  }
  const int pb = offsets[e], pe = offsets[e + 1];
  constexpr bool NT2 = ITER <= MOEQ_NT2_MAX_ITER;
  for (int p0 = pb; p0 < pe;) {
    if (NT2 && pe - p0 >= 2) {
      down_pass<BITS, ITER, LPR, CH, 2>(d, sw, hh, H, I, sorted, p0, 2, row0, H_end, g, y);
      p0 += 2;
    } else {
      down_pass<BITS, ITER, LPR, CH, 1>(d, sw, hh, H, I, sorted, p0, 1, row0, H_end, g, y);
      p0 += 1;
    }
  }
}

}  // namespace decode_detail

// Per-bit-width launchers (one translation unit each, decode_b{4,6,8}.hip).
#define MOEQ_DECODE_LAUNCHERS(B, SPEC)                                                                   \
  SPEC int decode_gateup_b##B(const moe_layer_desc* L, const uint16_t* x, const int32_t* offsets,        \
                              const int32_t* sorted, const int32_t* active, int slots, int rows_per_wave, \
                              int lpr, int iter, uint16_t* hh, hipStream_t s)
#define MOEQ_DOWN_LAUNCHER(B, SPEC)                                                                      \
  SPEC int decode_down_b##B(const moe_layer_desc* L, const uint16_t* hh,                                 \
                            const int32_t* offsets, const int32_t* sorted, const int32_t* active,        \
                            int slots, int rows_per_wave, int lpr, int iter, float* y, hipStream_t s)

MOEQ_DECODE_LAUNCHERS(4, );
MOEQ_DECODE_LAUNCHERS(6, );
MOEQ_DECODE_LAUNCHERS(8, );
MOEQ_DOWN_LAUNCHER(4, );
MOEQ_DOWN_LAUNCHER(6, );
MOEQ_DOWN_LAUNCHER(8, );

// (iter, lanes per row) combinations with a kernel: lpr is the largest power
// of two <= 64 dividing the chunks per row, iter the rest (1..4).
#define MOEQ_DEC_SWITCH(ITERV, LPRV, CALL, RC)                       \
  switch (ITERV * 100 + LPRV) {                                      \
    case 164: CALL(1, 64); break;                                    \
    case 132: CALL(1, 32); break;                                    \
    case 116: CALL(1, 16); break;                                    \
    case 108: CALL(1, 8); break;                                     \
    case 264: CALL(2, 64); break;                                    \
    case 364: CALL(3, 64); break;                                    \
    case 332: CALL(3, 32); break;                                    \
    case 316: CALL(3, 16); break;                                    \
    case 308: CALL(3, 8); break;                                     \
    case 464: CALL(4, 64); break;                                    \
    default: RC = set_error(MOEQ_ERR_UNSUPPORTED, "decode: no kernel for %d chunks x %d lanes", ITERV, LPRV); \
  }

#define MOEQ_DEFINE_DECODE(B)                                                                            \
  MOEQ_DECODE_LAUNCHERS(B, ) {                                                                           \
    const int tiles = (L->I + 4 * rows_per_wave - 1) / (4 * rows_per_wave);                              \
    const int grid = slots * tiles;                                                                      \
    int rc = MOEQ_OK;                                                                                    \
    MOEQ_DEC_SWITCH(iter, lpr, MOEQ_GATEUP_CALL, rc)                                                     \
    return rc != MOEQ_OK ? rc : check_launch("moe_qgemv_decode (gate/up)");                              \
  }                                                                                                      \
  MOEQ_DOWN_LAUNCHER(B, ) {                                                                              \
    const int tiles = (L->H + 4 * rows_per_wave - 1) / (4 * rows_per_wave);                              \
    const int grid = slots * tiles;                                                                      \
    int rc = MOEQ_OK;                                                                                    \
    MOEQ_DEC_SWITCH(iter, lpr, MOEQ_DOWN_CALL, rc)                                                       \
    return rc != MOEQ_OK ? rc : check_launch("moe_qgemv_decode (down)");                                 \
  }

}  // namespace moeq
