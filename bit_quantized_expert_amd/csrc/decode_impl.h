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
//   * rows are reduced across their LPR lanes with DPP; with ITER > 1 the
//     per-chunk partial sums of a row are added up in a small per-wave LDS
//     array, so only one chunk's activations occupy registers at a time.
// The down projection reads h in fp32, split into two bf16 terms (hi + lo),
// so its dot products carry about 16 significant bits of h.
//
// Grid: (expert slot, row tile).  Slots index the active-expert list built by
// moe_permute; blocks whose slot is past its end exit at once, so the host
// never needs the routing result.
#pragma once
#include "format.h"

namespace moeq {
namespace decode_detail {

constexpr int kMaxNT = 2;        // tokens per pass over the weights
constexpr int kUnroll = 2;       // row steps whose loads are issued together
constexpr int kMaxRowsPerWave = 64;

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
#pragma unroll
    for (int p = 0; p < F::PAIRS; ++p) {
      const int c0 = pair_code<BITS>(p, 0), c1 = pair_code<BITS>(p, 1);
      const uint32_t lo = (v[c0 >> 1] >> (16 * (c0 & 1))) & 0xFFFFu;
      const uint32_t hi = (v[c1 >> 1] >> (16 * (c1 & 1))) & 0xFFFFu;
      X[t][p] = lo | (hi << 16);
      s += bf16_bits_to_f32(lo) + bf16_bits_to_f32(hi);
    }
    XS[t] = s;
  }
}

// Same for fp32 rows (the intermediate h): each value v is split into
// hi = bf16(v) and lo = bf16(v - hi); XS is the fp32 sum of hi + lo.
template <int BITS, int NT>
MOEQ_DEV void load_x_f32(const float* __restrict__ x, int row0, int nt, int cpos,
                         uint32_t (&XH)[NT][Fmt<BITS>::PAIRS], uint32_t (&XL)[NT][Fmt<BITS>::PAIRS],
                         float (&XS)[NT], int ld) {
  using F = Fmt<BITS>;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float v[F::CODES];
    if (t < nt) {
      const float* src = x + (size_t)(row0 + t) * ld + (size_t)cpos * F::CODES;
#pragma unroll
      for (int i = 0; i < F::CODES / 4; ++i) {
        const float4 q = *reinterpret_cast<const float4*>(src + 4 * i);
        v[4 * i] = q.x; v[4 * i + 1] = q.y; v[4 * i + 2] = q.z; v[4 * i + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < F::CODES; ++i) v[i] = 0.0f;
    }
    float s = 0.0f;
#pragma unroll
    for (int p = 0; p < F::PAIRS; ++p) {
      const float a = v[pair_code<BITS>(p, 0)], b = v[pair_code<BITS>(p, 1)];
      const uint32_t ah = f32_to_bf16_bits(a), bh = f32_to_bf16_bits(b);
      const uint32_t al = f32_to_bf16_bits(a - bf16_bits_to_f32(ah));
      const uint32_t bl = f32_to_bf16_bits(b - bf16_bits_to_f32(bh));
      XH[t][p] = ah | (bh << 16);
      XL[t][p] = al | (bl << 16);
      s += (bf16_bits_to_f32(ah) + bf16_bits_to_f32(al)) + (bf16_bits_to_f32(bh) + bf16_bits_to_f32(bl));
    }
    XS[t] = s;
  }
}

// Partial dot products of one row chunk against NT tokens with the group's
// scale/zero applied: out[t] += s * (sum (off+q) x - (z+off) * sum x).
// NX = 2 adds the second (lo) activation term.
template <int BITS, int NT, int NX>
MOEQ_DEV void chunk_dot(const uint32_t (&d)[Fmt<BITS>::DW], uint32_t szw, const uint32_t (&X0)[NT][Fmt<BITS>::PAIRS],
                        const uint32_t (&X1)[NT][Fmt<BITS>::PAIRS], const float (&XS)[NT], float (&out)[NT]) {
  using F = Fmt<BITS>;
  uint32_t P[F::PAIRS];
  chunk_pairs<BITS>(d, P);
  const float s = f16_bits_to_f32(szw & 0xFFFFu);
  const float zc = f16_bits_to_f32(szw >> 16) + F::OFFSET;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float a = 0.0f;
#pragma unroll
    for (int p = 0; p < F::PAIRS; ++p) {
      a = dot2_bf16(P[p], X0[t][p], a);
      if constexpr (NX == 2) a = dot2_bf16(P[p], X1[t][p], a);
    }
    out[t] = fmaf(s, a - zc * XS[t], out[t]);
  }
}

struct Geo {
  int lpr, iter, rpw;   // lanes per row, chunks per lane, rows per wave step
  int rg, cl;           // this lane's row within the step and chunk column
  MOEQ_DEV Geo(int lpr_, int iter_) : lpr(lpr_), iter(iter_), rpw(64 / lpr_) {
    const int lane = threadIdx.x & 63;
    rg = lane / lpr;
    cl = lane % lpr;
  }
};

// -------------------------------------------------------------------------
// gate/up: h[p][i] = silu(Wg x_t)[i] * (Wu x_t)[i] for tokens p0..p0+nt
// -------------------------------------------------------------------------
template <int BITS, int NT>
MOEQ_DEV void gateup_rows(const uint8_t* __restrict__ gq, const uint32_t* __restrict__ gsz,
                          const uint8_t* __restrict__ uq, const uint32_t* __restrict__ usz,
                          const uint16_t* __restrict__ x, int H, int I, int kS, const int32_t* __restrict__ sorted,
                          int e, int p0, int nt, int row_begin, int row_end, const Geo& g, float* part,
                          float* __restrict__ h) {
  using F = Fmt<BITS>;
  int tok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) tok[t] = t < nt ? sorted[p0 + t] / kS : 0;
  const size_t rb = row_bytes(H, BITS), gpr = H / 64;
  for (int it = 0; it < g.iter; ++it) {
    const int cpos = g.cl + g.lpr * it;
    uint32_t X[NT][F::PAIRS];
    float XS[NT];
    load_x_bf16<BITS, NT>(x, tok, nt, cpos, X, XS, H);
    for (int r0 = row_begin; r0 < row_end; r0 += kUnroll * g.rpw) {
      uint32_t dg[kUnroll][F::DW], du[kUnroll][F::DW], sg[kUnroll], su[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (r0 + u * g.rpw < row_end) {
          const size_t grow = (size_t)e * I + r0 + u * g.rpw + g.rg;
          load_chunk<BITS>(gq + grow * rb + (size_t)cpos * F::BYTES, dg[u]);
          load_chunk<BITS>(uq + grow * rb + (size_t)cpos * F::BYTES, du[u]);
          sg[u] = gsz[grow * gpr + cpos / F::CHUNKS_PER_GROUP];
          su[u] = usz[grow * gpr + cpos / F::CHUNKS_PER_GROUP];
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (r0 + u * g.rpw >= row_end) break;
        const int row = r0 + u * g.rpw + g.rg;
        float cg[NT], cu[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) { cg[t] = 0.0f; cu[t] = 0.0f; }
        chunk_dot<BITS, NT, 1>(dg[u], sg[u], X, X, XS, cg);
        chunk_dot<BITS, NT, 1>(du[u], su[u], X, X, XS, cu);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float gv = group_sum(cg[t], g.lpr);
          const float uv = group_sum(cu[t], g.lpr);
          if (g.cl == 0 && t < nt) {
            if (g.iter == 1) {
              h[(size_t)(p0 + t) * I + row] = silu_f32(gv) * uv;
            } else {
              float* pp = part + 2 * (NT * (row - row_begin) + t);
              if (it == 0) { pp[0] = gv; pp[1] = uv; }
              else { pp[0] += gv; pp[1] += uv; }
            }
          }
        }
      }
    }
  }
  if (g.iter > 1) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int lane = threadIdx.x & 63;
    for (int i = lane; i < (row_end - row_begin) * NT; i += 64) {
      const int rl = i / NT, t = i % NT;
      if (t < nt) h[(size_t)(p0 + t) * I + row_begin + rl] = silu_f32(part[2 * i]) * part[2 * i + 1];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void gateup_gemv_kernel(const uint8_t* __restrict__ gq, const uint32_t* __restrict__ gsz,
                                                          const uint8_t* __restrict__ uq, const uint32_t* __restrict__ usz,
                                                          const uint16_t* __restrict__ x, int H, int I, int kS,
                                                          const int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ sorted,
                                                          const int32_t* __restrict__ active, int tiles,
                                                          int rows_per_wave, int lpr, int iter,
                                                          float* __restrict__ h) {
  __shared__ float part_all[4][2 * kMaxNT * kMaxRowsPerWave];
  const int slot = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  if (slot >= active[0]) return;
  const int e = active[1 + slot];
  const int pb = offsets[e], pe = offsets[e + 1];
  const int wave = threadIdx.x >> 6;
  const int row_begin = (tile * 4 + wave) * rows_per_wave;
  const int row_end = min(I, row_begin + rows_per_wave);
  if (row_begin >= I) return;
  const Geo g(lpr, iter);
  float* part = part_all[wave];
  for (int p0 = pb; p0 < pe;) {
    if (pe - p0 >= 2) {
      gateup_rows<BITS, 2>(gq, gsz, uq, usz, x, H, I, kS, sorted, e, p0, 2, row_begin, row_end, g, part, h);
      p0 += 2;
    } else {
      gateup_rows<BITS, 1>(gq, gsz, uq, usz, x, H, I, kS, sorted, e, p0, 1, row_begin, row_end, g, part, h);
      p0 += 1;
    }
  }
}

// -------------------------------------------------------------------------
// down: y[a][n] = (Wd h_p)[n] for the expert's assignments a = sorted[p]
// -------------------------------------------------------------------------
template <int BITS, int NT>
MOEQ_DEV void down_rows(const uint8_t* __restrict__ dq, const uint32_t* __restrict__ dsz, const float* __restrict__ h,
                        int H, int I, const int32_t* __restrict__ sorted, int e, int p0, int nt, int row_begin,
                        int row_end, const Geo& g, float* part, float* __restrict__ y) {
  using F = Fmt<BITS>;
  int arow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) arow[t] = t < nt ? sorted[p0 + t] : 0;
  const size_t rb = row_bytes(I, BITS), gpr = I / 64;
  for (int it = 0; it < g.iter; ++it) {
    const int cpos = g.cl + g.lpr * it;
    uint32_t XH[NT][F::PAIRS], XL[NT][F::PAIRS];
    float XS[NT];
    load_x_f32<BITS, NT>(h, p0, nt, cpos, XH, XL, XS, I);
    for (int r0 = row_begin; r0 < row_end; r0 += kUnroll * g.rpw) {
      uint32_t d[kUnroll][F::DW], sw[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (r0 + u * g.rpw < row_end) {
          const size_t grow = (size_t)e * H + r0 + u * g.rpw + g.rg;
          load_chunk<BITS>(dq + grow * rb + (size_t)cpos * F::BYTES, d[u]);
          sw[u] = dsz[grow * gpr + cpos / F::CHUNKS_PER_GROUP];
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        if (r0 + u * g.rpw >= row_end) break;
        const int row = r0 + u * g.rpw + g.rg;
        float c[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) c[t] = 0.0f;
        chunk_dot<BITS, NT, 2>(d[u], sw[u], XH, XL, XS, c);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const float v = group_sum(c[t], g.lpr);
          if (g.cl == 0 && t < nt) {
            if (g.iter == 1) {
              y[(size_t)arow[t] * H + row] = v;
            } else {
              float* pp = part + NT * (row - row_begin) + t;
              if (it == 0) *pp = v;
              else *pp += v;
            }
          }
        }
      }
    }
  }
  if (g.iter > 1) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int lane = threadIdx.x & 63;
    for (int i = lane; i < (row_end - row_begin) * NT; i += 64) {
      const int rl = i / NT, t = i % NT;
      if (t < nt) y[(size_t)arow[t] * H + row_begin + rl] = part[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

template <int BITS>
__global__ __launch_bounds__(256) void down_gemv_kernel(const uint8_t* __restrict__ dq, const uint32_t* __restrict__ dsz,
                                                        const float* __restrict__ h, int H, int I,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ sorted,
                                                        const int32_t* __restrict__ active, int tiles,
                                                        int rows_per_wave, int lpr, int iter, float* __restrict__ y) {
  __shared__ float part_all[4][kMaxNT * kMaxRowsPerWave];
  const int slot = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  if (slot >= active[0]) return;
  const int e = active[1 + slot];
  const int pb = offsets[e], pe = offsets[e + 1];
  const int wave = threadIdx.x >> 6;
  const int row_begin = (tile * 4 + wave) * rows_per_wave;
  const int row_end = min(H, row_begin + rows_per_wave);
  if (row_begin >= H) return;
  const Geo g(lpr, iter);
  float* part = part_all[wave];
  for (int p0 = pb; p0 < pe;) {
    if (pe - p0 >= 2) {
      down_rows<BITS, 2>(dq, dsz, h, H, I, sorted, e, p0, 2, row_begin, row_end, g, part, y);
      p0 += 2;
    } else {
      down_rows<BITS, 1>(dq, dsz, h, H, I, sorted, e, p0, 1, row_begin, row_end, g, part, y);
      p0 += 1;
    }
  }
}

}  // namespace decode_detail

// Per-bit-width launchers (one translation unit each, decode_b{4,6,8}.hip).
#define MOEQ_DECODE_LAUNCHERS(B, SPEC)                                                                   \
  SPEC int decode_gateup_b##B(const moe_layer_desc* L, const uint16_t* x, const int32_t* offsets,        \
                              const int32_t* sorted, const int32_t* active, int slots, int rows_per_wave, \
                              int lpr, int iter, float* h, hipStream_t s)
#define MOEQ_DOWN_LAUNCHER(B, SPEC)                                                                      \
  SPEC int decode_down_b##B(const moe_layer_desc* L, const float* h, const int32_t* offsets,             \
                            const int32_t* sorted, const int32_t* active, int slots, int rows_per_wave,   \
                            int lpr, int iter, float* y, hipStream_t s)

MOEQ_DECODE_LAUNCHERS(4, );
MOEQ_DECODE_LAUNCHERS(6, );
MOEQ_DECODE_LAUNCHERS(8, );
MOEQ_DOWN_LAUNCHER(4, );
MOEQ_DOWN_LAUNCHER(6, );
MOEQ_DOWN_LAUNCHER(8, );

#define MOEQ_DEFINE_DECODE(B)                                                                            \
  MOEQ_DECODE_LAUNCHERS(B, ) {                                                                           \
    const int tiles = (L->I + 4 * rows_per_wave - 1) / (4 * rows_per_wave);                              \
    decode_detail::gateup_gemv_kernel<B><<<slots * tiles, 256, 0, s>>>(                                  \
        L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, L->k + L->S, offsets, sorted, active,   \
        tiles, rows_per_wave, lpr, iter, h);                                                             \
    return check_launch("moe_qgemv_decode (gate/up)");                                                   \
  }                                                                                                      \
  MOEQ_DOWN_LAUNCHER(B, ) {                                                                              \
    const int tiles = (L->H + 4 * rows_per_wave - 1) / (4 * rows_per_wave);                              \
    decode_detail::down_gemv_kernel<B><<<slots * tiles, 256, 0, s>>>(L->down.q, L->down.sz, h, L->H, L->I, \
                                                                     offsets, sorted, active, tiles,     \
                                                                     rows_per_wave, lpr, iter, y);       \
    return check_launch("moe_qgemv_decode (down)");                                                      \
  }

}  // namespace moeq
