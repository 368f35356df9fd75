// bf16 matrix-core tile machinery for gfx950 (v_mfma_f32_32x32x16_bf16).
//
// A block of 256 threads (4 wavefronts in a 2 x 2 grid) computes a
// BM x BN tile of C = A * B^T, A [M][K] and B [N][K] both K-contiguous, in
// K-slices of 64.  Each wave owns a (32*WM) x (32*WN) sub-tile held as WM x WN
// 32x32 fp32 accumulators.  Operand tiles live in LDS as rows of 64 bf16 plus
// 8 bf16 of padding (144-byte stride) so that the 16-byte operand reads of
// 8 consecutive rows fall in distinct banks.
//
// 32x32x16 operand layout: lane l supplies 8 consecutive k of row (l % 32) of
// A (k = 8*(l/32) .. +7) and likewise of column (l % 32) of B; accumulator
// element r of lane l is C[8*(r/4) + 4*(l/32) + r%4][l % 32].
#pragma once
#include "format.h"

namespace moeq {

constexpr int kBK = 64;                  // K-slice: exactly one quantisation group
constexpr int kLds = kBK + 8;            // LDS row stride in bf16
constexpr int kGemmMinTokens = 64;       // router uses the GEMM from this batch size

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

template <int WM, int WN>
struct WaveAcc {
  f32x16_t c[WM][WN];
  MOEQ_DEV void zero() {
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) c[i][j][r] = 0.0f;
  }
};

// One K-slice of MFMAs for a wave whose sub-tile starts at rows m0 of As and
// n0 of Bs (LDS tiles, stride kLds).
template <int WM, int WN>
MOEQ_DEV void mfma_slice(const uint16_t* As, const uint16_t* Bs, int m0, int n0, int lane, WaveAcc<WM, WN>& acc) {
  const int r = lane & 31, kh = (lane >> 5) * 8;
#pragma unroll
  for (int s = 0; s < kBK / 16; ++s) {
    bf16x8_t a[WM], b[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
      a[i] = *reinterpret_cast<const bf16x8_t*>(As + (m0 + 32 * i + r) * kLds + 16 * s + kh);
#pragma unroll
    for (int j = 0; j < WN; ++j)
      b[j] = *reinterpret_cast<const bf16x8_t*>(Bs + (n0 + 32 * j + r) * kLds + 16 * s + kh);
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.c[i][j], 0, 0, 0);
  }
}

// Row / column of accumulator element r of tile (i, j) within the wave's sub-tile.
MOEQ_DEV int acc_row(int i, int r, int lane) { return 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }
MOEQ_DEV int acc_col(int j, int lane) { return 32 * j + (lane & 31); }

// ---------------------------------------------------------------------------
// Plain bf16 rows -> LDS.  ROWS rows of 64 bf16 (8 x 16 B each); rows whose
// source pointer is NULL are zero-filled.  Staged through registers so the
// global loads of the next slice can be in flight during the MFMAs.
// ---------------------------------------------------------------------------
template <int ROWS>
struct RowStage {
  static constexpr int N = ROWS * 8 / 256;   // 16-byte pieces per thread
  moeq_u32x4 v[N];
  // src(j, row) returns the row's base pointer, or nullptr for a zero row;
  // piece j of this thread covers row (threadIdx.x / 8 + 32 j)
  template <class Src>
  MOEQ_DEV void load(Src src, int k0) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int c = threadIdx.x + 256 * j;
      const uint16_t* p = src(j, c >> 3);
      if (p) v[j] = *reinterpret_cast<const moeq_u32x4*>(p + k0 + (c & 7) * 8);
      else v[j] = moeq_u32x4{0u, 0u, 0u, 0u};
    }
  }
  MOEQ_DEV void store(uint16_t* lds) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int c = threadIdx.x + 256 * j;
      *reinterpret_cast<moeq_u32x4*>(lds + (c >> 3) * kLds + (c & 7) * 8) = v[j];
    }
  }
};

// ---------------------------------------------------------------------------
// Quantised rows -> dequantised bf16 in LDS.  For each of ROWS weight rows,
// the K-slice [k0, k0+64) is one group: its packed chunks and its scale/zero
// word are loaded to registers, then dequantised as (q - z) * s in fp32 and
// rounded to bf16 when stored.
// ---------------------------------------------------------------------------
template <int BITS, int ROWS>
struct QuantStage {
  using F = Fmt<BITS>;
  static constexpr int CPG = F::CHUNKS_PER_GROUP;
  static constexpr int N = ROWS * CPG / 256;   // chunks per thread
  static_assert(N >= 1 && ROWS * CPG % 256 == 0, "tile too small");
  uint32_t d[N][F::DW];
  uint32_t sz[N];
  // row(r, q, s, grow) gives the projection's code and scale/zero arrays
  // and the row index (over all experts) of tile row r; the K-slice
  // [k0, k0 + 64) is group k0 / 64 (tiled layout, format.h)
  template <class RowPtr>
  MOEQ_DEV void load(RowPtr row, int k0, int K) {
    const size_t cpr = (size_t)(K / F::CODES), gpr = (size_t)(K / 64);
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int c = threadIdx.x + 256 * j;
      const int r = c / CPG, ch = c % CPG;
      const uint8_t* q;
      const uint32_t* s;
      size_t grow;
      row(r, q, s, grow);
      load_chunk<BITS>(q + chunk_offset<BITS>(grow, (size_t)(k0 / 64) * CPG + ch, cpr), d[j]);
      sz[j] = s[sz_index(grow, (size_t)(k0 / 64), gpr)];
    }
  }
  MOEQ_DEV void store(uint16_t* lds) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int c = threadIdx.x + 256 * j;
      const int r = c / CPG, ch = c % CPG;
      const float s = f16_bits_to_f32(sz[j] & 0xFFFFu);
      const float z = f16_bits_to_f32(sz[j] >> 16);
      uint32_t codes[F::CODES];
      unpack_codes(d[j], codes);
      uint32_t out[F::CODES / 2];
#pragma unroll
      for (int i = 0; i < F::CODES / 2; ++i) {
        const float w0 = ((float)codes[2 * i] - z) * s;
        const float w1 = ((float)codes[2 * i + 1] - z) * s;
        out[i] = f32_to_bf16_bits(w0) | (f32_to_bf16_bits(w1) << 16);
      }
      uint16_t* dst = lds + r * kLds + ch * F::CODES;
#pragma unroll
      for (int i = 0; i < F::CODES / 8; ++i)
        *reinterpret_cast<moeq_u32x4*>(dst + 8 * i) =
            moeq_u32x4{out[4 * i], out[4 * i + 1], out[4 * i + 2], out[4 * i + 3]};
    }
  }
  // codes of one chunk in natural order (field n holds code field_code(n))
  static MOEQ_DEV void unpack_codes(const uint32_t (&w)[F::DW], uint32_t (&c)[F::CODES]) {
    if constexpr (BITS == 4) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int n = 0; n < 8; ++n) c[field_code<4>(8 * j + n)] = (w[j] >> (4 * n)) & 0xFu;
    } else if constexpr (BITS == 6) {
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const int b = 6 * n, dw = b >> 5, sh = b & 31;
        uint32_t v = w[dw] >> sh;
        if (sh > 26) v |= w[dw + 1] << (32 - sh);
        c[field_code<6>(n)] = v & 0x3Fu;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int n = 0; n < 4; ++n) c[4 * j + n] = (w[j] >> (8 * n)) & 0xFFu;
    }
  }
};

// Plain bf16 NT GEMM with fp32 output and an optional per-column bias:
// C[m][n] = sum_k A[m][k] B[n][k] + bias[n].  M, N arbitrary, K % 64 == 0.
int gemm_bf16_nt(const uint16_t* A, const uint16_t* B, const float* bias, int M, int N, int K, float* C,
                 hipStream_t stream);

}  // namespace moeq
