// Shared pieces of the bf16 matrix-core kernels for gfx950
// (v_mfma_f32_32x32x16_bf16).
//
// 32x32x16 operand layout: lane l supplies 8 k-values of row (l % 32) of A
// and of column (l % 32) of B, lane half l / 32 the second 8 of the 16;
// accumulator element r of lane l is C[8*(r/4) + 4*(l/32) + r%4][l % 32].
#pragma once
#include "format.h"

namespace moeq {

constexpr int kBK = 64;                  // K-slice: exactly one quantisation group
constexpr int kLds = kBK + 8;            // LDS row stride in bf16 (144 bytes)
constexpr int kGemmMinTokens = 64;       // router uses the GEMM from this batch size

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// Plain bf16 NT GEMM with fp32 output and an optional per-column bias:
// C[m][n] = sum_k A[m][k] B[n][k] + bias[n].  M, N arbitrary, K % 64 == 0.
int gemm_bf16_nt(const uint16_t* A, const uint16_t* B, const float* bias, int M, int N, int K, float* C,
                 hipStream_t stream);

}  // namespace moeq
