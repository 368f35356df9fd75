// Prefill path: grouped GEMMs over expert-sorted tokens on the bf16 matrix
// cores, with the expert weights dequantised into LDS tiles on the fly.
//
//   gate/up kernel: per (expert, 128-token tile, 128-feature tile), the
//     gathered token rows of x times the gate and up rows of that expert
//     (interleaved in 32-row blocks inside one 256-row B tile), epilogue
//     h = silu(g) * u rounded to bf16, stored in expert-sorted order.
//   down kernel: per (expert, token tile, 128-feature tile of H), the h rows
//     times the down rows, epilogue y rounded to bf16 and scattered to
//     assignment order.
// A schedule kernel turns the per-expert counts into the list of
// (expert, token tile) work items on the device, so the host never reads the
// routing back; blocks past the end of the list exit at once.
// Prior art: a long prompt touches nearly all experts (Qwen-tin, "Memory
// layout and performance"), so every expert's weights are streamed once per
// token tile.
#include "gemm_bf16.h"

using namespace moeq;

namespace {

constexpr int BM = kPrefillBM;   // 128 tokens per tile

// sched[0] = number of work items; sched[2 + 2i], sched[3 + 2i] = (expert, token tile)
__global__ __launch_bounds__(1024) void schedule_kernel(const int32_t* __restrict__ counts, int nexp,
                                                        int32_t* __restrict__ sched) {
  __shared__ int part[1024];
  const int tid = threadIdx.x;
  const int per = (nexp + 1023) / 1024;
  const int e0 = min(nexp, tid * per), e1 = min(nexp, e0 + per);
  int mine = 0;
  for (int e = e0; e < e1; ++e) mine += (counts[e] + BM - 1) / BM;
  part[tid] = mine;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {   // inclusive Hillis-Steele scan
    const int v = tid >= o ? part[tid - o] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int pos = part[tid] - mine;
  for (int e = e0; e < e1; ++e) {
    const int nt = (counts[e] + BM - 1) / BM;
    for (int m = 0; m < nt; ++m, ++pos) {
      sched[2 + 2 * pos] = e;
      sched[3 + 2 * pos] = m;
    }
  }
  if (tid == 1023) sched[0] = part[1023];
}

template <int BITS>
__global__ __launch_bounds__(256) void gateup_kernel(const uint8_t* __restrict__ gq, const uint32_t* __restrict__ gsz,
                                                     const uint8_t* __restrict__ uq, const uint32_t* __restrict__ usz,
                                                     const uint16_t* __restrict__ x, int H, int I, int kS,
                                                     const int32_t* __restrict__ counts,
                                                     const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ sorted,
                                                     const int32_t* __restrict__ sched, uint16_t* __restrict__ h) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[256 * kLds];
  const int tile = blockIdx.x;
  if (tile >= sched[0]) return;
  const int e = sched[2 + 2 * tile], mt = sched[3 + 2 * tile];
  const int n0 = blockIdx.y * 128;
  const int base = offsets[e] + mt * BM;
  const int rows = min(BM, counts[e] - mt * BM);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;

  // token row pointers of the A tile (rows tid/8 + 32 j)
  const uint16_t* arow[RowStage<BM>::N];
#pragma unroll
  for (int j = 0; j < RowStage<BM>::N; ++j) {
    const int r = (threadIdx.x >> 3) + 32 * j;
    arow[j] = r < rows ? x + (size_t)(sorted[base + r] / kS) * H : nullptr;
  }
  auto brow = [&](int rr, const uint8_t*& q, const uint32_t*& s, size_t& row) {
    const int blk = rr >> 5, f = n0 + 32 * (blk >> 1) + (rr & 31);
    row = (size_t)e * I + f;
    if (blk & 1) { q = uq; s = usz; }
    else { q = gq; s = gsz; }
  };
  RowStage<BM> sa;
  QuantStage<BITS, 256> sb;
  auto asrc = [&](int j, int r) { (void)r; return arow[j]; };
  WaveAcc<2, 4> acc;
  acc.zero();
  sa.load(asrc, 0);
  sb.load(brow, 0, H);
  sa.store(As);
  sb.store(Bs);
  __syncthreads();
  for (int k0 = 0; k0 < H; k0 += kBK) {
    const bool more = k0 + kBK < H;
    if (more) { sa.load(asrc, k0 + kBK); sb.load(brow, k0 + kBK, H); }
    mfma_slice<2, 4>(As, Bs, 64 * wm, 128 * wn, lane, acc);
    __syncthreads();
    if (more) { sa.store(As); sb.store(Bs); }
    __syncthreads();
  }
  // epilogue: tiles (0,1) and (2,3) are (gate, up) of the same 32 features
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 64 * wm + acc_row(i, r, lane);
        if (m < rows) {
          const int f = n0 + 64 * wn + 32 * jp + (lane & 31);
          const float g = acc.c[i][2 * jp][r], u = acc.c[i][2 * jp + 1][r];
          h[(size_t)(base + m) * I + f] = (uint16_t)f32_to_bf16_bits(silu_f32(g) * u);
        }
      }
}

template <int BITS>
__global__ __launch_bounds__(256) void down_kernel(const uint8_t* __restrict__ dq, const uint32_t* __restrict__ dsz,
                                                   const uint16_t* __restrict__ h, int H, int I,
                                                   const int32_t* __restrict__ counts,
                                                   const int32_t* __restrict__ offsets,
                                                   const int32_t* __restrict__ sorted,
                                                   const int32_t* __restrict__ sched, uint16_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[128 * kLds];
  const int tile = blockIdx.x;
  if (tile >= sched[0]) return;
  const int e = sched[2 + 2 * tile], mt = sched[3 + 2 * tile];
  const int n0 = blockIdx.y * 128;
  const int base = offsets[e] + mt * BM;
  const int rows = min(BM, counts[e] - mt * BM);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  auto asrc = [&](int, int r) -> const uint16_t* { return r < rows ? h + (size_t)(base + r) * I : nullptr; };
  auto brow = [&](int rr, const uint8_t*& q, const uint32_t*& s, size_t& row) {
    row = (size_t)e * H + n0 + rr;
    q = dq;
    s = dsz;
  };
  RowStage<BM> sa;
  QuantStage<BITS, 128> sb;
  WaveAcc<2, 2> acc;
  acc.zero();
  sa.load(asrc, 0);
  sb.load(brow, 0, I);
  sa.store(As);
  sb.store(Bs);
  __syncthreads();
  for (int k0 = 0; k0 < I; k0 += kBK) {
    const bool more = k0 + kBK < I;
    if (more) { sa.load(asrc, k0 + kBK); sb.load(brow, k0 + kBK, I); }
    mfma_slice<2, 2>(As, Bs, 64 * wm, 64 * wn, lane, acc);
    __syncthreads();
    if (more) { sa.store(As); sb.store(Bs); }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 64 * wm + acc_row(i, r, lane);
      if (m < rows) {
        const size_t a = (size_t)sorted[base + m];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + 64 * wn + acc_col(j, lane);
          y[a * H + n] = (uint16_t)f32_to_bf16_bits(acc.c[i][j][r]);
        }
      }
    }
}

// plain NT GEMM (router logits at large batch)
__global__ __launch_bounds__(256) void gemm_nt_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                      const float* __restrict__ bias, int M, int N, int K,
                                                      float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint16_t As[128 * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[128 * kLds];
  const int m0 = blockIdx.x * 128, n0 = blockIdx.y * 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  auto asrc = [&](int, int r) -> const uint16_t* { return m0 + r < M ? A + (size_t)(m0 + r) * K : nullptr; };
  auto bsrc = [&](int, int r) -> const uint16_t* { return n0 + r < N ? B + (size_t)(n0 + r) * K : nullptr; };
  RowStage<128> sa, sb;
  WaveAcc<2, 2> acc;
  acc.zero();
  sa.load(asrc, 0);
  sb.load(bsrc, 0);
  sa.store(As);
  sb.store(Bs);
  __syncthreads();
  for (int k0 = 0; k0 < K; k0 += kBK) {
    const bool more = k0 + kBK < K;
    if (more) { sa.load(asrc, k0 + kBK); sb.load(bsrc, k0 + kBK); }
    mfma_slice<2, 2>(As, Bs, 64 * wm, 64 * wn, lane, acc);
    __syncthreads();
    if (more) { sa.store(As); sb.store(Bs); }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 64 * wm + acc_row(i, r, lane);
      if (m < M) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int n = n0 + 64 * wn + acc_col(j, lane);
          if (n < N) C[(size_t)m * N + n] = acc.c[i][j][r] + (bias ? bias[n] : 0.0f);
        }
      }
    }
}

}  // namespace

namespace moeq {
int gemm_bf16_nt(const uint16_t* A, const uint16_t* B, const float* bias, int M, int N, int K, float* C,
                 hipStream_t stream) {
  if (M == 0 || N == 0) return MOEQ_OK;
  dim3 grid((M + 127) / 128, (N + 127) / 128);
  gemm_nt_kernel<<<grid, 256, 0, stream>>>(A, B, bias, M, N, K, C);
  return check_launch("router GEMM");
}
}  // namespace moeq

extern "C" int moe_qgemm_prefill(const moe_layer_desc* L, const uint16_t* x, int T, const int32_t* counts,
                                 const int32_t* offsets, const int32_t* sorted, uint16_t* y, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  int rc = validate_layer(L);
  if (rc != MOEQ_OK) return rc;
  if (T < 0) return set_error(MOEQ_ERR_INVALID_ARG, "moe_qgemm_prefill: T=%d", T);
  if (T == 0) return MOEQ_OK;
  if (!x || !counts || !offsets || !sorted || !y)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_qgemm_prefill: NULL pointer");
  if (!aligned16(x)) return set_error(MOEQ_ERR_MISALIGNED, "moe_qgemm_prefill: x must be 16-byte aligned");
  if (L->gate.bits != L->up.bits)
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_qgemm_prefill: gate and up must share a bit width");
  if (L->I % 128 || L->H % 128)
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_qgemm_prefill: H=%d and I=%d must be multiples of 128", L->H, L->I);
  const WsLayout wl = ws_layout(L->H, L->I, L->E, L->S, L->k, T);
  if (!ws || ws_bytes < wl.total)
    return set_error(MOEQ_ERR_WORKSPACE, "moe_qgemm_prefill: workspace of %zu bytes, need %zu", ws_bytes, wl.total);
  char* w = static_cast<char*>(ws);
  int32_t* sched = reinterpret_cast<int32_t*>(w + wl.sched);
  uint16_t* h = reinterpret_cast<uint16_t*>(w + wl.h);
  const int nexp = L->E + L->S, kS = L->k + L->S;
  const long A = (long)T * kS;
  const long max_tiles = prefill_max_tiles(A, nexp);
  schedule_kernel<<<1, 1024, 0, stream>>>(counts, nexp, sched);
  if ((rc = check_launch("moe_qgemm_prefill (schedule)")) != MOEQ_OK) return rc;
  dim3 g1((unsigned)max_tiles, L->I / 128);
  switch (L->gate.bits) {
    case 4: gateup_kernel<4><<<g1, 256, 0, stream>>>(L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, kS, counts, offsets, sorted, sched, h); break;
    case 6: gateup_kernel<6><<<g1, 256, 0, stream>>>(L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, kS, counts, offsets, sorted, sched, h); break;
    default: gateup_kernel<8><<<g1, 256, 0, stream>>>(L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, kS, counts, offsets, sorted, sched, h); break;
  }
  if ((rc = check_launch("moe_qgemm_prefill (gate/up)")) != MOEQ_OK) return rc;
  dim3 g2((unsigned)max_tiles, L->H / 128);
  switch (L->down.bits) {
    case 4: down_kernel<4><<<g2, 256, 0, stream>>>(L->down.q, L->down.sz, h, L->H, L->I, counts, offsets, sorted, sched, y); break;
    case 6: down_kernel<6><<<g2, 256, 0, stream>>>(L->down.q, L->down.sz, h, L->H, L->I, counts, offsets, sorted, sched, y); break;
    default: down_kernel<8><<<g2, 256, 0, stream>>>(L->down.q, L->down.sz, h, L->H, L->I, counts, offsets, sorted, sched, y); break;
  }
  return check_launch("moe_qgemm_prefill (down)");
}
