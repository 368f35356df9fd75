// Decode-batch routing: router logits, top-k with renormalised weights and
// the grouping of assignments by expert, in two small launches tuned for
// latency (decode is where small launches dominate: Raon-1-mini on an RTX
// 5070 Ti, optimisation table).
//
//  1. router_rows_kernel: one wavefront (one 64-thread block) per router row
//     (router_row, router.h): the row is loaded once into registers, the
//     tokens come straight from global memory (they stay in L2), dot
//     products in fp32 via dot2, DPP reduction.  Many tiny blocks spread the
//     row loads over every CU.
//  2. select_group_kernel: one block of 16 wavefronts; each wavefront selects
//     the top k of one token (candidates in registers, DPP arg-max), then
//     the block groups the assignments by expert exactly as moe_permute does.
// The kernel boundary orders the two; no cross-block synchronisation.
#include "router.h"

using namespace moeq;

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRowChunks = 8;                 // H <= 4096 (8 x 16 B per lane)
constexpr int kMaxA = 1024;
constexpr int kMaxExp = 1024;

template <int NCH>
__global__ __launch_bounds__(64) void router_rows_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wr,
                                                         const float* __restrict__ bias, int T, int E,
                                                         float* __restrict__ logits) {
  router_row<NCH>(x, wr, bias, T, E, (int)blockIdx.x, logits);
}

MOEQ_DEV int block_excl_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int s = tmp[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

// NS = candidate slots per lane = ceil(E / 64).
// Grouping by expert: a token's k experts are distinct, so the rank of
// assignment (t, j) among the assignments of its expert e is the number of
// earlier tokens that chose e.  For T <= 64 each expert keeps a 64-bit mask of
// the tokens that chose it and the rank is a popcount; longer batches count
// the earlier assignments directly.
template <int NS>
__global__ __launch_bounds__(kThreads) void select_group_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                                int S, int32_t* __restrict__ topk_idx,
                                                                float* __restrict__ topk_w,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted,
                                                                int32_t* __restrict__ inverse,
                                                                int32_t* __restrict__ active, int* __restrict__ status) {
  __shared__ int sid[kMaxA];
  __shared__ int cnt[kMaxExp];
  __shared__ int offs[kMaxExp];
  __shared__ int tmp[kWaves];
  __shared__ unsigned int mlo[kMaxExp], mhi[kMaxExp];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kS = k + S, nexp = E + S, A = T * kS;
  const bool masks = T <= 64;
  for (int ee = threadIdx.x; ee < nexp; ee += kThreads) { cnt[ee] = 0; mlo[ee] = 0u; mhi[ee] = 0u; }
  __syncthreads();
  for (int t = wave; t < T; t += kWaves) {
    int bi;
    float w;
    select_token<NS>(logits + (size_t)t * E, E, k, k, bi, w);
    if (lane < k) {
      sid[t * kS + lane] = bi;
      topk_idx[(size_t)t * k + lane] = bi;
      topk_w[(size_t)t * k + lane] = w;
      if (masks) atomicOr(t < 32 ? &mlo[bi] : &mhi[bi], 1u << (t & 31));
      else atomicAdd(&cnt[bi], 1);
    }
    for (int j = lane; j < S; j += 64) sid[t * kS + k + j] = E + j;
  }
  __syncthreads();
  if (masks)
    for (int ee = threadIdx.x; ee < E; ee += kThreads) cnt[ee] = __popc(mlo[ee]) + __popc(mhi[ee]);
  for (int ee = E + threadIdx.x; ee < nexp; ee += kThreads) cnt[ee] = T;   // shared experts serve every token
  __syncthreads();
  const int per = (nexp + kThreads - 1) / kThreads;
  const int e0 = min(nexp, (int)threadIdx.x * per), e1 = min(nexp, e0 + per);
  int sum = 0, nz = 0;
  for (int ee = e0; ee < e1; ++ee) { sum += cnt[ee]; nz += cnt[ee] > 0; }
  int total, total_nz;
  int pos = block_excl_scan(sum, tmp, total);
  int apos = block_excl_scan(nz, tmp, total_nz);
  for (int ee = e0; ee < e1; ++ee) {
    const int c = cnt[ee];
    counts[ee] = c;
    offsets[ee] = pos;
    offs[ee] = pos;
    pos += c;
    if (c > 0) active[1 + apos++] = ee;
  }
  if (threadIdx.x == 0) { offsets[nexp] = total; active[0] = total_nz; status[0] = A - total; }
  __syncthreads();
  for (int a = threadIdx.x; a < A; a += kThreads) {
    const int t = a / kS, id = sid[a];
    int r;
    if (id >= E) {
      r = t;
    } else if (masks) {
      const unsigned int lo = t >= 32 ? mlo[id] : (mlo[id] & ((1u << t) - 1u));
      const unsigned int hi = t <= 32 ? 0u : (mhi[id] & ((1u << (t - 32)) - 1u));
      r = __popc(lo) + __popc(hi);
    } else {
      // earlier tokens' assignments only: the token's own experts are distinct
      r = 0;
      const int b_end = t * kS;
#pragma unroll 8
      for (int b = 0; b < b_end; ++b) r += (sid[b] == id);
    }
    const int p = offs[id] + r;
    sorted[p] = a;
    inverse[a] = p;
  }
}

}  // namespace

namespace moeq {

int launch_router_rows(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H, int E,
                       float* logits, hipStream_t stream) {
  switch (H / 512) {
    case 1: router_rows_kernel<1><<<E, 64, 0, stream>>>(x, wr, bias, T, E, logits); break;
    case 2: router_rows_kernel<2><<<E, 64, 0, stream>>>(x, wr, bias, T, E, logits); break;
    case 4: router_rows_kernel<4><<<E, 64, 0, stream>>>(x, wr, bias, T, E, logits); break;
    default: router_rows_kernel<8><<<E, 64, 0, stream>>>(x, wr, bias, T, E, logits); break;
  }
  return check_launch("router logits");
}

}  // namespace moeq

extern "C" int moe_route_permute_decode(const uint16_t* x, const uint16_t* w_router, const float* bias, int T,
                                        int H, int E, int k, int S, float* logits, int32_t* topk_idx,
                                        float* topk_w, int32_t* counts, int32_t* offsets, int32_t* sorted,
                                        int32_t* inverse, int32_t* active, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  if (T < 0 || E <= 0 || k <= 0 || S < 0 || k > E)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_route_permute_decode: T=%d E=%d k=%d S=%d", T, E, k, S);
  if (E + S > kMaxExp) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_route_permute_decode: E+S=%d > %d", E + S, kMaxExp);
  if (k > 64) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_route_permute_decode: k=%d > 64", k);
  if ((long)T * (k + S) > kMaxA)
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_route_permute_decode: T*(k+S)=%ld > %d", (long)T * (k + S), kMaxA);
  if (H <= 0 || H % 512 || H / 512 > kMaxRowChunks || (H / 512) & (H / 512 - 1))
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_route_permute_decode: H=%d must be 512, 1024, 2048 or 4096", H);
  if (!x || !w_router || !logits || !topk_idx || !topk_w || !counts || !offsets || !sorted || !inverse || !active)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_route_permute_decode: NULL pointer");
  if (!aligned16(x) || !aligned16(w_router))
    return set_error(MOEQ_ERR_MISALIGNED, "moe_route_permute_decode: x and w_router must be 16-byte aligned");
  if (!ws || ws_bytes < 256) return set_error(MOEQ_ERR_WORKSPACE, "moe_route_permute_decode: workspace too small");
  if (T == 0) return MOEQ_OK;
  int* status = static_cast<int*>(ws);
  int rc = launch_router_rows(x, w_router, bias, T, H, E, logits, stream);
  if (rc != MOEQ_OK) return rc;
  const int ns = (E + 63) / 64;
  if (ns <= 1) select_group_kernel<1><<<1, kThreads, 0, stream>>>(logits, T, E, k, S, topk_idx, topk_w, counts, offsets, sorted, inverse, active, status);
  else if (ns <= 2) select_group_kernel<2><<<1, kThreads, 0, stream>>>(logits, T, E, k, S, topk_idx, topk_w, counts, offsets, sorted, inverse, active, status);
  else if (ns <= 4) select_group_kernel<4><<<1, kThreads, 0, stream>>>(logits, T, E, k, S, topk_idx, topk_w, counts, offsets, sorted, inverse, active, status);
  else if (ns <= 8) select_group_kernel<8><<<1, kThreads, 0, stream>>>(logits, T, E, k, S, topk_idx, topk_w, counts, offsets, sorted, inverse, active, status);
  else select_group_kernel<16><<<1, kThreads, 0, stream>>>(logits, T, E, k, S, topk_idx, topk_w, counts, offsets, sorted, inverse, active, status);
  return check_launch("moe_route_permute_decode (select)");
}
