// Grouping of (token, expert) assignments by expert: histogram, exclusive
// scan and a stable scatter, deterministic (no atomic decides an order).
//
// Assignment a = t*(k+S) + j has expert idx[t][j] for j < k and E + (j-k)
// for the shared slots.  Within a block of 1024 assignments the rank of an
// assignment among the block's assignments of the same expert is counted
// directly (each thread scans the ids before it in LDS); block histograms are
// scanned per expert across blocks, then across experts.  Batches of up to
// 1024 assignments (all decode batches) take one fused single-block kernel.
#include "common.h"

using namespace moeq;

namespace {

constexpr int kB = kPermBlock;   // 1024 assignments and threads per block
constexpr int kMaxExperts = 4096;

MOEQ_DEV int assignment_expert(const int32_t* __restrict__ idx, long a, int k, int kS, int E) {
  const long t = a / kS;
  const int j = (int)(a - t * kS);
  if (j >= k) return E + (j - k);
  const int e = idx[t * k + j];
  return (e >= 0 && e < E) ? e : -1;   // -1: out of range, skipped and counted
}

// Exclusive scan of one int per thread over a block of 1024 threads.
MOEQ_DEV int block_exclusive_scan(int v, int* tmp /* >= 16 ints */, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < 16; ++w) {
    const int s = tmp[w];
    if (w < wave) before += s;
    all += s;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

// rank of assignment `a` among the earlier assignments of the same expert in
// the block's id array sid[0..n)
MOEQ_DEV int local_rank(const int* sid, int i, int id) {
  int r = 0;
  for (int j = 0; j < i; ++j) r += (sid[j] == id);
  return r;
}

// Per-thread contiguous range of experts for the scans.
MOEQ_DEV void expert_range(int nexp, int& e0, int& e1) {
  const int per = (nexp + kB - 1) / kB;
  e0 = min(nexp, (int)threadIdx.x * per);
  e1 = min(nexp, e0 + per);
}

// Scan `cnt` (per-expert counts in LDS) into offsets/counts/active; offsets
// also go to `offs_lds` when given.  Returns the total.
MOEQ_DEV int scan_experts(const int* cnt, int nexp, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                          int32_t* __restrict__ active, int* tmp, int* offs_lds = nullptr) {
  int e0, e1;
  expert_range(nexp, e0, e1);
  int sum = 0, nz = 0;
  for (int e = e0; e < e1; ++e) { sum += cnt[e]; nz += cnt[e] > 0; }
  int total, total_nz;
  int pos = block_exclusive_scan(sum, tmp, total);
  int apos = block_exclusive_scan(nz, tmp, total_nz);
  for (int e = e0; e < e1; ++e) {
    const int c = cnt[e];
    counts[e] = c;
    offsets[e] = pos;
    if (offs_lds) offs_lds[e] = pos;
    pos += c;
    if (c > 0) active[1 + apos++] = e;
  }
  if (threadIdx.x == 0) { offsets[nexp] = total; active[0] = total_nz; }
  return total;
}

// A <= 1024: everything in one block.
__global__ __launch_bounds__(1024) void permute_small_kernel(const int32_t* __restrict__ idx, int A, int k, int kS,
                                                              int E, int nexp, int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted,
                                                              int32_t* __restrict__ inverse,
                                                              int32_t* __restrict__ active, int* __restrict__ status) {
  __shared__ int sid[kB];
  __shared__ int cnt[kMaxExperts];
  __shared__ int tmp[16];
  __shared__ int offs[kMaxExperts];
  const int a = threadIdx.x;
  const int id = a < A ? assignment_expert(idx, a, k, kS, E) : -2;
  sid[a] = id;
  for (int e = a; e < nexp; e += kB) cnt[e] = 0;
  __syncthreads();
  if (id >= 0) atomicAdd(&cnt[id], 1);   // counts only: order-free
  const int rank = id >= 0 ? local_rank(sid, a, id) : 0;
  __syncthreads();
  const int total = scan_experts(cnt, nexp, counts, offsets, active, tmp, offs);
  __syncthreads();
  if (a < A) {
    if (id >= 0) {
      const int p = offs[id] + rank;
      sorted[p] = a;
      inverse[a] = p;
    } else {
      inverse[a] = -1;
    }
  }
  if (a == 0) status[0] = A - total;
}

// Large A, pass 1: per-block histograms hist[b][e].
__global__ __launch_bounds__(1024) void permute_hist_kernel(const int32_t* __restrict__ idx, long A, int k, int kS,
                                                             int E, int nexp, int32_t* __restrict__ hist) {
  __shared__ int cnt[kMaxExperts];
  const long a = (long)blockIdx.x * kB + threadIdx.x;
  for (int e = threadIdx.x; e < nexp; e += kB) cnt[e] = 0;
  __syncthreads();
  const int id = a < A ? assignment_expert(idx, a, k, kS, E) : -2;
  if (id >= 0) atomicAdd(&cnt[id], 1);
  __syncthreads();
  int32_t* hb = hist + (size_t)blockIdx.x * nexp;
  for (int e = threadIdx.x; e < nexp; e += kB) hb[e] = cnt[e];
}

// Large A, pass 2 (one block): per expert, exclusive scan over blocks (in
// place in hist), then the scan over experts.
__global__ __launch_bounds__(1024) void permute_scan_kernel(int nblk, int nexp, long A, int32_t* __restrict__ hist,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ active, int* __restrict__ status) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int tmp[16];
  // the block counts 16 at a time, all loaded before the running sum
  for (int e = threadIdx.x; e < nexp; e += kB) {
    int run = 0;
    for (int b0 = 0; b0 < nblk; b0 += 16) {
      int v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = b0 + i < nblk ? hist[(size_t)(b0 + i) * nexp + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (b0 + i < nblk) {
          hist[(size_t)(b0 + i) * nexp + e] = run;
          run += v[i];
        }
      }
    }
    cnt[e] = run;
  }
  __syncthreads();
  const int total = scan_experts(cnt, nexp, counts, offsets, active, tmp);
  if (threadIdx.x == 0) status[0] = (int)(A - total);
}

// Large A, pass 3: stable scatter.  The rank of an assignment among the
// block's earlier ones of the same expert is the count in the earlier
// 256-assignment parts of the block (histograms of the parts, order-free
// atomic counts) plus a direct count over the earlier ids of its own part.
constexpr int kPart = 256;
__global__ __launch_bounds__(1024) void permute_scatter_kernel(const int32_t* __restrict__ idx, long A, int k, int kS,
                                                                int E, int nexp, const int32_t* __restrict__ hist,
                                                                const int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ sorted,
                                                                int32_t* __restrict__ inverse) {
  __shared__ int sid[kB];
  __shared__ int part_cnt[kB / kPart - 1][kMaxExperts];   // the last part's counts are never needed
  const long a = (long)blockIdx.x * kB + threadIdx.x;
  const int id = a < A ? assignment_expert(idx, a, k, kS, E) : -2;
  const int part = threadIdx.x / kPart;
  for (int i = threadIdx.x; i < (kB / kPart - 1) * nexp; i += kB) part_cnt[i / nexp][i % nexp] = 0;
  sid[threadIdx.x] = id;
  __syncthreads();
  if (id >= 0 && part < kB / kPart - 1) atomicAdd(&part_cnt[part][id], 1);
  __syncthreads();
  if (a >= A) return;
  if (id < 0) { inverse[a] = -1; return; }
  int rank = 0;
  for (int q = 0; q < part; ++q) rank += part_cnt[q][id];
  const int p0 = part * kPart;
  for (int j = p0; j < (int)threadIdx.x; ++j) rank += (sid[j] == id);
  const int p = offsets[id] + hist[(size_t)blockIdx.x * nexp + id] + rank;
  sorted[p] = (int32_t)a;
  inverse[a] = p;
}

// The same scatter for up to 1024 experts with parts of one wavefront: the
// direct count runs over at most 63 earlier ids instead of 255, and the 15
// earlier parts' counts (at most 64 each) are packed four to a 32-bit LDS
// word.  The ranks, and so the output, are the same.
constexpr int kPartW = 64;
constexpr int kScatterWMaxExperts = 1024;
__global__ __launch_bounds__(1024) void permute_scatter_w_kernel(const int32_t* __restrict__ idx, long A, int k,
                                                                  int kS, int E, int nexp,
                                                                  const int32_t* __restrict__ hist,
                                                                  const int32_t* __restrict__ offsets,
                                                                  int32_t* __restrict__ sorted,
                                                                  int32_t* __restrict__ inverse) {
  constexpr int NP = kB / kPartW - 1;   // the last part's counts are never needed
  constexpr int NW = kScatterWMaxExperts / 4;
  __shared__ int sid[kB];
  __shared__ uint32_t pc[NP][NW];
  const long a = (long)blockIdx.x * kB + threadIdx.x;
  const int id = a < A ? assignment_expert(idx, a, k, kS, E) : -2;
  const int part = threadIdx.x / kPartW;
  for (int i = threadIdx.x; i < NP * NW; i += kB) pc[i / NW][i % NW] = 0u;
  sid[threadIdx.x] = id;
  __syncthreads();
  if (id >= 0 && part < NP) atomicAdd(&pc[part][id >> 2], 1u << (8 * (id & 3)));
  __syncthreads();
  if (a >= A) return;
  if (id < 0) { inverse[a] = -1; return; }
  int rank = 0;
  for (int q = 0; q < part; ++q) rank += (int)((pc[q][id >> 2] >> (8 * (id & 3))) & 0xFFu);
  const int p0 = part * kPartW;
  for (int j = p0; j < (int)threadIdx.x; ++j) rank += (sid[j] == id);
  const int p = offsets[id] + hist[(size_t)blockIdx.x * nexp + id] + rank;
  sorted[p] = (int32_t)a;
  inverse[a] = p;
}

}  // namespace

extern "C" int moe_permute(const int32_t* topk_idx, int T, int k, int E, int S, int32_t* counts, int32_t* offsets,
                           int32_t* sorted, int32_t* inverse, int32_t* active, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
  if (T < 0 || k <= 0 || E <= 0 || S < 0 || k > E)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_permute: T=%d k=%d E=%d S=%d", T, k, E, S);
  if (E + S > kMaxExperts) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_permute: E+S=%d > %d", E + S, kMaxExperts);
  if (!counts || !offsets || !active || (T > 0 && (!topk_idx || !sorted || !inverse)))
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_permute: NULL pointer");
  const int nexp = E + S, kS = k + S;
  const long A = (long)T * kS;
  const int nblk = perm_blocks(A);
  const size_t need = 256 + align_up((size_t)nblk * nexp * sizeof(int32_t), 256);
  if (!ws || ws_bytes < need) return set_error(MOEQ_ERR_WORKSPACE, "moe_permute: workspace of %zu bytes, need %zu", ws_bytes, need);
  char* w = static_cast<char*>(ws);
  int* status = reinterpret_cast<int*>(w);
  int32_t* hist = reinterpret_cast<int32_t*>(w + 256);
  if (A <= kB) {
    permute_small_kernel<<<1, kB, 0, stream>>>(topk_idx, (int)A, k, kS, E, nexp, counts, offsets, sorted, inverse,
                                               active, status);
    return check_launch("moe_permute");
  }
  permute_hist_kernel<<<nblk, kB, 0, stream>>>(topk_idx, A, k, kS, E, nexp, hist);
  int rc = check_launch("moe_permute (histogram)");
  if (rc != MOEQ_OK) return rc;
  permute_scan_kernel<<<1, kB, 0, stream>>>(nblk, nexp, A, hist, counts, offsets, active, status);
  if ((rc = check_launch("moe_permute (scan)")) != MOEQ_OK) return rc;
  if (nexp <= kScatterWMaxExperts)
    permute_scatter_w_kernel<<<nblk, kB, 0, stream>>>(topk_idx, A, k, kS, E, nexp, hist, offsets, sorted, inverse);
  else
    permute_scatter_kernel<<<nblk, kB, 0, stream>>>(topk_idx, A, k, kS, E, nexp, hist, offsets, sorted, inverse);
  return check_launch("moe_permute (scatter)");
}
