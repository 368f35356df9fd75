// Stacked decode in one launch: a batch-1 token through L MoE blocks
// (RMSNorm -> router -> top-k -> gate/up -> down -> weighted combine ->
// residual), each block's phases separated by grid-wide barriers, the
// blocks' weights streamed by every CU of the chip.  The pages' decode lever
// is exactly this: small per-step kernel launches left most of the bandwidth
// unused, a persistent per-layer MoE megakernel recovered it (Raon-1-mini,
// optimisation table and result paragraph).
//
// A layer, for the residual stream x (bf16 [H], in global memory):
//   A  every block: n = RMSNorm(x) into LDS (and its 64-group sums);
//      router rows spread over all wavefronts: logits[e] = n . Wr[e]
//   -- grid barrier --
//   B  every block: top-k of the logits (first wavefront), into LDS;
//      gate/up units (slot j, 64-row tile of I, K slice p of H) spread over
//      all wavefronts: partial gate and up sums per row; the unit that
//      completes a (slot, tile) adds its P partials in slice order and
//      writes h = bf16(silu(g) u)
//   -- grid barrier --
//   C  every block: h of all slots into LDS (and its group sums);
//      down units (64-row tile of H, slot j, K slice p of I): partial rows;
//      the unit that completes a tile adds the partials (slices, then slots
//      in ascending order, weighted) and writes x = bf16(x + bf16(sum))
//   -- grid barrier --
// The dot products are the decode GEMV's (format.h): codes become bf16
// (128 + q, or q at 8 bits) pairs, v_dot2_f32_bf16 with the activations'
// pairs (read from LDS, the same address on every lane), and the group's
// scale and zero enter once per group in fp32.
//
// Everything one block writes and another reads (logits, partial sums, h,
// x, the barrier words) goes through device-scope atomic loads and stores,
// which the hardware keeps coherent across the XCDs' separate L2 caches.
// A wavefront orders its stores before its signal by waiting for its
// vector-memory counter to reach zero (s_waitcnt vmcnt(0): on gfx9 the
// counter covers stores too, and a device-scope store counts as done once it
// is visible device-wide) immediately before every arrival; the loads that
// follow an arrival depend on the arrival's returned value, so they are
// issued after it.  So no device-scope fence (an L2 write-back or
// invalidate) is needed anywhere: the weights stay cached, and a barrier
// costs one round of atomics.
//
// The table starts with a 64-byte header (layer count and H, I, E, k, S = 0)
// that every block checks against the launch's dimensions before it touches
// a layer; on a mismatch every block leaves at once (none has reached a
// barrier) and the workspace's error word gets bit 2.  A barrier wait that
// gives up (after about 2^26 sleeps) sets bit 1.  The error word is sticky
// until moe_stack_read_status reads it.
#include "decode_impl.h"

using namespace moeq;
using decode_detail::load_chunk_g;

namespace {

constexpr int kMaxH = 8192;      // LDS: n, bf16
constexpr int kMaxKI = 16384;    // LDS: h of all slots, bf16
constexpr int kMaxK = 16;

struct StackHeader {  // 64 bytes before the layers
  uint32_t magic, nlayers;
  int H, I, E, k;
  uint32_t pad[10];
};
static_assert(sizeof(StackHeader) == 64, "table header");
constexpr uint32_t kStackMagic = 0x4B545351u;   // "QSTK"

struct StackLayer {   // one block's weights (device pointers), 64 bytes
  const uint8_t* gq;
  const uint32_t* gsz;
  const uint8_t* uq;
  const uint32_t* usz;
  const uint8_t* dq;
  const uint32_t* dsz;
  const uint16_t* wr;
  int gbits, dbits;
};
static_assert(sizeof(StackLayer) == 64, "table entry");

struct StackDims {
  int H, I, E, k, L;
  int P;    // K slices of a gate/up row (over H)
  int PD;   // K slices of a down row (over I)
  float eps;
};

struct StackWs {
  float* logits;     // [E]
  float* gu_part;    // [k][I/64][P][2][64]
  uint32_t* h;       // [k][I/2]: bf16 pairs
  float* y_part;     // [H/64][k][PD][64]
  int* gu_cnt;       // [k][I/64], 16 ints apart, zero between uses
  int* y_cnt;        // [H/64], 16 ints apart, zero between uses
  unsigned* bar;     // [0] arrivals (zero between barriers), [1] generation
  int* err;          // bit 1: a barrier wait gave up; bit 2: table mismatch
};

// device-coherent accesses (see the header comment)
MOEQ_DEV float ld_f(const float* p) { return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MOEQ_DEV void st_f(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MOEQ_DEV uint32_t ld_u(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOEQ_DEV void st_u(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
// Wait until every vector-memory operation this wavefront issued has
// completed (s_waitcnt vmcnt(0), expcnt and lgkmcnt left free): its
// device-scope stores are then visible to every XCD and its loads have
// returned.  Issued right before each arrival at a counter.
MOEQ_DEV void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// keeps the compiler from moving memory operations across this point
MOEQ_DEV void wave_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup"); }

// Grid-wide barrier of the co-resident blocks (cooperative launch), in two
// levels so that no word is hit by more than a group's blocks: block b
// arrives at the count of group b % 8 (the blocks one XCD receives); the
// last of a group clears that count and arrives at the top count; the last
// of those clears it and advances the generation word of every group, on
// which each group's blocks wait.  Every wavefront waits for its own stores
// to complete before the block meets at __syncthreads, and the first thread
// waits for its generation load and for each clearing store before its next
// arrival.  A wait gives up after about 2^26 sleeps (seconds) and sets bit 1
// of err, so that every wavefront always reaches the end of the kernel.
//   bar[16 g]: count of group g; bar[128]: top count; bar[144 + 16 g]:
//   generation of group g (words 64 bytes apart)
MOEQ_DEV void grid_barrier(unsigned* bar, unsigned nblocks, int* err) {
  wait_vmem();   // this wavefront's stores are visible device-wide
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned grp = blockIdx.x % 8u;
    const unsigned ngroups = nblocks < 8u ? nblocks : 8u;
    const unsigned members = nblocks / 8u + (grp < nblocks % 8u ? 1u : 0u);
    unsigned* gen = bar + 144 + 16 * grp;
    const unsigned g0 = __hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_vmem();   // the generation is read before arriving
    wave_acquire();
    if (__hip_atomic_fetch_add(bar + 16 * grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == members) {
      __hip_atomic_store(bar + 16 * grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait_vmem();   // cleared before the group arrives above
      wave_acquire();
      if (__hip_atomic_fetch_add(bar + 128, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == ngroups) {
        __hip_atomic_store(bar + 128, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        wait_vmem();   // cleared before any generation moves
        wave_acquire();
        for (unsigned y = 0; y < ngroups; ++y)
          __hip_atomic_fetch_add(bar + 144 + 16 * y, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    unsigned spins = 0;
    while (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g0) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > (1u << 26)) {
        __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
    wave_acquire();
  }
  __syncthreads();
}

// Loads v(i) for i < n (n <= 64) all at once into b, so that they are in
// flight together.
template <class Fn>
MOEQ_DEV void load_all(int n, float (&b)[64], Fn&& v) {
#pragma unroll
  for (int i = 0; i < 64; ++i) b[i] = i < n ? v(i) : 0.0f;
}

template <int BITS, int NM>
MOEQ_DEV void unit_dot(const uint8_t* const (&q)[NM], const uint32_t* const (&sz)[NM], size_t row, int K, int g0,
                       int G, const uint16_t* xl, const float* xsl, float (&out)[NM]) {
  using F = Fmt<BITS>;
  constexpr int CPG = F::CHUNKS_PER_GROUP;
  const size_t cpr = (size_t)(K / F::CODES), gpr = (size_t)(K / 64);
#pragma unroll
  for (int m = 0; m < NM; ++m) out[m] = 0.0f;
  for (int g = g0; g < g0 + G; g += 2) {
    const int ng = min(2, g0 + G - g);
    uint32_t d[NM][2 * CPG][F::DW];
    uint32_t w[NM][2];
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      if (gg < ng) {
#pragma unroll
        for (int m = 0; m < NM; ++m) {
#pragma unroll
          for (int c = 0; c < CPG; ++c)
            load_chunk_g<BITS>((gbytes)(q[m] + chunk_offset<BITS>(row, (size_t)(g + gg) * CPG + c, cpr)),
                               d[m][gg * CPG + c]);
          w[m][gg] = sz[m][sz_index(row, (size_t)(g + gg), gpr)];
        }
      }
    }
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      if (gg < ng) {
        const float x_sum = xsl[g + gg];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
          for (int c = 0; c < CPG; ++c) {
            uint32_t P[F::PAIRS];
            chunk_pairs<BITS>(d[m][gg * CPG + c], P);
            const uint4* xp = reinterpret_cast<const uint4*>(xl + (size_t)(g + gg) * 64 + c * F::CODES);
#pragma unroll
            for (int p = 0; p < F::PAIRS; p += 4) {
              const uint4 X = xp[p / 4];
              a0 = dot2_bf16(P[p], X.x, a0);
              a1 = dot2_bf16(P[p + 1], X.y, a1);
              a0 = dot2_bf16(P[p + 2], X.z, a0);
              a1 = dot2_bf16(P[p + 3], X.w, a1);
            }
          }
          const float s = f16_bits_to_f32(w[m][gg] & 0xFFFFu);
          const float zc = f16_bits_to_f32(w[m][gg] >> 16) + F::OFFSET;
          out[m] = fmaf(s, (a0 + a1) - zc * x_sum, out[m]);
        }
      }
    }
  }
}

template <int NM>
MOEQ_DEV void unit_dot_bits(int bits, const uint8_t* const (&q)[NM], const uint32_t* const (&sz)[NM], size_t row,
                            int K, int g0, int G, const uint16_t* xl, const float* xsl, float (&out)[NM]) {
  switch (bits) {
    case 4: unit_dot<4, NM>(q, sz, row, K, g0, G, xl, xsl, out); break;
    case 6: unit_dot<6, NM>(q, sz, row, K, g0, G, xl, xsl, out); break;
    default: unit_dot<8, NM>(q, sz, row, K, g0, G, xl, xsl, out); break;
  }
}

// Top-k of E logits (first wavefront of the block) into LDS.
template <int NS>
MOEQ_DEV void select_into(const float* logits, int E, int k, int* sel_idx, float* sel_w) {
  int idx;
  float w;
  select_token<NS>(logits, E, k, k, idx, w);
  const int lane = threadIdx.x & 63;
  if (lane < k) {
    sel_idx[lane] = idx;
    sel_w[lane] = w;
  }
}

MOEQ_DEV void select_any(const float* logits, int E, int k, int* sel_idx, float* sel_w) {
  if (E <= 64) select_into<1>(logits, E, k, sel_idx, sel_w);
  else if (E <= 128) select_into<2>(logits, E, k, sel_idx, sel_w);
  else if (E <= 256) select_into<4>(logits, E, k, sel_idx, sel_w);
  else if (E <= 512) select_into<8>(logits, E, k, sel_idx, sel_w);
  else select_into<16>(logits, E, k, sel_idx, sel_w);
}

// Whether this wavefront is the last of total to arrive at a counter (its
// stores complete before it arrives); the last one then sees everyone's.
MOEQ_DEV bool last_arrival(int* cnt, int total) {
  wait_vmem();
  wave_acquire();
  int old = 0;
  if ((threadIdx.x & 63) == 0) old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = __shfl(old, 0);
  if (old != total - 1) return false;
  wave_acquire();
  return true;
}

// bf16 of this lane and of the next one as one word (for even lanes)
MOEQ_DEV uint32_t pair_with_next(uint32_t b) { return b | (__shfl_down(b, 1) << 16); }

__global__ __launch_bounds__(256) void stack_decode_kernel(const StackHeader* hdr, StackDims d, StackWs ws,
                                                           uint32_t* x2) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kMaxH];
  __shared__ float xsum[kMaxH / 64];
  __shared__ __attribute__((aligned(16))) uint16_t hs[kMaxKI];
  __shared__ float hsum[kMaxKI / 64];
  __shared__ float lg[1024];
  __shared__ int sel_idx[kMaxK];
  __shared__ float sel_w[kMaxK];
  __shared__ float red[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int gw = (int)blockIdx.x * 4 + wave, nw = (int)gridDim.x * 4;
  const int H = d.H, I = d.I, k = d.k;
  const int tI = I / 64, tH = H / 64;
  const unsigned nb = gridDim.x;
  {
    // every block reads the same header, so all leave or none does
    const StackHeader h0 = *hdr;
    if (h0.magic != kStackMagic || (int)h0.nlayers < d.L || h0.H != H || h0.I != I || h0.E != d.E || h0.k != k) {
      if (blockIdx.x == 0 && threadIdx.x == 0) __hip_atomic_fetch_or(ws.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
  const StackLayer* table = reinterpret_cast<const StackLayer*>(hdr + 1);
  for (int l = 0; l < d.L; ++l) {
    const StackLayer Ly = table[l];
    // ---- A: RMSNorm (every block), router rows (all wavefronts).  The
    // first router row's weights (they do not depend on x) are loaded first.
    constexpr int kRouterChunks = 4;   // H <= 2048 fully; the rest of longer rows after x
    uint4 wfirst[kRouterChunks];
    if (gw < d.E) {
      const uint16_t* wrow = Ly.wr + (size_t)gw * H;
#pragma unroll
      for (int c = 0; c < kRouterChunks; ++c)
        if (c * 512 < H) wfirst[c] = *reinterpret_cast<const uint4*>(wrow + c * 512 + lane * 8);
    }
    float ss = 0.0f;
    for (int i0 = threadIdx.x; i0 < H / 2; i0 += 256 * 4) {
      uint32_t v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = i0 + 256 * u < H / 2 ? ld_u(x2 + i0 + 256 * u) : 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (i0 + 256 * u < H / 2) {
          const float a = bf16_bits_to_f32(v[u] & 0xFFFFu), b = bf16_bits_to_f32(v[u] >> 16);
          reinterpret_cast<uint32_t*>(xs)[i0 + 256 * u] = v[u];
          ss = fmaf(a, a, ss);
          ss = fmaf(b, b, ss);
        }
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float r = 1.0f / sqrtf(tot / (float)H + d.eps);
    for (int i = threadIdx.x; i < H; i += 256) xs[i] = (uint16_t)f32_to_bf16_bits(bf16_bits_to_f32(xs[i]) * r);
    __syncthreads();
    for (int g = wave; g < tH; g += 4) {
      const float s = wave_sum(bf16_bits_to_f32(xs[g * 64 + lane]));
      if (lane == 0) xsum[g] = s;
    }
    for (int e = gw; e < d.E; e += nw) {
      const uint16_t* wrow = Ly.wr + (size_t)e * H;
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < kRouterChunks; ++c) {
        if (c * 512 < H) {
          const uint4 wv = e == gw ? wfirst[c] : *reinterpret_cast<const uint4*>(wrow + c * 512 + lane * 8);
          const uint4 nv = *reinterpret_cast<const uint4*>(xs + c * 512 + lane * 8);
          acc = dot2_bf16(wv.x, nv.x, acc);
          acc = dot2_bf16(wv.y, nv.y, acc);
          acc = dot2_bf16(wv.z, nv.z, acc);
          acc = dot2_bf16(wv.w, nv.w, acc);
        }
      }
      for (int c = kRouterChunks * 512 + lane * 8; c < H; c += 512) {
        const uint4 wv = *reinterpret_cast<const uint4*>(wrow + c);
        const uint4 nv = *reinterpret_cast<const uint4*>(xs + c);
        acc = dot2_bf16(wv.x, nv.x, acc);
        acc = dot2_bf16(wv.y, nv.y, acc);
        acc = dot2_bf16(wv.z, nv.z, acc);
        acc = dot2_bf16(wv.w, nv.w, acc);
      }
      acc = wave_sum(acc);
      if (lane == 0) st_f(ws.logits + e, acc);
    }
    grid_barrier(ws.bar, nb, ws.err);
    // ---- B: top-k (every block), gate/up units (all wavefronts)
    for (int e = threadIdx.x; e < d.E; e += 256) lg[e] = ld_f(ws.logits + e);
    __syncthreads();
    if (wave == 0) select_any(lg, d.E, k, sel_idx, sel_w);
    __syncthreads();
    {
      const int P = d.P, G = tH / P;
      const int nunits = k * tI * P;
      for (int u = gw; u < nunits; u += nw) {
        const int j = u / (tI * P), t = (u / P) % tI, p = u % P;
        const size_t row = (size_t)min(max(sel_idx[j], 0), d.E - 1) * I + (size_t)t * 64 + lane;
        const uint8_t* const q[2] = {Ly.gq, Ly.uq};
        const uint32_t* const sz[2] = {Ly.gsz, Ly.usz};
        float o[2];
        unit_dot_bits<2>(Ly.gbits, q, sz, row, H, p * G, G, xs, xsum, o);
        float* part = ws.gu_part + (size_t)(j * tI + t) * P * 128;
        st_f(part + p * 128 + lane, o[0]);
        st_f(part + p * 128 + 64 + lane, o[1]);
        if (last_arrival(ws.gu_cnt + 16 * (j * tI + t), P)) {
          float gs = 0.0f, us = 0.0f;
          for (int p0 = 0; p0 < P; p0 += 32) {   // slices in order, 32 at a time (64 loads in flight)
            float b[64];
            const int np = min(32, P - p0);
            load_all(2 * np, b, [&](int i) { return ld_f(part + (p0 + (i >> 1)) * 128 + (i & 1) * 64 + lane); });
#pragma unroll
            for (int i = 0; i < 32; ++i)
              if (i < np) { gs += b[2 * i]; us += b[2 * i + 1]; }
          }
          const uint32_t hw = pair_with_next(f32_to_bf16_bits(silu_f32(gs) * us));
          if (!(lane & 1)) st_u(ws.h + ((size_t)j * I + t * 64 + lane) / 2, hw);
          if (lane == 0) __hip_atomic_store(ws.gu_cnt + 16 * (j * tI + t), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    grid_barrier(ws.bar, nb, ws.err);
    // ---- C: h into LDS (every block), down units (all wavefronts)
    for (int i0 = threadIdx.x; i0 < k * I / 2; i0 += 256 * 8) {
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = i0 + 256 * u < k * I / 2 ? ld_u(ws.h + i0 + 256 * u) : 0u;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + 256 * u < k * I / 2) reinterpret_cast<uint32_t*>(hs)[i0 + 256 * u] = v[u];
    }
    __syncthreads();
    for (int g = wave; g < k * tI; g += 4) {
      const float s = wave_sum(bf16_bits_to_f32(hs[g * 64 + lane]));
      if (lane == 0) hsum[g] = s;
    }
    __syncthreads();
    {
      const int PD = d.PD, G = tI / PD;
      const int nunits = tH * k * PD;
      for (int u = gw; u < nunits; u += nw) {
        const int t = u / (k * PD), j = (u / PD) % k, p = u % PD;
        const size_t row = (size_t)min(max(sel_idx[j], 0), d.E - 1) * H + (size_t)t * 64 + lane;
        const uint8_t* const q[1] = {Ly.dq};
        const uint32_t* const sz[1] = {Ly.dsz};
        float o[1];
        unit_dot_bits<1>(Ly.dbits, q, sz, row, I, p * G, G, hs + (size_t)j * I, hsum + j * tI, o);
        float* part = ws.y_part + (size_t)t * k * PD * 64;
        st_f(part + (j * PD + p) * 64 + lane, o[0]);
        if (last_arrival(ws.y_cnt + 16 * t, k * PD)) {
          // slots in ascending order, each the sum of its slices in order;
          // the partials (slot-major) are loaded 64 at a time
          float acc = 0.0f, yj = 0.0f;
          const int n = k * PD;
          for (int i0 = 0; i0 < n; i0 += 64) {
            float b[64];
            load_all(min(64, n - i0), b, [&](int i) { return ld_f(part + (i0 + i) * 64 + lane); });
#pragma unroll
            for (int i = 0; i < 64; ++i) {
              if (i0 + i < n) {
                yj += b[i];
                if ((i0 + i) % PD == PD - 1) {
                  acc = fmaf(sel_w[(i0 + i) / PD], yj, acc);
                  yj = 0.0f;
                }
              }
            }
          }
          // x rows t*64 .. t*64 + 63 as 32 pairs
          const uint32_t xw = ld_u(x2 + (t * 64 + (lane & ~1)) / 2);
          const float xo = bf16_bits_to_f32((lane & 1) ? (xw >> 16) : (xw & 0xFFFFu));
          const float yb = bf16_bits_to_f32(f32_to_bf16_bits(acc));
          const uint32_t nw2 = pair_with_next(f32_to_bf16_bits(xo + yb));
          if (!(lane & 1)) st_u(x2 + (t * 64 + lane) / 2, nw2);
          if (lane == 0) __hip_atomic_store(ws.y_cnt + 16 * t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    grid_barrier(ws.bar, nb, ws.err);
  }
}

int device_blocks(int* nb) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return set_error(MOEQ_ERR_HIP, "moe_stack: device query failed");
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, stack_decode_kernel, 256, 0) != hipSuccess || per < 1)
    return set_error(MOEQ_ERR_HIP, "moe_stack: occupancy query failed");
#ifndef MOEQ_STACK_BLOCKS_PER_CU
#define MOEQ_STACK_BLOCKS_PER_CU 2
#endif
  *nb = cus * (per < MOEQ_STACK_BLOCKS_PER_CU ? per : MOEQ_STACK_BLOCKS_PER_CU);
  return MOEQ_OK;
}

// K slices of a row of n groups: the largest power of two p dividing n with
// units * p <= waves and at least kMinGroups groups per slice (at least 1).
#ifndef MOEQ_STACK_MIN_GROUPS
#define MOEQ_STACK_MIN_GROUPS 1
#endif
constexpr int kMinGroups = MOEQ_STACK_MIN_GROUPS;
int slices(int n, int units, int waves) {
  int p = 1;
  while (n % (2 * p) == 0 && n / (2 * p) >= kMinGroups && units * 2 * p <= waves) p *= 2;
  return p;
}

struct StackLayout {
  size_t logits, gu_part, h, y_part, gu_cnt, y_cnt, bar, total;
  int P, PD, nb;
};

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

int stack_layout(const moe_layer_desc* L, StackLayout* o) {
  int rc = device_blocks(&o->nb);
  if (rc != MOEQ_OK) return rc;
  const int tI = L->I / 64, tH = L->H / 64, waves = 4 * o->nb;
  o->P = slices(tH, L->k * tI, waves);
  o->PD = slices(tI, tH * L->k, waves);
  size_t off = 0;
  o->logits = off;  off = up256(off + (size_t)L->E * 4);
  o->gu_part = off; off = up256(off + (size_t)L->k * tI * o->P * 128 * 4);
  o->h = off;       off = up256(off + (size_t)L->k * L->I * 2);
  o->y_part = off;  off = up256(off + (size_t)tH * L->k * o->PD * 64 * 4);
  o->gu_cnt = off;  off = up256(off + (size_t)L->k * tI * 64);   // counters 64 bytes apart
  o->y_cnt = off;   off = up256(off + (size_t)tH * 64);
  o->bar = off;     off = up256(off + 288 * 4);   // barrier words (see grid_barrier), then the error flag
  o->total = off;
  return MOEQ_OK;
}

int stack_dims_ok(const moe_layer_desc* L) {
  if (!L) return set_error(MOEQ_ERR_INVALID_ARG, "moe_stack: NULL layer");
  if (L->H <= 0 || L->I <= 0 || L->E <= 0 || L->k <= 0 || L->S < 0)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_stack: H=%d I=%d E=%d k=%d S=%d", L->H, L->I, L->E, L->k, L->S);
  if (L->S != 0) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_stack: shared experts (S=%d) not supported", L->S);
  if (L->H % 512 || L->H > kMaxH) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_stack: H=%d not a multiple of 512 up to %d", L->H, kMaxH);
  if (L->I % 64 || L->k * L->I > kMaxKI)
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_stack: I=%d not a multiple of 64 or k*I above %d", L->I, kMaxKI);
  if (L->k > kMaxK || L->k > L->E || L->E > 1024)
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_stack: k=%d E=%d (k <= 16, k <= E <= 1024)", L->k, L->E);
  return MOEQ_OK;
}

}  // namespace

extern "C" size_t moe_stack_table_bytes(int nlayers) {
  return nlayers > 0 ? sizeof(StackHeader) + (size_t)nlayers * sizeof(StackLayer) : 0;
}

extern "C" size_t moe_stack_workspace_bytes(const moe_layer_desc* L) {
  StackLayout o;
  if (stack_dims_ok(L) != MOEQ_OK || stack_layout(L, &o) != MOEQ_OK) return 0;
  return o.total;
}

extern "C" int moe_stack_table_write(const moe_layer_desc* layers, const uint16_t* const* w_router, int nlayers,
                                     void* table, size_t table_bytes) {
  if (!layers || !w_router || !table || nlayers <= 0)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_stack_table_write: NULL pointer or nlayers=%d", nlayers);
  if (table_bytes < moe_stack_table_bytes(nlayers))
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_stack_table_write: table of %zu bytes, %d layers need %zu", table_bytes,
                     nlayers, moe_stack_table_bytes(nlayers));
  if (!aligned16(table)) return set_error(MOEQ_ERR_MISALIGNED, "moe_stack_table_write: table must be 16-byte aligned");
  for (int l = 0; l < nlayers; ++l) {
    const moe_layer_desc* L = layers + l;
    int rc = validate_layer(L);
    if (rc == MOEQ_OK) rc = stack_dims_ok(L);
    if (rc == MOEQ_OK && (L->H != layers[0].H || L->I != layers[0].I || L->E != layers[0].E || L->k != layers[0].k))
      rc = set_error(MOEQ_ERR_INVALID_ARG, "moe_stack_table_write: layer %d has other dimensions than layer 0", l);
    if (rc == MOEQ_OK && L->gate.bits != L->up.bits)
      rc = set_error(MOEQ_ERR_UNSUPPORTED, "moe_stack_table_write: layer %d: gate and up must share a bit width", l);
    if (rc == MOEQ_OK && !w_router[l]) rc = set_error(MOEQ_ERR_INVALID_ARG, "moe_stack_table_write: router %d NULL", l);
    if (rc == MOEQ_OK && !aligned16(w_router[l]))
      rc = set_error(MOEQ_ERR_MISALIGNED, "moe_stack_table_write: router %d must be 16-byte aligned", l);
    if (rc != MOEQ_OK) return rc;
  }
  StackHeader hd{};
  hd.magic = kStackMagic;
  hd.nlayers = (uint32_t)nlayers;
  hd.H = layers[0].H;
  hd.I = layers[0].I;
  hd.E = layers[0].E;
  hd.k = layers[0].k;
  hipError_t he = hipMemcpy(table, &hd, sizeof(hd), hipMemcpyHostToDevice);
  if (he != hipSuccess) return set_error(MOEQ_ERR_HIP, "moe_stack_table_write: %s", hipGetErrorString(he));
  char* body = static_cast<char*>(table) + sizeof(StackHeader);
  // staged through a fixed host buffer, 64 layers at a time (no allocation)
  StackLayer buf[64];
  for (int l0 = 0; l0 < nlayers; l0 += 64) {
    const int n = nlayers - l0 < 64 ? nlayers - l0 : 64;
    for (int i = 0; i < n; ++i) {
      const moe_layer_desc* L = layers + l0 + i;
      buf[i] = StackLayer{L->gate.q, L->gate.sz, L->up.q, L->up.sz, L->down.q, L->down.sz, w_router[l0 + i],
                          L->gate.bits, L->down.bits};
    }
    const hipError_t e = hipMemcpy(body + (size_t)l0 * sizeof(StackLayer), buf,
                                   (size_t)n * sizeof(StackLayer), hipMemcpyHostToDevice);
    if (e != hipSuccess) return set_error(MOEQ_ERR_HIP, "moe_stack_table_write: %s", hipGetErrorString(e));
  }
  return MOEQ_OK;
}

extern "C" int moe_stack_decode(const moe_layer_desc* dims, const void* table, size_t table_bytes, int nlayers,
                                float eps, uint16_t* x, void* ws, size_t ws_bytes, hipStream_t stream) {
  int rc = stack_dims_ok(dims);
  if (rc != MOEQ_OK) return rc;
  if (!table || !x || nlayers < 0) return set_error(MOEQ_ERR_INVALID_ARG, "moe_stack_decode: NULL pointer or nlayers=%d", nlayers);
  if (table_bytes < moe_stack_table_bytes(nlayers > 0 ? nlayers : 1))
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_stack_decode: table of %zu bytes cannot hold %d layers", table_bytes, nlayers);
  if (!(eps >= 0.0f)) return set_error(MOEQ_ERR_INVALID_ARG, "moe_stack_decode: eps=%g", (double)eps);
  if (!aligned16(x) || !aligned16(table)) return set_error(MOEQ_ERR_MISALIGNED, "moe_stack_decode: x and table must be 16-byte aligned");
  if (nlayers == 0) return MOEQ_OK;
  StackLayout o;
  if ((rc = stack_layout(dims, &o)) != MOEQ_OK) return rc;
  if (!ws || ws_bytes < o.total)
    return set_error(MOEQ_ERR_WORKSPACE, "moe_stack_decode: workspace of %zu bytes, need %zu", ws_bytes, o.total);
  char* w = static_cast<char*>(ws);
  StackWs sw{reinterpret_cast<float*>(w + o.logits), reinterpret_cast<float*>(w + o.gu_part),
             reinterpret_cast<uint32_t*>(w + o.h), reinterpret_cast<float*>(w + o.y_part),
             reinterpret_cast<int*>(w + o.gu_cnt), reinterpret_cast<int*>(w + o.y_cnt),
             reinterpret_cast<unsigned*>(w + o.bar), reinterpret_cast<int*>(w + o.bar) + 280};
  StackDims sd{dims->H, dims->I, dims->E, dims->k, nlayers, o.P, o.PD, eps};
  const StackHeader* tp = static_cast<const StackHeader*>(table);
  uint32_t* x2 = reinterpret_cast<uint32_t*>(x);
  void* args[] = {&tp, &sd, &sw, &x2};
  const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(stack_decode_kernel), dim3(o.nb),
                                                  dim3(256), args, 0, stream);
  if (e != hipSuccess) return set_error(MOEQ_ERR_HIP, "moe_stack_decode: cooperative launch failed: %s", hipGetErrorString(e));
  return check_launch("moe_stack_decode");
}

extern "C" int moe_stack_read_status(void* ws, size_t ws_bytes, const moe_layer_desc* dims, int* err,
                                     hipStream_t stream) {
  if (!ws || !err) return set_error(MOEQ_ERR_INVALID_ARG, "moe_stack_read_status: NULL workspace or output");
  int rc = stack_dims_ok(dims);
  if (rc != MOEQ_OK) return rc;
  StackLayout o;
  if ((rc = stack_layout(dims, &o)) != MOEQ_OK) return rc;
  if (ws_bytes < o.total)
    return set_error(MOEQ_ERR_WORKSPACE, "moe_stack_read_status: workspace of %zu bytes, need %zu", ws_bytes, o.total);
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return set_error(MOEQ_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
  char* w = static_cast<char*>(ws);
  int v = 0;
  e = hipMemcpy(&v, w + o.bar + 280 * sizeof(int), sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return set_error(MOEQ_ERR_HIP, "hipMemcpy: %s", hipGetErrorString(e));
  if (v != 0) {
    // a wait that gave up leaves counts behind: zero every control word
    // (the counters, the barrier words and the error word) for the next call
    e = hipMemset(w + o.gu_cnt, 0, o.total - o.gu_cnt);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return set_error(MOEQ_ERR_HIP, "hipMemset: %s", hipGetErrorString(e));
  }
  *err = v;
  return MOEQ_OK;
}
