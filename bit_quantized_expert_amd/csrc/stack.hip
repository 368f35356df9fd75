// Stacked decode in one launch: a batch-1 token through L MoE blocks
// (RMSNorm -> router -> top-k -> gate/up -> down -> weighted combine ->
// residual), the blocks' weights streamed by every CU of the chip.  The
// pages' decode lever is exactly this: small per-step kernel launches left
// most of the bandwidth unused, a persistent per-layer MoE megakernel
// recovered it (Raon-1-mini, optimisation table and result paragraph).
//
// A layer, for the residual stream x (bf16 [H]):
//   A  every workgroup: n = RMSNorm(x) into LDS (and its 64-group sums),
//      from x held in registers; router rows over the first wavefronts:
//      logits[e] = n . Wr[e]
//   B  every workgroup: top-k of the logits into LDS.  Gate/up: workgroup u
//      computes eight whole rows (all of K) of one slot's gate and up
//      projections, lane l taking row l % 8 and 64-groups l / 8 + 8 w + 32 i
//      (w: its wavefront); the 32 group lanes of a row are added in the
//      wavefront (butterfly) and the four wavefronts in LDS, in a fixed
//      order, and h = bf16(silu(g) u) of the eight rows goes out
//   C  down: workgroup t takes eight rows of x, all k slots and all of I
//      (lane l: row l % 8, (slot, 64-group) items l / 8 + 8 w + 32 i), every
//      item weighted by its slot's routing weight, adds them the same way
//      and writes x = bf16(x + bf16(sum)).  Its weights are loaded right
//      after the top-k, before its gate/up rows, and are in registers when h
//      arrives.
// Eight rows of one 64-row tile hold, chunk after chunk, whole 128-byte
// lines (4- and 8-bit), so these units read only whole lines, and the only
// values that cross workgroups are x, the logits and h: three hand-offs a
// layer.  The router, the gate/up units and the down units sit on different
// workgroups where the grid allows, so that the router's workgroups load
// the next layer's router rows while the down units run.
// Logits, h and x are written once per XCD (eight copies) and each
// workgroup reads the copy of its XCD, so that the pollers of one value
// spread over eight times as many lines.
// The dot products are the decode GEMV's (format.h): codes become bf16
// (128 + q, or q at 8 bits) pairs, v_dot2_f32_bf16 with the activations'
// pairs (read from LDS), and the group's scale and zero enter once per group
// in fp32.
//
// No barrier and no counter: every value one wavefront hands to another
// (logits, partial sums, h, x between layers) is stored as a 64-bit word,
// the 32-bit value beside a 32-bit tag (call number * 1024 + layer), with a
// device-scope atomic store, which lands whole and is coherent across the
// XCDs' separate L2 caches.  A consumer loads the words it needs with
// device-scope atomic loads and loads again those whose tag is older than
// the one it waits for.  A producer thus never waits for its stores to
// complete, and a hand-over costs one store and one load.  A word with a
// newer tag than awaited is taken as well: only a wavefront whose result no
// one uses can fall that far behind (a value of layer l + 1 exists only
// after every down unit of layer l has finished, and each of those has read
// every h word and needed every gate/up unit, which read every logit).  A small kernel launched before
// each call advances the call number.  The router rows are loaded before x
// arrives.
//
// The table starts with a 64-byte header (layer count and H, I, E, k) that
// every block checks against the launch's dimensions before it touches a
// layer; on a mismatch every block leaves at once and the workspace's error
// word gets bit 2.  A wait that gives up (after 2^18 polls, a fraction of a
// second) sets bit 1 and goes on with what it read, so that every wavefront
// reaches the end of the kernel.  The error word is sticky until
// moe_stack_read_status reads it.
#include "decode_impl.h"
#include "rows8.h"

#include <type_traits>

using namespace moeq;
using decode_detail::load_chunk_g;

namespace {

constexpr int kMaxH = 8192;      // LDS: n, bf16
constexpr int kMaxKI = 16384;    // LDS: h of every slot, bf16 (k * I)
constexpr int kMaxK = 16;
constexpr int kMaxLayers = 1024; // tags: call * 1024 + layer
constexpr unsigned kSpinLimit = 1u << 18;
// Copies of the values every workgroup reads (logits, h, x): one per XCD, so
// that the pollers of one value spread over that many lines.
#ifndef MOEQ_STACK_REPLICAS
#define MOEQ_STACK_REPLICAS 8
#endif
constexpr int kRep = MOEQ_STACK_REPLICAS;
#ifndef MOEQ_STACK_GENERIC_ONLY
#define MOEQ_STACK_GENERIC_ONLY 0
#endif
#ifndef MOEQ_STACK_SLEEP
#define MOEQ_STACK_SLEEP 1
#endif

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
  float eps;
};

// Tagged words: value in the low half, tag in the high half.
struct StackWs {
  uint64_t* logits;    // [kRep][E] fp32
  uint64_t* h;         // [kRep][k][I/2] bf16 pairs
  uint64_t* x;         // [kRep][H/2] bf16 pairs: x between layers
  uint32_t* epoch;     // call number
  int* err;            // bit 1: a wait gave up; bit 2: table mismatch
  uint64_t* tl;        // event times per (layer, wavefront), or null
};

// The hand-off accesses go through global-address-space pointers, so that
// they compile to global (not flat) loads and stores: flat accesses also
// count as LDS accesses and would make every LDS wait wait for them.
typedef __attribute__((address_space(1))) uint32_t gu32;
typedef __attribute__((address_space(1))) uint64_t gu64;
// 16 bytes through a global pointer as a uint4
MOEQ_DEV uint4 ld_g16(const void* p) {
  typedef const __attribute__((address_space(1))) moeq_u32x4* g4;
  const moeq_u32x4 v = *(g4)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
MOEQ_DEV uint32_t ld_u(const uint32_t* p) {
  return __hip_atomic_load((gu32*)(const_cast<uint32_t*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOEQ_DEV void st_u(uint32_t* p, uint32_t v) {
  __hip_atomic_store((gu32*)(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOEQ_DEV uint64_t ld_t(const uint64_t* p) {
  return __hip_atomic_load((gu64*)(const_cast<uint64_t*>(p)), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A workspace base pointer as a value the compiler takes as new in every
// layer, held in scalar registers: addresses built from it stay scalar base
// plus lane offset and are not computed ahead for all layers (which would
// hold a vector address per load for the whole kernel).
template <class T>
MOEQ_DEV T* fresh_base(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  // each half through uint32_t: readfirstlane returns int, which would
  // sign-extend a low half with bit 31 set into the high half
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  uint64_t a = ((uint64_t)hi << 32) | lo;
  asm volatile("" : "+s"(a));
  return reinterpret_cast<T*>(a);
}
MOEQ_DEV void st_t(uint64_t* p, uint32_t v, uint32_t tag) {
  __hip_atomic_store((gu64*)(p), ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOEQ_DEV bool fresh(uint64_t w, uint32_t tag) { return (int32_t)((uint32_t)(w >> 32) - tag) >= 0; }
MOEQ_DEV float val_f(uint64_t w) { return __uint_as_float((uint32_t)w); }

// Loads word addr(i) for i < n (n <= M, may differ per lane) into b, all in
// flight together, then loads again every word with a tag older than `tag`
// until none is left (the whole wavefront decides together).
template <int M, class Addr>
MOEQ_DEV void poll(int n, uint64_t (&b)[M], Addr&& addr, uint32_t tag, int* err) {
  // (every element is assigned: a conditionally assigned one would let the
  // compiler carry an older value across loops)
#pragma unroll
  for (int i = 0; i < M; ++i) b[i] = i < n ? ld_t(addr(i)) : 0;
  for (unsigned spins = 0;; ++spins) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (i < n && !fresh(b[i], tag)) ok = false;
    if (__all(ok)) return;
    // give up after kSpinLimit polls, or after 1024 once another wait has
    // given up (so that a failed call ends in well under a second)
    if (spins == kSpinLimit || ((spins & 1023) == 1023 && (ld_u(reinterpret_cast<const uint32_t*>(err)) & 1))) {
      if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    __builtin_amdgcn_s_sleep(MOEQ_STACK_SLEEP);
#pragma unroll
    for (int i = 0; i < M; ++i)
      if (i < n && !fresh(b[i], tag)) b[i] = ld_t(addr(i));
  }
}

MOEQ_DEV void event(const StackWs& ws, int l, int gw, int nw, int i) {
  if (ws.tl && (threadIdx.x & 63) == 0) ws.tl[((size_t)l * nw + gw) * 16 + i] = wall_clock64();
}


// Top-k of E logits (first wavefront of the block) into LDS: select_token's
// choices and weights.
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

// bf16 of this lane and of the next one as one word (for even lanes)
MOEQ_DEV uint32_t pair_with_next(uint32_t b) { return b | (__shfl_down(b, 1) << 16); }

__global__ __launch_bounds__(256) void stack_epoch_kernel(uint32_t* epoch) {
  if (threadIdx.x == 0) __hip_atomic_fetch_add(epoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// CH, CI, CK, CE: H, I, k, E fixed at compile time (0: taken from d at run
// time); the stacked workload's shape has an instantiation of its own, in
// which the unit and item indices need no run-time divisions.
template <int CH, int CI, int CK, int CE>
__global__ __launch_bounds__(256, 2) void stack_decode_kernel(const StackHeader* hdr, StackDims d, StackWs ws0,
                                                              uint32_t* x2_0) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kMaxH];
  __shared__ float xsum[kMaxH / 64];
  __shared__ __attribute__((aligned(16))) uint16_t hs[kMaxKI];
  __shared__ float hsum[kMaxKI / 64];
  __shared__ __attribute__((aligned(16))) uint16_t xr[kMaxH];   // x itself (the residual)
  __shared__ float lg[1024];
  __shared__ int sel_idx[kMaxK];
  __shared__ float sel_w[kMaxK];
  __shared__ float red[4];
  __shared__ float rsum[64];
  {
    // every block reads the same header, so all leave or none does
    const StackHeader h0 = *hdr;
    if (h0.magic != kStackMagic || (int)h0.nlayers < d.L || h0.H != d.H || h0.I != d.I || h0.E != d.E || h0.k != d.k) {
      if (blockIdx.x == 0 && threadIdx.x == 0) __hip_atomic_fetch_or(ws0.err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
  }
  const StackLayer* table = reinterpret_cast<const StackLayer*>(hdr + 1);
  const uint32_t base = ld_u(ws0.epoch) << 10;
  for (int l = 0; l < d.L; ++l) {
    // the dimensions as values the compiler takes as new in every layer, so
    // that what derives from them is computed where it is used rather than
    // ahead of the loop for all layers (where it would occupy registers)
    int H = CH ? CH : d.H, I = CI ? CI : d.I, k = CK ? CK : d.k, E = CE ? CE : d.E, wave = (int)threadIdx.x >> 6;
    if constexpr (!CH) asm volatile("" : "+s"(H));
    if constexpr (!CI) asm volatile("" : "+s"(I));
    if constexpr (!CK) asm volatile("" : "+s"(k));
    if constexpr (!CE) asm volatile("" : "+s"(E));
    wave = uniform(wave);
    const int lane = threadIdx.x & 63;
    const int gw = (int)blockIdx.x * 4 + wave, nw = (int)gridDim.x * 4;
    const StackLayer Ly = table[l];
    const uint32_t tag = base + (uint32_t)l;
    const int rep = (int)blockIdx.x % kRep;   // the copy this workgroup reads
    StackWs ws = ws0;
    ws.logits = fresh_base(ws0.logits);
    ws.h = fresh_base(ws0.h);
    ws.x = fresh_base(ws0.x);
    uint32_t* x2 = fresh_base(x2_0);
    // ---- A: RMSNorm (every block), router rows.  The first router row's
    // weights (they do not depend on x) are loaded before x.
    constexpr int kRouterChunks = 4;   // H <= 2048 fully; the rest of longer rows after x
    uint4 wfirst[kRouterChunks];
#pragma unroll
    for (int c = 0; c < kRouterChunks; ++c) wfirst[c] = make_uint4(0, 0, 0, 0);
    if (gw < E) {
      const uint16_t* wrow = Ly.wr + (size_t)gw * H;
#pragma unroll
      for (int c = 0; c < kRouterChunks; ++c)
        if (c * 512 < H) wfirst[c] = ld_g16(wrow + c * 512 + lane * 8);
    }
    // x as H/2 bf16 pairs, H/512 of them per thread (kept in registers), 4
    // at a time
    const int nx = H / 512;
    uint32_t xv[kMaxH / 512];
    {
      const uint64_t* xrep = ws.x + (size_t)rep * (H / 2);
      float ss = 0.0f;
#pragma unroll
      for (int u0 = 0; u0 < kMaxH / 512; u0 += 4) {
        if (u0 < nx) {
          uint64_t xb[4];
          const int nu = min(4, nx - u0);
          if (l == 0) {
#pragma unroll
            for (int u = 0; u < 4; ++u) xb[u] = u < nu ? ld_u(x2 + threadIdx.x + 256 * (u0 + u)) : 0;
          } else {
            poll(nu, xb, [&](int u) { return xrep + threadIdx.x + 256 * (u0 + u); }, tag - 1, ws.err);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const uint32_t v = (uint32_t)xb[u];
            xv[u0 + u] = v;
            if (u < nu) {
              const float a = bf16_bits_to_f32(v & 0xFFFFu), b = bf16_bits_to_f32(v >> 16);
              reinterpret_cast<uint32_t*>(xr)[threadIdx.x + 256 * (u0 + u)] = v;
              ss = fmaf(a, a, ss);
              ss = fmaf(b, b, ss);
            }
          }
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) xv[u0 + u] = 0;
        }
      }
      ss = wave_sum(ss);
      if (lane == 0) red[wave] = ss;
    }
    event(ws, l, gw, nw, 0);
    __syncthreads();
    {
      // n = bf16(x r) from the registers; the 32 pairs of a 64-group sit in
      // one half of a wavefront (pair index tid + 256 u), so its sum is a
      // 32-lane sum
      const float tot = (red[0] + red[1]) + (red[2] + red[3]);
      const float r = 1.0f / sqrtf(tot / (float)H + d.eps);
#pragma unroll
      for (int u = 0; u < kMaxH / 512; ++u) {
        if (u < nx) {
          const uint32_t na = f32_to_bf16_bits(bf16_bits_to_f32(xv[u] & 0xFFFFu) * r);
          const uint32_t nb2 = f32_to_bf16_bits(bf16_bits_to_f32(xv[u] >> 16) * r);
          reinterpret_cast<uint32_t*>(xs)[threadIdx.x + 256 * u] = na | (nb2 << 16);
          const float gsum = group_sum(bf16_bits_to_f32(na) + bf16_bits_to_f32(nb2), 32);
          if ((lane & 31) == 0) xsum[2 * wave + 8 * u + (lane >> 5)] = gsum;
        }
      }
    }
    __syncthreads();
    event(ws, l, gw, nw, 7);
    for (int e = gw; e < E; e += nw) {
      const uint16_t* wrow = Ly.wr + (size_t)e * H;
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < kRouterChunks; ++c) {
        if (c * 512 < H) {
          const uint4 wv = e == gw ? wfirst[c] : ld_g16(wrow + c * 512 + lane * 8);
          const uint4 nv = *reinterpret_cast<const uint4*>(xs + c * 512 + lane * 8);
          acc = dot2_bf16(wv.x, nv.x, acc);
          acc = dot2_bf16(wv.y, nv.y, acc);
          acc = dot2_bf16(wv.z, nv.z, acc);
          acc = dot2_bf16(wv.w, nv.w, acc);
        }
      }
      for (int c = kRouterChunks * 512 + lane * 8; c < H; c += 512) {
        const uint4 wv = ld_g16(wrow + c);
        const uint4 nv = *reinterpret_cast<const uint4*>(xs + c);
        acc = dot2_bf16(wv.x, nv.x, acc);
        acc = dot2_bf16(wv.y, nv.y, acc);
        acc = dot2_bf16(wv.z, nv.z, acc);
        acc = dot2_bf16(wv.w, nv.w, acc);
      }
      acc = wave_sum(acc);
      if (lane < kRep) st_t(ws.logits + (size_t)lane * E + e, __float_as_uint(acc), tag);
    }
    event(ws, l, gw, nw, 8);
    // ---- B: top-k (every workgroup)
    {
      uint64_t lb[4];   // E <= 1024: at most 4 logits per thread
      const int nl = (E - (int)threadIdx.x + 255) / 256;
      const uint64_t* lr = ws.logits + (size_t)rep * E;
      poll(nl, lb, [&](int i) { return lr + threadIdx.x + 256 * i; }, tag, ws.err);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < nl) lg[threadIdx.x + 256 * i] = val_f(lb[i]);
    }
    __syncthreads();
    event(ws, l, gw, nw, 1);
    if (wave == 0) select_any(lg, E, k, sel_idx, sel_w);
    __syncthreads();
    event(ws, l, gw, nw, 9);
    // Units: gate/up unit u (slot u / (I/8), rows 8 (u % (I/8)) ..) over all
    // workgroups; down unit t (rows 8 t .. 8 t + 7 of x) over the last
    // workgroups, so that with more workgroups than down units the router's
    // workgroups (the first ones) have none; both in xcd_unit's order.
    const int nb = (int)gridDim.x;
    const int r8 = lane & 7, ql = (lane >> 3) + 8 * wave;   // row of the eight; group lane 0 .. 31
    const int nG = H / 64, nGL = (nG + 31) / 32;            // groups of a gate/up row; per lane
    const int nGI = I / 64, nIt = k * nGI, nIL = (nIt + 31) / 32;   // down items of a row; per lane
    const int nU = k * (I / 8), nD = H / 8;
    const int nDw = min(nD, nb), D0 = nb - nDw;   // workgroups D0 .. nb - 1 take the down units
    const int t0 = (int)blockIdx.x >= D0 ? xcd_unit((int)blockIdx.x - D0, nDw) : nD;   // first down unit
    const bool last = l + 1 == d.L;
    auto expert_of = [&](int j) { return (size_t)min(max(sel_idx[j], 0), E - 1); };
    auto experts = [&](auto gb, auto db) {
      constexpr int GB = decltype(gb)::value, DB = decltype(db)::value;
      // the first down unit's first two items (this lane's)
      Grp dn[2];
      auto load_dn = [&]() {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int idx = ql + 32 * i;
          const bool on = t0 < nD && i < nIL && idx < nIt;
          const int j = on ? idx / nGI : 0, g = on ? idx % nGI : 0;
          grp_load<DB>(dn[i], Ly.dq, Ly.dsz, expert_of(j) * H + (size_t)t0 * 8 + r8, I, g, on);
        }
      };
      // gate/up unit u
      auto gu_unit = [&](int u) {
        const int j = u / (I / 8), r0 = (u % (I / 8)) * 8;
        const size_t row = expert_of(j) * I + r0 + r8;
        float ag = 0.0f, au = 0.0f;
        Grp G[2][2];
        auto load = [&](int i0) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int g = ql + 32 * (i0 + i);
            const bool on = i0 + i < nGL && g < nG;
            grp_load<GB>(G[i][0], Ly.gq, Ly.gsz, row, H, g, on);
            grp_load<GB>(G[i][1], Ly.uq, Ly.usz, row, H, g, on);
          }
        };
        auto dot = [&](int i0) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int g = ql + 32 * (i0 + i);
            if (i0 + i < nGL && g < nG) {
              ag += grp_dot<GB>(G[i][0], xs + g * 64, xsum[g]);
              au += grp_dot<GB>(G[i][1], xs + g * 64, xsum[g]);
            }
          }
        };
        load(0);
        dot(0);
        for (int i0 = 2; i0 < nGL; i0 += 2) {
          load(i0);
          dot(i0);
        }
        event(ws, l, gw, nw, 12);
        ag = sum_stride8(ag);
        au = sum_stride8(au);
        __syncthreads();   // rsum is free
        if (lane < 8) {
          rsum[wave * 16 + lane] = ag;
          rsum[wave * 16 + 8 + lane] = au;
        }
        __syncthreads();
        if (wave == 0) {
          const float gs = ((rsum[r8] + rsum[16 + r8]) + rsum[32 + r8]) + rsum[48 + r8];
          const float us = ((rsum[8 + r8] + rsum[24 + r8]) + rsum[40 + r8]) + rsum[56 + r8];
          const uint32_t hw = pair_with_next(f32_to_bf16_bits(silu_f32(gs) * us));
          if (lane < 8 && !(lane & 1))
#pragma unroll
            for (int c = 0; c < kRep; ++c) st_t(ws.h + (size_t)c * (k * I / 2) + ((size_t)j * I + r0 + lane) / 2, hw, tag);
        }
      };
      for (int u = xcd_unit((int)blockIdx.x, nb); u < nU; u += nb) gu_unit(u);
      // the down weights after the gate/up rows: they then arrive during the
      // h hand-off instead of sharing the bandwidth with the gate/up rows,
      // which h waits for (issued before the gate/up rows or before their
      // reduction, they cost 4 % a token)
      event(ws, l, gw, nw, 3);
      load_dn();
      event(ws, l, gw, nw, 2);
      if (t0 >= nD) return;
      // ---- C: h of every slot from this XCD's copy into LDS, with its
      // 64-group sums (a group is 32 words, held by 32 consecutive threads)
      {
        const uint64_t* hrep = ws.h + (size_t)rep * (k * I / 2);
        uint32_t* hs32 = reinterpret_cast<uint32_t*>(hs);
        const int nhw = k * I / 2;
        for (int w0 = 0; w0 < nhw; w0 += 256 * 8) {
          uint64_t hb[8];
          const int rem = nhw - w0 - (int)threadIdx.x;
          const int nh = rem <= 0 ? 0 : min(8, (rem + 255) / 256);
          poll(nh, hb, [&](int i) { return hrep + w0 + threadIdx.x + 256 * i; }, tag, ws.err);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t v = (uint32_t)hb[i];
            const int wi = w0 + (int)threadIdx.x + 256 * i;
            if (i < nh) hs32[wi] = v;
            const float gsum = group_sum(i < nh ? bf16_bits_to_f32(v & 0xFFFFu) + bf16_bits_to_f32(v >> 16) : 0.0f, 32);
            if (i < nh && (lane & 31) == 0) hsum[wi / 32] = gsum;
          }
        }
      }
      __syncthreads();
      event(ws, l, gw, nw, 4);
      // down unit t; PRE: the items of its first two group lanes are in dn
      auto down_unit = [&](int t, auto pre) {
        auto load = [&](int i0) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int idx = ql + 32 * (i0 + i);
            const bool on = i0 + i < nIL && idx < nIt;
            const int j = on ? idx / nGI : 0, g = on ? idx % nGI : 0;
            grp_load<DB>(dn[i], Ly.dq, Ly.dsz, expert_of(j) * H + (size_t)t * 8 + r8, I, g, on);
          }
        };
        float acc = 0.0f;
        auto dot = [&](int i0) {
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int idx = ql + 32 * (i0 + i);
            if (i0 + i < nIL && idx < nIt) {
              const int j = idx / nGI, g = idx % nGI;
              acc = fmaf(sel_w[j], grp_dot<DB>(dn[i], hs + j * I + g * 64, hsum[j * nGI + g]), acc);
            }
          }
        };
        if constexpr (!decltype(pre)::value) load(0);
        dot(0);
        for (int i0 = 2; i0 < nIL; i0 += 2) {
          load(i0);
          dot(i0);
        }
        event(ws, l, gw, nw, 10);
        acc = sum_stride8(acc);
        __syncthreads();   // rsum is free
        if (lane < 8) rsum[wave * 8 + lane] = acc;
        __syncthreads();
        event(ws, l, gw, nw, 11);
        if (wave == 0) {
          const float y = ((rsum[r8] + rsum[8 + r8]) + rsum[16 + r8]) + rsum[24 + r8];
          const float xo = bf16_bits_to_f32(xr[t * 8 + r8]);
          const float yb = bf16_bits_to_f32(f32_to_bf16_bits(y));
          const uint32_t nx2 = pair_with_next(f32_to_bf16_bits(xo + yb));
          if (lane < 8 && !(lane & 1)) {
            if (last) {
              st_u(x2 + (t * 8 + lane) / 2, nx2);
            } else {
#pragma unroll
              for (int c = 0; c < kRep; ++c) st_t(ws.x + (size_t)c * (H / 2) + (t * 8 + lane) / 2, nx2, tag);
            }
          }
        }
      };
      down_unit(t0, std::true_type{});
      for (int t = t0 + nDw; t < nD; t += nDw) down_unit(t, std::false_type{});
      event(ws, l, gw, nw, 5);
    };
    auto by_down = [&](auto gb) {
      switch (Ly.dbits) {
        case 4: experts(gb, std::integral_constant<int, 4>{}); break;
        case 6: experts(gb, std::integral_constant<int, 6>{}); break;
        default: experts(gb, std::integral_constant<int, 8>{}); break;
      }
    };
    switch (Ly.gbits) {
      case 4: by_down(std::integral_constant<int, 4>{}); break;
      case 6: by_down(std::integral_constant<int, 6>{}); break;
      default: by_down(std::integral_constant<int, 8>{}); break;
    }
    __syncthreads();
    event(ws, l, gw, nw, 6);
  }
}

using StackKernel = void (*)(const StackHeader*, StackDims, StackWs, uint32_t*);

StackKernel stack_kernel_for(const moe_layer_desc* L) {
#if !MOEQ_STACK_GENERIC_ONLY
  if (L->H == 2048 && L->I == 512 && L->k == 8 && L->E == 128) return stack_decode_kernel<2048, 512, 8, 128>;
#endif
  return stack_decode_kernel<0, 0, 0, 0>;
}

int device_blocks(StackKernel kern, int* nb) {
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return set_error(MOEQ_ERR_HIP, "moe_stack: device query failed");
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void*>(kern), 256, 0) != hipSuccess || per < 1)
    return set_error(MOEQ_ERR_HIP, "moe_stack: occupancy query failed");
#ifndef MOEQ_STACK_BLOCKS_PER_CU
#define MOEQ_STACK_BLOCKS_PER_CU 2
#endif
  *nb = cus * (per < MOEQ_STACK_BLOCKS_PER_CU ? per : MOEQ_STACK_BLOCKS_PER_CU);
  return MOEQ_OK;
}

struct StackLayout {
  size_t logits, h, x, ctl, tl, total;
  int nb;
};

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

// With MOEQ_STACK_TIMELINE defined, the workspace ends with the event times
// of every (layer, wavefront) of a call of up to that many layers.
#ifdef MOEQ_STACK_TIMELINE
constexpr int kTimelineLayers = MOEQ_STACK_TIMELINE;
#else
constexpr int kTimelineLayers = 0;
#endif

int stack_layout(const moe_layer_desc* L, StackLayout* o) {
  int rc = device_blocks(stack_kernel_for(L), &o->nb);
  if (rc != MOEQ_OK) return rc;
  const int waves = 4 * o->nb;
  size_t off = 0;
  o->logits = off;  off = up256(off + (size_t)kRep * L->E * 8);
  o->h = off;       off = up256(off + (size_t)kRep * L->k * L->I / 2 * 8);
  o->x = off;       off = up256(off + (size_t)kRep * L->H / 2 * 8);
  o->ctl = off;     off = up256(off + 256);   // call number, error word
  o->tl = off;      off = up256(off + (size_t)kTimelineLayers * waves * 16 * 8);
  o->total = off;
  return MOEQ_OK;
}

int stack_dims_ok(const moe_layer_desc* L) {
  if (!L) return set_error(MOEQ_ERR_INVALID_ARG, "moe_stack: NULL layer");
  if (L->H <= 0 || L->I <= 0 || L->E <= 0 || L->k <= 0 || L->S < 0)
    return set_error(MOEQ_ERR_INVALID_ARG, "moe_stack: H=%d I=%d E=%d k=%d S=%d", L->H, L->I, L->E, L->k, L->S);
  if (L->S != 0) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_stack: shared experts (S=%d) not supported", L->S);
  if (L->H % 512 || L->H > kMaxH) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_stack: H=%d not a multiple of 512 up to %d", L->H, kMaxH);
  if (L->I % 64 || (long)L->k * L->I > kMaxKI)
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_stack: I=%d not a multiple of 64, or k*I=%ld above %d", L->I,
                     (long)L->k * L->I, kMaxKI);
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
  if (nlayers > kMaxLayers) return set_error(MOEQ_ERR_UNSUPPORTED, "moe_stack_decode: nlayers=%d above %d", nlayers, kMaxLayers);
  if (nlayers == 0) return MOEQ_OK;
  StackLayout o;
  if ((rc = stack_layout(dims, &o)) != MOEQ_OK) return rc;
  if (!ws || ws_bytes < o.total)
    return set_error(MOEQ_ERR_WORKSPACE, "moe_stack_decode: workspace of %zu bytes, need %zu", ws_bytes, o.total);
  char* w = static_cast<char*>(ws);
  uint64_t* tl = nlayers <= kTimelineLayers ? reinterpret_cast<uint64_t*>(w + o.tl) : nullptr;
  StackWs sw{reinterpret_cast<uint64_t*>(w + o.logits), reinterpret_cast<uint64_t*>(w + o.h),
             reinterpret_cast<uint64_t*>(w + o.x), reinterpret_cast<uint32_t*>(w + o.ctl),
             reinterpret_cast<int*>(w + o.ctl) + 16, tl};
  StackDims sd{dims->H, dims->I, dims->E, dims->k, nlayers, eps};
  stack_epoch_kernel<<<1, 64, 0, stream>>>(sw.epoch);
  if ((rc = check_launch("moe_stack_decode (call number)")) != MOEQ_OK) return rc;
  const StackHeader* tp = static_cast<const StackHeader*>(table);
  uint32_t* x2 = reinterpret_cast<uint32_t*>(x);
  void* args[] = {&tp, &sd, &sw, &x2};
  const hipError_t e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(stack_kernel_for(dims)), dim3(o.nb),
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
  e = hipMemcpy(&v, w + o.ctl + 16 * sizeof(int), sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return set_error(MOEQ_ERR_HIP, "hipMemcpy: %s", hipGetErrorString(e));
  if (v != 0) {
    // the word is sticky until read; the tagged words need no reset (a
    // later call waits for its own tags)
    const int zero = 0;
    e = hipMemcpy(w + o.ctl + 16 * sizeof(int), &zero, sizeof(int), hipMemcpyHostToDevice);
    if (e != hipSuccess) return set_error(MOEQ_ERR_HIP, "hipMemcpy: %s", hipGetErrorString(e));
  }
  *err = v;
  return MOEQ_OK;
}
