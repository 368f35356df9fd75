// Prefill path: grouped GEMMs over expert-sorted tokens on the bf16 matrix
// cores, with the expert weights dequantised in registers on the fly.
//
//   gate/up kernel: per (expert, 128-token tile, 128 features of I), the
//     gathered token rows of x times the gate and up rows of that expert,
//     epilogue h = silu(g) * u rounded to bf16, stored in expert-sorted order.
//   down kernel: per (expert, 128-token tile, 256 features of H), the h rows
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

// ---------------------------------------------------------------------------
// Expert GEMMs: C[tokens][features] = A (token rows, bf16, staged in LDS) x
// W^T (quantised weight rows).  Each wavefront owns whole columns (features)
// of the block tile: its lanes load those weight rows' codes straight into
// registers, dequantise them to bf16 there and feed them to the matrix cores
// as the B operand, so the weights never pass through LDS and no two
// wavefronts dequantise the same weights.  The token rows (A) go through a
// double-buffered LDS tile shared by the block's four wavefronts, one
// barrier per K-slice of 64 (= one quantisation group).  The codes of a
// slice are loaded two slices ahead, the token rows one slice ahead.
//
// The contraction does not depend on the order of k, so each MFMA step
// takes the 16 k-values whose codes a lane pair holds (step_k), and A is
// read to match: lane half h at step st supplies k = 32 (st / 2) + 16 h +
// 8 (st % 2) .. + 7 of the slice.
//   4-bit: a slice is 2 chunks of 32 codes; lane half h loads bytes 8h ..
//          8h + 7 of each (codes 16h .. 16h + 15 of the chunk).
//   6-, 8-bit: a slice is 4 chunks of 16 codes; lane half h loads chunks h
//          and h + 2 whole.
// ---------------------------------------------------------------------------

MOEQ_DEV int step_k(int st, int h) { return 32 * (st >> 1) + 16 * h + 8 * (st & 1); }

// One weight row (B column) of one expert matrix, as this lane reads it:
// the uniform base of the expert's rows plus 32-bit lane offsets, so the
// loads take the scalar-base ("saddr") form.
template <int BITS>
struct BCol {
  using F = Fmt<BITS>;
  static constexpr uint32_t QSLICE = 64 * 64 * BITS / 8;   // code bytes of one slice of a 64-row tile
  gbytes q, sz;        // uniform: the expert's first code byte and scale/zero word
  uint32_t qo, so;     // this lane's byte offsets at slice 0
  // m: the matrix (codes, scale/zero words); e, N: expert and rows per
  // expert; r: the row within the expert; K: row length
  MOEQ_DEV void init(const uint8_t* mq, const uint32_t* msz, int e, int N, int r, int K, int h) {
    const size_t cpr = (size_t)(K / F::CODES), gpr = (size_t)(K / 64);
    const size_t row0 = (size_t)e * N;   // a multiple of 64: offsets below split exactly
    q = uniform_ptr(mq + chunk_offset<BITS>(row0, 0, cpr));
    sz = uniform_ptr(reinterpret_cast<const uint8_t*>(msz + sz_index(row0, 0, gpr)));
    qo = (uint32_t)chunk_offset<BITS>((size_t)r, 0, cpr) + (BITS == 4 ? 8u * h : (uint32_t)h * 64u * F::BYTES);
    so = (uint32_t)sz_index((size_t)r, 0, gpr) * 4u;
  }
};

// This lane's codes of one B column for one slice, and the group's
// scale/zero word.
template <int BITS>
struct SliceCodes {
  static constexpr int NW = BITS == 4 ? 4 : (BITS == 6 ? 6 : 8);
  uint32_t d[NW];
  uint32_t sz;
  MOEQ_DEV void load(const BCol<BITS>& b, int s) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef const __attribute__((address_space(1))) u32x2* g2;
    typedef const __attribute__((address_space(1))) moeq_u32x3* g3;
    typedef const __attribute__((address_space(1))) moeq_u32x4* g4;
    const gbytes qs = b.q + (size_t)s * BCol<BITS>::QSLICE + b.qo;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (BITS == 4) {   // dwords 2h, 2h + 1 of chunk j
        const u32x2 v = *reinterpret_cast<g2>(qs + 1024 * j);
        d[2 * j] = v.x; d[2 * j + 1] = v.y;
      } else if constexpr (BITS == 6) {   // chunk h + 2j
        const moeq_u32x3 v = *reinterpret_cast<g3>(qs + 1536 * j);
        d[3 * j] = v.x; d[3 * j + 1] = v.y; d[3 * j + 2] = v.z;
      } else {
        const moeq_u32x4 v = *reinterpret_cast<g4>(qs + 2048 * j);
        d[4 * j] = v.x; d[4 * j + 1] = v.y; d[4 * j + 2] = v.z; d[4 * j + 3] = v.w;
      }
    }
    sz = load_word_g(b.sz + (size_t)s * 256 + b.so);
  }
};

// fp16 1024.0 in both halves of a VGPR (opaque, as magic_128_pair)
MOEQ_DEV uint32_t magic_1024_pair() {
  uint32_t m = 0x64006400u;
  asm volatile("" : "+v"(m));
  return m;
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
MOEQ_DEV float f16_lo(uint32_t v) { return (float)__builtin_bit_cast(f16x2_t, v).x; }
MOEQ_DEV float f16_hi(uint32_t v) { return (float)__builtin_bit_cast(f16x2_t, v).y; }

// Dequantisation of one group.  A code q is held as the fp16 value
// v = 1024 + m q, m = 1, 4 or 16 (the code OR-ed into the mantissa at bit 0,
// 2 or 4, wherever it lands without a shift), and
//     w = (q - z) s = v (s / m) - (1024 / m + z) s,
// one fma in fp32 with one rounding (v_fma_mix reads the fp16 half itself).
struct GroupDq {
  float s1, n1, sm, nm;   // (s / m, -(1024 / m + z) s) for m = 1 and m = M
  template <int M>
  MOEQ_DEV static GroupDq make(uint32_t sz) {
    const float s = f16_bits_to_f32(sz & 0xFFFFu), z = f16_bits_to_f32(sz >> 16);
    GroupDq g;
    g.s1 = s;
    g.n1 = -(1024.0f + z) * s;
    g.sm = s * (1.0f / M);
    g.nm = -(1024.0f / M + z) * s;
    return g;
  }
};

MOEQ_DEV uint32_t bf16_pair(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// The 8 weights this lane supplies at MFMA step st, dequantised and rounded
// to bf16: codes (2j, 2j + 1) of the step's 8 become pair P[j].
template <int BITS>
MOEQ_DEV bf16x8_t dequant_step(const SliceCodes<BITS>& sc, const GroupDq& g, int st) {
  const uint32_t M = magic_1024_pair();
  const int j = st >> 1, sub = st & 1;
  uint32_t r[4];
  if constexpr (BITS == 4) {
    // nibbles i and i + 4 of the dword hold codes 2i and 2i + 1
    const uint32_t d = sc.d[2 * j + sub], t = d >> 8;
    r[0] = bf16_pair(fmaf(f16_lo(and_or(d, 0x000F000Fu, M)), g.s1, g.n1), fmaf(f16_hi(and_or(d, 0x000F000Fu, M)), g.s1, g.n1));
    const uint32_t p1 = and_or(d, 0x00F000F0u, M), p3 = and_or(t, 0x00F000F0u, M), p2 = and_or(t, 0x000F000Fu, M);
    r[1] = bf16_pair(fmaf(f16_lo(p1), g.sm, g.nm), fmaf(f16_hi(p1), g.sm, g.nm));
    r[2] = bf16_pair(fmaf(f16_lo(p2), g.s1, g.n1), fmaf(f16_hi(p2), g.s1, g.n1));
    r[3] = bf16_pair(fmaf(f16_lo(p3), g.sm, g.nm), fmaf(f16_hi(p3), g.sm, g.nm));
  } else if constexpr (BITS == 6) {
    // pair i of the chunk = codes (2i, 2i + 1) from fields 3 apart (18
    // bits): the low code at bit 0 (m = 1), the high one at bit 18 (bit 2
    // of the upper half, m = 4); field_code() gives the fields.
    const uint32_t d0 = sc.d[3 * j], d1 = sc.d[3 * j + 1], d2 = sc.d[3 * j + 2];
    uint32_t P[4];
    if (sub == 0) {
      P[0] = and_or(d0, 0x00FC003Fu, M);                                      // fields 0, 3
      P[1] = and_or(d0 >> 6, 0x00FC003Fu, M);                                 // fields 1, 4
      P[2] = and_or(__builtin_amdgcn_alignbit(d1, d0, 30), 0x00FC003Fu, M);   // fields 5, 8
      P[3] = and_or(d1 >> 4, 0x00FC003Fu, M);                                 // fields 6, 9
    } else {
      P[0] = and_or(__builtin_amdgcn_alignbit(d2, d1, 28), 0x00FC003Fu, M);   // fields 10, 13
      P[1] = and_or(d2 >> 2, 0x00FC003Fu, M);                                 // fields 11, 14
      P[2] = and_or(d1 << 8, 0x00FC0000u, and_or(d0 >> 12, 0x3Fu, M));        // fields 2, 7
      P[3] = and_or(d2 >> 8, 0x00FC003Fu, M);                                 // fields 12, 15
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = bf16_pair(fmaf(f16_lo(P[i]), g.s1, g.n1), fmaf(f16_hi(P[i]), g.sm, g.nm));
  } else {
    // bytes (2i, 2i + 1) under the fp16 exponent byte 0x64
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t v = sc.d[4 * j + 2 * sub + i];
      const uint32_t pa = __builtin_amdgcn_perm(M, v, 0x05010500u), pb = __builtin_amdgcn_perm(M, v, 0x05030502u);
      r[2 * i] = bf16_pair(fmaf(f16_lo(pa), g.s1, g.n1), fmaf(f16_hi(pa), g.s1, g.n1));
      r[2 * i + 1] = bf16_pair(fmaf(f16_lo(pb), g.s1, g.n1), fmaf(f16_hi(pb), g.s1, g.n1));
    }
  }
  return __builtin_bit_cast(bf16x8_t, r);
}

template <int BITS>
MOEQ_DEV GroupDq group_dq(uint32_t sz) { return GroupDq::make<BITS == 4 ? 16 : (BITS == 6 ? 4 : 1)>(sz); }

// A (token rows) staging: BM rows x 64 bf16 per slice through registers
// into one of two LDS tiles; rows past the tile's valid count are zeros.
template <int BM>
struct ATile {
  static constexpr int N = BM * 8 / 256;   // 16-byte pieces per thread
  moeq_u32x4 v[N];
  // rows[j]: token row tid / 8 + 32 j of the tile, or null past the end
  MOEQ_DEV void load(const uint16_t* const (&rows)[N], int k0) {
#pragma unroll
    for (int j = 0; j < N; ++j)
      v[j] = rows[j] ? *reinterpret_cast<const moeq_u32x4*>(rows[j] + k0 + (threadIdx.x & 7) * 8)
                     : moeq_u32x4{0u, 0u, 0u, 0u};
  }
  MOEQ_DEV void store(uint16_t* lds) const {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int c = threadIdx.x + 256 * j;
      *reinterpret_cast<moeq_u32x4*>(lds + (c >> 3) * kLds + (c & 7) * 8) = v[j];
    }
  }
};

// A (token rows) via direct global -> LDS loads (global_load_lds_dwordx4),
// no registers involved: a slice of the tile is BM rows x 128 bytes, written
// as 1 KB pieces of 8 rows whose 64 lanes fill consecutive 16-byte slots.
// Slot t of row r holds the row's 16-byte part t ^ (r % 8): the MFMA operand
// reads of 8 consecutive rows at one k then hit 8 different slots, i.e.
// every LDS bank once.
// One 16-byte global -> LDS load per lane: lane l's data lands at
// lds + 16 l (the LDS address must be the same on every lane).  A plain
// function rather than a template member, so that the builtin is seen once.
MOEQ_DEV void load_lds_16(const uint16_t* g, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

template <int BM>
struct ADma {
  static constexpr int N = BM / 32;   // pieces per wavefront per slice
  const uint16_t* src[N];             // this lane's source at slice 0
  // Token row of piece j for this lane: row_of(j); rowp[j]: pointer to it
  // (any valid row past the tile's end: those results are never stored)
  MOEQ_DEV static int row_of(int j) { return 8 * (N * (int)(threadIdx.x >> 6) + j) + (int)((threadIdx.x & 63) >> 3); }
  MOEQ_DEV void init(const uint16_t* const (&rowp)[N]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < N; ++j) src[j] = rowp[j] + 8 * ((lane & 7) ^ (lane >> 3));
  }
  MOEQ_DEV void issue(int s, uint16_t* tile) const {
    const int wv = uniform(threadIdx.x >> 6);
#pragma unroll
    for (int j = 0; j < N; ++j)
      load_lds_16(src[j] + 64 * s, tile + 512 * (N * wv + j));
  }
};

// s_waitcnt on the vector-memory counter only: at most N of this wave's
// loads still outstanding (gfx9 encoding: vmcnt[3:0], expcnt and lgkmcnt
// left at their maxima)
template <int N>
MOEQ_DEV void wait_vmcnt() {
  static_assert(N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0xF70 | N);
}

// Barrier without a memory fence: the LDS tiles are filled by the loads
// above, whose completion each wave waits for itself (wait_vmcnt) before
// arriving; a fenced barrier would wait for every load in flight,
// including the ones issued for later slices.  The empty asm statements
// keep the compiler from moving memory accesses across it.
MOEQ_DEV void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The K loop shared by both kernels: acc[i][c] += A rows 32i .. 32i + 31 of
// the tile times B column c of this lane, over ns slices.  Three LDS tiles
// and three slices of codes in registers: slice s is computed while the
// loads of slices s + 1 and s + 2 are in flight.
template <int BITS, int BM>
struct Mainloop {
  static constexpr int MT = BM / 32;
  static constexpr int TILE = BM * 64;                 // elements of one LDS tile
  static constexpr int LOADS = ADma<BM>::N + 6;        // loads per slice: A pieces, 2 x (2 code + 1 word)
  const ADma<BM>& ad;
  const BCol<BITS>& b0;
  const BCol<BITS>& b1;
  int ns;
  f32x16_t (&acc)[MT][2];
  uint16_t* As;
  int hh;
  int aoff[4];   // element offset of this lane's A operand (M-tile 0) at each step

  MOEQ_DEV Mainloop(const ADma<BM>& ad_, const BCol<BITS>& b0_, const BCol<BITS>& b1_, int ns_,
                    f32x16_t (&acc_)[MT][2], uint16_t* As_)
      : ad(ad_), b0(b0_), b1(b1_), ns(ns_), acc(acc_), As(As_) {
    const int lane = threadIdx.x & 63;
    hh = lane >> 5;
#pragma unroll
    for (int st = 0; st < 4; ++st) aoff[st] = (lane & 31) * 64 + 8 * ((step_k(st, hh) >> 3) ^ (lane & 7));
  }

  MOEQ_DEV void run() {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) { acc[i][0][r] = 0.0f; acc[i][1][r] = 0.0f; }
    SliceCodes<BITS> c[3][2];   // ring: slices s, s + 1, s + 2
    __builtin_amdgcn_sched_barrier(0);
    ad.issue(0, As);
    c[0][0].load(b0, 0);
    c[0][1].load(b1, 0);
    const int s1 = min(1, ns - 1);
    ad.issue(s1, As + TILE);
    c[1][0].load(b0, s1);
    c[1][1].load(b1, s1);
    __builtin_amdgcn_sched_barrier(0);
    for (int s = 0; s < ns; s += 3) {
      slice(s, c[0], c[2]);
      if (s + 1 < ns) slice(s + 1, c[1], c[0]);
      if (s + 2 < ns) slice(s + 2, c[2], c[1]);
    }
  }

  MOEQ_DEV void slice(int s, const SliceCodes<BITS> (&cur)[2], SliceCodes<BITS> (&ahead)[2]) {
    // this wave's loads of slice s are done once only the next slice's
    // remain (every slice issues the same loads, see below)
    wait_vmcnt<LOADS>();
    tile_barrier();   // every wave's tile s is in LDS; tile s - 1 is no longer read
    __builtin_amdgcn_sched_barrier(0);
    // the loads of slice s + 2; past the end, the last slice again (its
    // data goes unused) so that the count of loads in flight never depends
    // on s
    const int sn = min(s + 2, ns - 1);
    ad.issue(sn, As + TILE * ((s + 2) % 3));
    ahead[0].load(b0, sn);
    ahead[1].load(b1, sn);
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* A = As + TILE * (s % 3);
    const GroupDq g0 = group_dq<BITS>(cur[0].sz), g1 = group_dq<BITS>(cur[1].sz);
    // software pipeline over the 4 MFMA steps: the weights of step st + 1
    // are dequantised while the matrix cores run step st, the vector and
    // matrix instructions interleaved (a few VALU per MFMA)
    bf16x8_t w0 = dequant_step<BITS>(cur[0], g0, 0), w1 = dequant_step<BITS>(cur[1], g1, 0);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t a[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) a[i] = *reinterpret_cast<const bf16x8_t*>(A + 2048 * i + aoff[st]);
      bf16x8_t n0 = w0, n1 = w1;
      if (st < 3) {
        n0 = dequant_step<BITS>(cur[0], g0, st + 1);
        n1 = dequant_step<BITS>(cur[1], g1, st + 1);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], w0, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], w1, acc[i][1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);   // the A reads first
#pragma unroll
      for (int i = 0; i < 2 * MT; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // then up to 5 VALU
      }
      w0 = n0;
      w1 = n1;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
};

// Block -> (work item, feature tile): the feature tiles of one work item (one
// expert's token tile) land on one XCD (blocks are dealt to the 8 XCDs
// round-robin) back to back, so the token rows they all read come from that
// XCD's L2 after the first.  The grid is (work items rounded up to a
// multiple of 8) x nft.
MOEQ_DEV void block_tile(int nft, int& w, int& ft) {
  const int b = (int)blockIdx.x, r = b % 8, slot = b / 8;
  w = (slot / nft) * 8 + r;
  ft = slot % nft;
}

// gate/up: per (expert, BM-token tile, 128 features of I): h = silu(x Wg^T) *
// (x Wu^T) rounded to bf16, rows in expert-sorted order.  Wavefront wv owns
// features 32 wv .. 32 wv + 31 of the tile, of both gate and up.
template <int BITS, int BM>
__global__ __launch_bounds__(256, 2) void mfma_gateup_kernel(const uint8_t* __restrict__ gq,
                                                             const uint32_t* __restrict__ gsz,
                                                             const uint8_t* __restrict__ uq,
                                                             const uint32_t* __restrict__ usz,
                                                             const uint16_t* __restrict__ x, int H, int I, int kS,
                                                             const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ sorted,
                                                             const int32_t* __restrict__ sched,
                                                             uint16_t* __restrict__ h) {
  constexpr int MT = BM / 32;
  __shared__ __attribute__((aligned(16))) uint16_t As[3][BM * 64];
  int wi, ft;
  block_tile(I / 128, wi, ft);
  if (wi >= sched[0]) return;
  const int e = sched[2 + 2 * wi], mt = sched[3 + 2 * wi];
  const int base = offsets[e] + mt * BM;
  const int rows = min(BM, counts[e] - mt * BM);
  const int lane = threadIdx.x & 63, hh = lane >> 5;
  const int wv = uniform(threadIdx.x >> 6);
  const int f = ft * 128 + 32 * wv + (lane & 31);   // this lane's feature (B column)
  ADma<BM> ad;
  {
    const uint16_t* rowp[ADma<BM>::N];
#pragma unroll
    for (int j = 0; j < ADma<BM>::N; ++j)
      rowp[j] = x + (size_t)(sorted[base + min(ADma<BM>::row_of(j), rows - 1)] / kS) * H;
    ad.init(rowp);
  }
  BCol<BITS> bg, bu;
  bg.init(gq, gsz, e, I, f, H, hh);
  bu.init(uq, usz, e, I, f, H, hh);
  f32x16_t acc[MT][2];
  Mainloop<BITS, BM>(ad, bg, bu, H / 64, acc, &As[0][0]).run();
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (m < rows) h[(size_t)(base + m) * I + f] = (uint16_t)f32_to_bf16_bits(silu_f32(acc[i][0][r]) * acc[i][1][r]);
    }
}

// down: per (expert, BM-token tile, 256 features of H): y = h Wd^T rounded to
// bf16 and scattered to assignment order.  Wavefront wv owns features
// 64 wv + (0 .. 31) and 64 wv + 32 + (0 .. 31) of the tile (two B columns
// per lane).
template <int BITS, int BM>
__global__ __launch_bounds__(256, 2) void mfma_down_kernel(const uint8_t* __restrict__ dq,
                                                           const uint32_t* __restrict__ dsz,
                                                           const uint16_t* __restrict__ h, int H, int I,
                                                           const int32_t* __restrict__ counts,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ sorted,
                                                           const int32_t* __restrict__ sched,
                                                           uint16_t* __restrict__ y) {
  constexpr int MT = BM / 32;
  __shared__ __attribute__((aligned(16))) uint16_t As[3][BM * 64];
  int wi, ft;
  block_tile(H / 256, wi, ft);
  if (wi >= sched[0]) return;
  const int e = sched[2 + 2 * wi], mt = sched[3 + 2 * wi];
  const int base = offsets[e] + mt * BM;
  const int rows = min(BM, counts[e] - mt * BM);
  const int lane = threadIdx.x & 63, hh = lane >> 5;
  const int wv = uniform(threadIdx.x >> 6);
  const int f0 = ft * 256 + 64 * wv + (lane & 31);   // features f0 and f0 + 32
  ADma<BM> ad;
  {
    const uint16_t* rowp[ADma<BM>::N];
#pragma unroll
    for (int j = 0; j < ADma<BM>::N; ++j) rowp[j] = h + (size_t)(base + min(ADma<BM>::row_of(j), rows - 1)) * I;
    ad.init(rowp);
  }
  BCol<BITS> c0, c1;
  c0.init(dq, dsz, e, H, f0, I, hh);
  c1.init(dq, dsz, e, H, f0 + 32, I, hh);
  f32x16_t acc[MT][2];
  Mainloop<BITS, BM>(ad, c0, c1, I / 64, acc, &As[0][0]).run();
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (m < rows) {
        const size_t a = (size_t)sorted[base + m];
        y[a * H + f0] = (uint16_t)f32_to_bf16_bits(acc[i][0][r]);
        y[a * H + f0 + 32] = (uint16_t)f32_to_bf16_bits(acc[i][1][r]);
      }
    }
}

// Router logits at large batch: C[m][n] = sum_k A[m][k] B[n][k] + bias[n],
// fp32 out.  One block per 32 x 32 output tile; its four wavefronts take
// every fourth 64-slice of K, with the operands loaded from global memory
// (L2) straight into MFMA registers (lane l: 8 consecutive k of row l % 32),
// and their partial tiles are added in LDS in a fixed order, so the result
// does not depend on timing.  Rows past M or N read row M - 1 or N - 1 and
// are not stored.
__global__ __launch_bounds__(256) void gemm_nt_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                      const float* __restrict__ bias, int M, int N, int K,
                                                      float* __restrict__ C) {
  __shared__ f32x16_t part[3][64];
  const int m0 = blockIdx.x * 32, n0 = blockIdx.y * 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r = lane & 31, hh = lane >> 5;
  const uint16_t* ap = A + (size_t)min(m0 + r, M - 1) * K + 8 * hh;
  const uint16_t* bp = B + (size_t)min(n0 + r, N - 1) * K + 8 * hh;
  const int ns = K / 64;
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  bf16x8_t a[4], b[4];
  auto load = [&](int s) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a[t] = *reinterpret_cast<const bf16x8_t*>(ap + 64 * s + 16 * t);
      b[t] = *reinterpret_cast<const bf16x8_t*>(bp + 64 * s + 16 * t);
    }
  };
  if (wave < ns) load(wave);
  for (int s = wave; s < ns; s += 4) {
    bf16x8_t ca[4], cb[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) { ca[t] = a[t]; cb[t] = b[t]; }
    if (s + 4 < ns) load(s + 4);
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ca[t], cb[t], acc, 0, 0, 0);
  }
  if (wave > 0) part[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) acc += part[w][lane];
  const int n = n0 + r;
  if (n >= N) return;
  const float bn = bias ? bias[n] : 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = m0 + 8 * (i >> 2) + 4 * hh + (i & 3);
    if (m < M) C[(size_t)m * N + n] = acc[i] + bn;
  }
}

// Router logits for large batches and expert counts: 128 x 128 output
// tiles, both operands staged through double-buffered LDS tiles in
// K-slices of 64; wavefront (wm, wn) owns the 64 x 64 sub-tile (wm, wn).
__global__ __launch_bounds__(256) void gemm_nt_tiled_kernel(const uint16_t* __restrict__ A,
                                                            const uint16_t* __restrict__ B,
                                                            const float* __restrict__ bias, int M, int N, int K,
                                                            float* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][128 * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][128 * kLds];
  const int m0 = blockIdx.x * 128, n0 = blockIdx.y * 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1, hh = lane >> 5;
  const uint16_t* arow[4];
  const uint16_t* brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (threadIdx.x >> 3) + 32 * j;
    arow[j] = m0 + r < M ? A + (size_t)(m0 + r) * K : nullptr;
    brow[j] = n0 + r < N ? B + (size_t)(n0 + r) * K : nullptr;
  }
  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc[i][0][r] = 0.0f; acc[i][1][r] = 0.0f; }
  ATile<128> sa, sb;
  sa.load(arow, 0);
  sb.load(brow, 0);
  sa.store(As[0]);
  sb.store(Bs[0]);
  const int ns = K / 64;
  for (int s = 0; s < ns; ++s) {
    __syncthreads();
    if (s + 1 < ns) {
      sa.load(arow, (s + 1) * 64);
      sb.load(brow, (s + 1) * 64);
    }
    const uint16_t* a_s = As[s & 1] + (64 * wm + (lane & 31)) * kLds + 8 * hh;
    const uint16_t* b_s = Bs[s & 1] + (64 * wn + (lane & 31)) * kLds + 8 * hh;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *reinterpret_cast<const bf16x8_t*>(a_s + 32 * i * kLds + 16 * t);
        b[i] = *reinterpret_cast<const bf16x8_t*>(b_s + 32 * i * kLds + 16 * t);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < ns) {
      sa.store(As[(s + 1) & 1]);
      sb.store(Bs[(s + 1) & 1]);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + 64 * wn + 32 * j + (lane & 31);
    if (n >= N) continue;
    const float bn = bias ? bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (m < M) C[(size_t)m * N + n] = acc[i][j][r] + bn;
      }
  }
}

}  // namespace

namespace moeq {
int gemm_bf16_nt(const uint16_t* A, const uint16_t* B, const float* bias, int M, int N, int K, float* C,
                 hipStream_t stream) {
  if (M == 0 || N == 0) return MOEQ_OK;
  const long tiles128 = (long)((M + 127) / 128) * ((N + 127) / 128);
  if (tiles128 >= 128) {   // enough large tiles to fill the chip
    dim3 grid((M + 127) / 128, (N + 127) / 128);
    gemm_nt_tiled_kernel<<<grid, 256, 0, stream>>>(A, B, bias, M, N, K, C);
  } else {
    dim3 grid((M + 31) / 32, (N + 31) / 32);
    gemm_nt_kernel<<<grid, 256, 0, stream>>>(A, B, bias, M, N, K, C);
  }
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
  if (L->I % 128 || L->H % 256)
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_qgemm_prefill: I=%d must be a multiple of 128 and H=%d of 256",
                     L->I, L->H);
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
  const unsigned nw = (unsigned)((max_tiles + 7) / 8 * 8);   // work items, padded for the XCD mapping
  const unsigned g1 = nw * (unsigned)(L->I / 128), g2 = nw * (unsigned)(L->H / 256);
  switch (L->gate.bits) {
    case 4: mfma_gateup_kernel<4, BM><<<g1, 256, 0, stream>>>(L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, kS, counts, offsets, sorted, sched, h); break;
    case 6: mfma_gateup_kernel<6, BM><<<g1, 256, 0, stream>>>(L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, kS, counts, offsets, sorted, sched, h); break;
    default: mfma_gateup_kernel<8, BM><<<g1, 256, 0, stream>>>(L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, kS, counts, offsets, sorted, sched, h); break;
  }
  if ((rc = check_launch("moe_qgemm_prefill (gate/up)")) != MOEQ_OK) return rc;
  switch (L->down.bits) {
    case 4: mfma_down_kernel<4, BM><<<g2, 256, 0, stream>>>(L->down.q, L->down.sz, h, L->H, L->I, counts, offsets, sorted, sched, y); break;
    case 6: mfma_down_kernel<6, BM><<<g2, 256, 0, stream>>>(L->down.q, L->down.sz, h, L->H, L->I, counts, offsets, sorted, sched, y); break;
    default: mfma_down_kernel<8, BM><<<g2, 256, 0, stream>>>(L->down.q, L->down.sz, h, L->H, L->I, counts, offsets, sorted, sched, y); break;
  }
  return check_launch("moe_qgemm_prefill (down)");
}
