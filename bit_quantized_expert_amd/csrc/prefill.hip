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
// routing back; blocks past the end of the list exit at once.  Experts with
// at most kPrefillGemvMax assignments (under a skewed router most of the
// experts a chunk touches get a token or two) are left out of that list and
// go to the decode GEMV kernels instead, which stream their weights once at
// ~1 VALU per weight and token rather than a dequantised matrix-core slice
// loop per token tile.
// Prior art: a long prompt touches nearly all experts (Qwen-tin, "Memory
// layout and performance"), so every expert's weights are streamed once per
// token tile.
#include "gemm_bf16.h"
#include "decode_impl.h"

#include <type_traits>

using namespace moeq;

namespace {

constexpr int BM = kPrefillBM;   // 128 tokens per tile

// sched[0] = number of work items; sched[2 + 2i], sched[3 + 2i] = (expert, token tile).
// Work items are listed by the number of 32-row M-tiles they fill, most
// first (full tiles, then partial ones from the largest down), so that
// blocks dealt out last are the short ones and fill the tail of the launch.
// gemv[0] = number of experts with 1 .. kPrefillGemvMax assignments, gemv[1
// ..] their ids, ascending (the decode kernels' list of active experts).
// One block of 256 threads; thread i takes a contiguous range of experts;
// the four per-bucket counts and the list count are scanned together.
__global__ __launch_bounds__(256) void schedule_kernel(const int32_t* __restrict__ counts, int nexp, int nrouted,
                                                       int32_t* __restrict__ sched, int32_t* __restrict__ gemv) {
  constexpr int NBK = BM / 32;   // buckets: 1 .. NBK M-tiles
  static_assert(NBK == 4, "four buckets");
  __shared__ int4 part[256];
  __shared__ int partg[256];
  const int tid = threadIdx.x;
  const int per = (nexp + 255) / 256;
  const int e0 = min(nexp, tid * per), e1 = min(nexp, e0 + per);
  auto mtiles = [](int c, int m) { return (min(BM, c - m * BM) + 31) / 32; };
  // routed experts only: the GEMV list kernels take routed ids; the list is
  // used only when it holds at least kPrefillGemvMin experts (a shorter one
  // costs more as its own launches than it saves on the matrix cores)
  auto small = [nrouted](int e, int c) { return e < nrouted && c > 0 && c <= kPrefillGemvMax; };
  int mg = 0;
  for (int e = e0; e < e1; ++e) mg += small(e, counts[e]) ? 1 : 0;
  int vg = mg;
  partg[tid] = vg;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {   // inclusive scan of the list counts
    const int ug = tid >= o ? partg[tid - o] : 0;
    __syncthreads();
    vg += ug;
    partg[tid] = vg;
    __syncthreads();
  }
  const bool use = partg[255] >= kPrefillGemvMin;
  auto on_gemv = [&](int e, int c) { return use && small(e, c); };
  int mine[NBK + 1] = {0, 0, 0, 0, 0};
  for (int e = e0; e < e1; ++e) {
    const int c = counts[e];
    if (on_gemv(e, c)) continue;
    mine[4] += c / BM;   // full tiles
    if (c % BM) mine[mtiles(c, c / BM)] += 1;
  }
  int4 v = make_int4(mine[1], mine[2], mine[3], mine[4]);
  part[tid] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {   // inclusive Hillis-Steele scan of the four bucket counts
    const int4 u = tid >= o ? part[tid - o] : make_int4(0, 0, 0, 0);
    __syncthreads();
    v.x += u.x; v.y += u.y; v.z += u.z; v.w += u.w;
    part[tid] = v;
    __syncthreads();
  }
  const int4 tot = part[255];
  int pg = vg - mg;   // this thread's first slot in the GEMV list
  // bucket order 4, 3, 2, 1: exclusive start of this thread in each
  int pos[NBK + 1];
  pos[4] = v.w - mine[4];
  pos[3] = tot.w + v.z - mine[3];
  pos[2] = tot.w + tot.z + v.y - mine[2];
  pos[1] = tot.w + tot.z + tot.y + v.x - mine[1];
  for (int e = e0; e < e1; ++e) {
    const int c = counts[e], nt = (c + BM - 1) / BM;
    if (on_gemv(e, c)) {
      gemv[1 + pg++] = e;
      continue;
    }
    for (int m = 0; m < nt; ++m) {
      const int p = pos[mtiles(c, m)]++;
      sched[2 + 2 * p] = e;
      sched[3 + 2 * p] = m;
    }
  }
  if (tid == 0) {
    sched[0] = tot.x + tot.y + tot.z + tot.w;
    gemv[0] = use ? partg[255] : 0;
  }
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

// One global -> LDS load of 4, 12 or 16 bytes per lane: lane l's data lands
// at lds + 16 l (+ 4 l for 4 bytes); the LDS address must be the same on
// every lane.  Plain functions rather than template members, so that each
// builtin is seen once.
MOEQ_DEV void load_lds_16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
MOEQ_DEV void load_lds_12(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 12, 0, 0);
}
MOEQ_DEV void load_lds_4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 4, 0, 0);
}
MOEQ_DEV void load_lds_16(gbytes g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
MOEQ_DEV void load_lds_12(gbytes g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 12, 0, 0);
}

// The codes of a wavefront's two B columns (32 weight rows each) for one
// slice, and those rows' scale/zero words, moved global -> LDS by the
// wavefront itself (no other wavefront reads them).  One wavefront's stage
// in LDS:
//   column c = 0, 1: NI loads of 64 lanes x 16 bytes; load j, lane L holds
//   the chunk row (chunk 2j + L / 32 of the slice, row L % 32): the whole
//   16 bytes at 4 and 8 bits, 12 of the 16 at 6 bits;
//   then the 64 scale/zero words, [column][row].
template <int BITS>
struct BDma {
  using F = Fmt<BITS>;
  static constexpr int NI = BITS == 4 ? 1 : 2;             // loads per column per slice
  static constexpr int COL = NI * 1024;                    // LDS bytes per column
  static constexpr int STAGE = 2 * COL + 256;              // LDS bytes per wavefront per slice
  static constexpr int LOADS = 2 * NI + 1;                 // vector-memory loads per slice
  static constexpr size_t QSLICE = 64 * 64 * BITS / 8;     // code bytes of one slice of a 64-row tile
  gbytes q0[2];            // uniform: column c's first code byte (row 0 of its 32-row block, chunk 0)
  uint32_t qo[NI];         // this lane's byte offsets from them (the same for both columns)
  const uint32_t* szsrc;   // this lane's scale/zero source at slice 0 (column lane / 32)
  // q, szm: the columns' matrices; row[c]: the first of column c's 32 rows
  // (over all experts' rows, a multiple of 32); K: row length
  MOEQ_DEV void init(const uint8_t* const (&q)[2], const uint32_t* const (&szm)[2], const size_t (&row)[2], int K) {
    const int lane = threadIdx.x & 63;
    const size_t cpr = (size_t)(K / F::CODES), gpr = (size_t)(K / 64);
#pragma unroll
    for (int c = 0; c < 2; ++c) q0[c] = uniform_ptr(q[c] + chunk_offset<BITS>(row[c], 0, cpr));
    // chunk 2j + lane / 32 of the slice, row lane % 32 of the block: rows of
    // one tile are F::BYTES apart, chunks 64 F::BYTES
#pragma unroll
    for (int j = 0; j < NI; ++j) qo[j] = (uint32_t)(((2 * j + (lane >> 5)) * 64 + (lane & 31)) * F::BYTES);
    const int c = lane >> 5;
    szsrc = szm[c] + sz_index(row[c] + (lane & 31), 0, gpr);
  }
  MOEQ_DEV void issue(int s, uint8_t* stage) const {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const gbytes base = q0[c] + (size_t)s * QSLICE;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        if constexpr (BITS == 6) load_lds_12(base + qo[j], stage + c * COL + 1024 * j);
        else load_lds_16(base + qo[j], stage + c * COL + 1024 * j);
      }
    }
    load_lds_4(szsrc + (size_t)s * 64, stage + 2 * COL);
  }
};

// This lane's codes of one B column for one slice, and the group's
// scale/zero word, read from the wavefront's LDS stage.
//   4-bit: dwords 2h, 2h + 1 of chunks 0 and 1 -> d[2j], d[2j + 1];
//   6-, 8-bit: chunks h and h + 2 whole -> d[NW/2 j ..].
template <int BITS>
struct SliceCodes {
  static constexpr int NW = BITS == 4 ? 4 : (BITS == 6 ? 6 : 8);
  uint32_t d[NW];
  uint32_t sz;
  MOEQ_DEV void read(const uint8_t* stage, int c) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
    const uint8_t* col = stage + c * BDma<BITS>::COL;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if constexpr (BITS == 4) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(col + 512 * j + 16 * r + 8 * h);
        d[2 * j] = v.x; d[2 * j + 1] = v.y;
      } else if constexpr (BITS == 6) {
        const moeq_u32x3 v = *reinterpret_cast<const moeq_u32x3*>(col + 1024 * j + 16 * (32 * h + r));
        d[3 * j] = v.x; d[3 * j + 1] = v.y; d[3 * j + 2] = v.z;
      } else {
        const moeq_u32x4 v = *reinterpret_cast<const moeq_u32x4*>(col + 1024 * j + 16 * (32 * h + r));
        d[4 * j] = v.x; d[4 * j + 1] = v.y; d[4 * j + 2] = v.z; d[4 * j + 3] = v.w;
      }
    }
    sz = *reinterpret_cast<const uint32_t*>(stage + 2 * BDma<BITS>::COL + 4 * (32 * c + r));
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
// 2 or 4, wherever it lands without a shift).  v - 1024 = m q exactly (one
// packed fp16 subtraction per pair), and
//     w = (q - z) s = (m q) (s / m) - z s
// is one fma in fp32 with one rounding: z s is a product of two fp16 values
// (22 significant bits), exact in fp32, and (m q)(s / m) = q s is exact, so
// w is fp32((q - z) s) rounded once, the plain dequantised weight.  It is
// then rounded to bf16 for the matrix cores.
struct GroupDq {
  float s1, sm, nzs;   // s / 1, s / M, -(z s)
  template <int M>
  MOEQ_DEV static GroupDq make(uint32_t sz) {
    const float s = f16_bits_to_f32(sz & 0xFFFFu), z = f16_bits_to_f32(sz >> 16);
    GroupDq g;
    g.s1 = s;
    g.sm = s * (1.0f / M);
    g.nzs = -(z * s);
    return g;
  }
};

typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
// (1024 + m q_lo, 1024 + m q_hi) -> (m q_lo, m q_hi), exact
MOEQ_DEV f16x2v minus_1024(uint32_t p) {
  return __builtin_bit_cast(f16x2v, p) - f16x2v{(_Float16)1024.0f, (_Float16)1024.0f};
}

MOEQ_DEV uint32_t bf16_pair(float lo, float hi) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const bf2 v = {(__bf16)lo, (__bf16)hi};   // v_cvt_pk_bf16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// One pair of weights: codes (m_lo q_lo, m_hi q_hi) held as 1024 + m q in
// the fp16 halves of p, scales s_lo = s / m_lo and s_hi = s / m_hi.
MOEQ_DEV uint32_t dq_pair(uint32_t p, float s_lo, float s_hi, float nzs) {
  const f16x2v t = minus_1024(p);
  return bf16_pair(fmaf((float)t.x, s_lo, nzs), fmaf((float)t.y, s_hi, nzs));
}

// The 8 weights this lane supplies at MFMA step st, dequantised and rounded
// to bf16: codes (2j, 2j + 1) of the step's 8 become pair P[j].  M:
// magic_1024_pair().
template <int BITS>
MOEQ_DEV bf16x8_t dequant_step(const SliceCodes<BITS>& sc, const GroupDq& g, int st, uint32_t M) {
  const int j = st >> 1, sub = st & 1;
  uint32_t r[4];
  if constexpr (BITS == 4) {
    // nibbles i and i + 4 of the dword hold codes 2i and 2i + 1
    const uint32_t d = sc.d[2 * j + sub], t = d >> 8;
    r[0] = dq_pair(and_or(d, 0x000F000Fu, M), g.s1, g.s1, g.nzs);
    r[1] = dq_pair(and_or(d, 0x00F000F0u, M), g.sm, g.sm, g.nzs);
    r[2] = dq_pair(and_or(t, 0x000F000Fu, M), g.s1, g.s1, g.nzs);
    r[3] = dq_pair(and_or(t, 0x00F000F0u, M), g.sm, g.sm, g.nzs);
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
    for (int i = 0; i < 4; ++i) r[i] = dq_pair(P[i], g.s1, g.sm, g.nzs);
  } else {
    // bytes (2i, 2i + 1) under the fp16 exponent byte 0x64
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t v = sc.d[4 * j + 2 * sub + i];
      r[2 * i] = dq_pair(__builtin_amdgcn_perm(M, v, 0x05010500u), g.s1, g.s1, g.nzs);
      r[2 * i + 1] = dq_pair(__builtin_amdgcn_perm(M, v, 0x05030502u), g.s1, g.s1, g.nzs);
    }
  }
  return __builtin_bit_cast(bf16x8_t, r);
}

template <int BITS>
MOEQ_DEV GroupDq group_dq(uint32_t sz) { return GroupDq::make<BITS == 4 ? 16 : (BITS == 6 ? 4 : 1)>(sz); }

// A (token rows) staging: BM rows x 64 bf16 per slice through registers
// into one of two LDS tiles.
template <int BM>
struct ATile {
  static constexpr int N = BM * 8 / 256;   // 16-byte pieces per thread
  moeq_u32x4 v[N];
  // rows[j]: row tid / 8 + 32 j of the tile (every pointer valid: rows past
  // the operand's end repeat its last row, whose products are not stored),
  // so that the loads are unconditional and the compiler counts them exactly
  MOEQ_DEV void load(const uint16_t* const (&rows)[N], int k0) {
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = *reinterpret_cast<const moeq_u32x4*>(rows[j] + k0 + (threadIdx.x & 7) * 8);
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
// Slot t of row r holds the row's 16-byte part t ^ swz(r), swz(r) =
// (r / 2) % 8: rows are 128 bytes, so even and odd rows start on opposite
// halves of the 64 banks, and the MFMA operand reads of 16 consecutive rows
// at one k hit 16 different (half, slot) pairs, i.e. every bank once.
template <int BM>
struct ADma {
  static constexpr int N = BM / 32;   // pieces per wavefront per slice
  const uint16_t* src[N];             // this lane's source at slice 0
  // Token row of piece j for this lane: row_of(j); rowp[j]: pointer to it
  // (any valid row past the tile's end: those results are never stored)
  MOEQ_DEV static int row_of(int j) { return 8 * (N * (int)(threadIdx.x >> 6) + j) + (int)((threadIdx.x & 63) >> 3); }
  MOEQ_DEV static int swz(int r) { return (r >> 1) & 7; }
  MOEQ_DEV void init(const uint16_t* const (&rowp)[N]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < N; ++j) src[j] = rowp[j] + 8 * ((lane & 7) ^ swz(row_of(j)));
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

// LDS stages of the token-row tiles (NA) and of the code slices (NB) per
// bit width: three of each where they fit two blocks per CU into the
// 160 KB of LDS, else two.
template <int BITS> struct Stages { static constexpr int NA = BITS == 4 ? 3 : 2, NB = BITS == 4 ? 3 : 2; };

template <int BITS, int BM>
constexpr int lds_bytes() {
  return Stages<BITS>::NA * BM * 64 * 2 + Stages<BITS>::NB * 4 * BDma<BITS>::STAGE;
}

// The K loop shared by both kernels: acc[i][c] += A rows 32i .. 32i + 31 of
// the tile times B column c of this lane, over ns slices.  Slice s is
// computed while the loads of the next NA - 1 token-row tiles and NB - 1
// code slices are in flight; all of them go global -> LDS without
// registers, so the only waits for them are the explicit wait_vmcnt ones.
template <int BITS, int BM, int MTA>
struct Mainloop {
  static constexpr int MT = BM / 32;   // M-tiles of the LDS tile; MTA of them hold rows
  static constexpr int NA = Stages<BITS>::NA, NB = Stages<BITS>::NB;
  static constexpr int ATILE = BM * 64 * 2;              // bytes of one token-row tile
  // token rows moved per slice: only those of the MTA M-tiles that hold rows
  // (a tile of one or two tokens loads 32 rows, not BM)
  using AD = ADma<32 * MTA>;
  static constexpr int LA = AD::N, LB = BDma<BITS>::LOADS;
  // loads issued after those of slice s + 1 when slice s ends (each slice
  // issues token rows, then codes; see run())
  static constexpr int WAIT = (NA == 3 && NB == 3) ? LA + LB : (NA == 2 && NB == 3) ? LB : 0;
  static_assert(NA == 2 || NB == 3, "stage combination");
  // the next slice's first B operands are dequantised during the last
  // MFMA step of this one, except at 6 bits where the unpacking needs the
  // registers (there they are dequantised when the slice starts)
  static constexpr bool EARLY_DQ = BITS != 6;
  const AD& ad;
  const BDma<BITS>& bd;
  int ns;
  f32x16_t (&acc)[MT][2];
  uint8_t* lds;   // NA token-row tiles, then NB x 4 wavefront code stages
  int hh, wv;
  int aoff[4];    // byte offset of this lane's A operand (M-tile 0) at each step

  MOEQ_DEV Mainloop(const AD& ad_, const BDma<BITS>& bd_, int ns_, f32x16_t (&acc_)[MT][2], uint8_t* lds_)
      : ad(ad_), bd(bd_), ns(ns_), acc(acc_), lds(lds_) {
    const int lane = threadIdx.x & 63;
    hh = lane >> 5;
    wv = uniform(threadIdx.x >> 6);
#pragma unroll
    for (int st = 0; st < 4; ++st)
      aoff[st] = 2 * ((lane & 31) * 64 + 8 * ((step_k(st, hh) >> 3) ^ ADma<BM>::swz(lane & 31)));
  }
  MOEQ_DEV uint16_t* a_tile(int t) const { return reinterpret_cast<uint16_t*>(lds + ATILE * t); }
  MOEQ_DEV uint8_t* b_stage(int t) const { return lds + NA * ATILE + (4 * t + wv) * BDma<BITS>::STAGE; }

  // the loads of what slice t will compute; past the end the last slice
  // again (its data goes unused), so that the count of loads in flight
  // never depends on t
  MOEQ_DEV void issue_a(int t) const { ad.issue(min(t, ns - 1), a_tile(t % NA)); }
  MOEQ_DEV void issue_b(int t) const { bd.issue(min(t, ns - 1), b_stage(t % NB)); }

  // A slice's codes read from LDS, with the B operands of its first MFMA
  // step already dequantised
  struct Ready {
    SliceCodes<BITS> cur[2];
    GroupDq g[2];
    bf16x8_t w[2];
  };
  MOEQ_DEV void prepare(int s, Ready& r) const {
    r.cur[0].read(b_stage(s % NB), 0);
    r.cur[1].read(b_stage(s % NB), 1);
    if constexpr (EARLY_DQ) dequant_first(r);
  }
  MOEQ_DEV static void dequant_first(Ready& r) {
    r.g[0] = group_dq<BITS>(r.cur[0].sz);
    r.g[1] = group_dq<BITS>(r.cur[1].sz);
    const uint32_t M = magic_1024_pair();
    r.w[0] = dequant_step<BITS>(r.cur[0], r.g[0], 0, M);
    r.w[1] = dequant_step<BITS>(r.cur[1], r.g[1], 0, M);
  }

  MOEQ_DEV void run() {
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) { acc[i][0][r] = 0.0f; acc[i][1][r] = 0.0f; }
    __builtin_amdgcn_sched_barrier(0);
    // what slices -2 and -1 would have issued
#pragma unroll
    for (int t = -2; t < 0; ++t) {
      if (t + NA - 1 >= 0) issue_a(t + NA - 1);
      __builtin_amdgcn_sched_barrier(0);
      if (t + NB - 1 >= 0) issue_b(t + NB - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmcnt<WAIT>();
    Ready r;
    prepare(0, r);
    tile_barrier();
    __builtin_amdgcn_sched_barrier(0);
    for (int s = 0; s < ns; ++s) {
      issue_a(s + NA - 1);
      __builtin_amdgcn_sched_barrier(0);
      issue_b(s + NB - 1);
      __builtin_amdgcn_sched_barrier(0);
      slice(s, r);
      // every wave's token-row tile s + 1 is in LDS; tile s is no longer read
      tile_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    // the loads issued past the last slice still write LDS: let them land
    // before the caller reuses it
    wait_vmcnt<0>();
    tile_barrier();
  }

  // Slice s from r; on return r holds slice s + 1 (its codes are this
  // wave's own loads, so they are read before the barrier, while the last
  // MFMAs of slice s run).  Past the last slice r reads the repeated last
  // slice, which goes unused.
  MOEQ_DEV void slice(int s, Ready& r) {
    // the wave's issue priority is raised while it feeds the matrix cores
    // and lowered for the loads and the barrier, so that of the two waves
    // on a SIMD the one with MFMAs to issue goes first (1-3 % faster)
    __builtin_amdgcn_s_setprio(1);
    const uint8_t* A = reinterpret_cast<const uint8_t*>(a_tile(s % NA));
    if constexpr (!EARLY_DQ) dequant_first(r);
    const SliceCodes<BITS> cur[2] = {r.cur[0], r.cur[1]};
    const GroupDq g0 = r.g[0], g1 = r.g[1];
    // software pipeline over the 4 MFMA steps: the A operands and the
    // weights of step st + 1 are fetched and dequantised while the matrix
    // cores run step st, vector and matrix instructions interleaved
    bf16x8_t w0 = r.w[0], w1 = r.w[1];
    const uint32_t M = magic_1024_pair();
    bf16x8_t a[MTA];
#pragma unroll
    for (int i = 0; i < MTA; ++i) a[i] = *reinterpret_cast<const bf16x8_t*>(A + 4096 * i + aoff[0]);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      __builtin_amdgcn_sched_barrier(0);
      bf16x8_t an[MTA], n0 = w0, n1 = w1;
      if (st < 3) {
#pragma unroll
        for (int i = 0; i < MTA; ++i) an[i] = *reinterpret_cast<const bf16x8_t*>(A + 4096 * i + aoff[st + 1]);
        n0 = dequant_step<BITS>(cur[0], g0, st + 1, M);
        n1 = dequant_step<BITS>(cur[1], g1, st + 1, M);
      } else {
        // this wave's loads of slice s + 1 are complete once WAIT remain
        wait_vmcnt<WAIT>();
        prepare(s + 1, r);
      }
#pragma unroll
      for (int i = 0; i < MTA; ++i) {
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], w0, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], w1, acc[i][1], 0, 0, 0);
      }
      if (st < 3) __builtin_amdgcn_sched_group_barrier(0x100, MTA, 0);   // LDS reads first
      else __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int i = 0; i < 2 * MTA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // then up to 5 VALU
      }
      if (st < 3) {
#pragma unroll
        for (int i = 0; i < MTA; ++i) a[i] = an[i];
      }
      w0 = n0;
      w1 = n1;
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
  }
};

// Block -> (work item, feature tile): the feature tiles of one work item (one
// expert's token tile) land on one XCD (blocks are dealt to the 8 XCDs
// round-robin) back to back, so the token rows they all read come from that
// XCD's L2 after the first; and runs of xrun consecutive work items (the
// token tiles of one expert sit next to each other in the schedule) go to
// the same XCD, so that its L2 serves their common weight rows.  The grid is
// (work items rounded up to a multiple of 8 xrun) x nft.
MOEQ_DEV void block_tile(int nft, int xrun, int& w, int& ft) {
  const int b = (int)blockIdx.x, r = b % 8, slot = b / 8;
  const int n = slot / nft;   // this XCD's n-th work item
  w = (n / xrun) * 8 * xrun + r * xrun + n % xrun;
  ft = slot % nft;
}

// Runs of 8 work items per XCD once a batch fills at least this many
// 128-token tiles (fewer items would leave the XCDs' last runs uneven).
constexpr int kXcdRunMinTiles = 64;

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Epilogue staging: the block's output tile goes through LDS as rows of
// bf16 (stride PITCH bytes) so that it leaves in 16-byte stores.
template <int COLS>
struct OutTile {
  static constexpr int PITCH = COLS * 2 + 16;
  static constexpr int BYTES = 128 * PITCH;
};

// Runs fn(std::integral_constant<int, MTA>) for MTA = the M-tiles holding rows.
template <class Fn>
MOEQ_DEV void with_mtiles(int rows, Fn&& fn) {
  switch ((rows + 31) / 32) {
    case 1: fn(std::integral_constant<int, 1>()); break;
    case 2: fn(std::integral_constant<int, 2>()); break;
    case 3: fn(std::integral_constant<int, 3>()); break;
    default: fn(std::integral_constant<int, 4>()); break;
  }
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
                                                             const int32_t* __restrict__ sched, int xrun,
                                                             uint16_t* __restrict__ h) {
  static_assert(BM == 128, "tile");
  using Out = OutTile<128>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[cmax(lds_bytes<BITS, BM>(), Out::BYTES)];
  int wi, ft;
  block_tile(I / 128, xrun, wi, ft);
  if (wi >= sched[0]) return;
  const int e = sched[2 + 2 * wi], mt = sched[3 + 2 * wi];
  const int base = offsets[e] + mt * BM;
  const int rows = min(BM, counts[e] - mt * BM);
  const int lane = threadIdx.x & 63, hh = lane >> 5;
  const int wv = uniform(threadIdx.x >> 6);
  BDma<BITS> bd;
  {
    const uint8_t* const q[2] = {gq, uq};
    const uint32_t* const sz[2] = {gsz, usz};
    const size_t row0 = (size_t)e * I + ft * 128 + 32 * wv;   // gate and up rows of this wavefront
    const size_t row[2] = {row0, row0};
    bd.init(q, sz, row, H);
  }
  with_mtiles(rows, [&](auto mta) {
    constexpr int MTA = decltype(mta)::value;
    using ML = Mainloop<BITS, BM, MTA>;
    typename ML::AD ad;
    {
      const uint16_t* rowp[ML::AD::N];
#pragma unroll
      for (int j = 0; j < ML::AD::N; ++j)
        rowp[j] = x + (size_t)(sorted[base + min(ML::AD::row_of(j), rows - 1)] / kS) * H;
      ad.init(rowp);
    }
    f32x16_t acc[BM / 32][2];
    ML(ad, bd, H / 64, acc, lds).run();
    // h tile -> LDS: lane (l % 32, half hh) holds column 32 wv + l % 32 of
    // rows 32 i + 8 (r / 4) + 4 hh + r % 4
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
        *reinterpret_cast<uint16_t*>(lds + m * Out::PITCH + 2 * (32 * wv + (lane & 31))) =
            (uint16_t)f32_to_bf16_bits(silu_f32(acc[i][0][r]) * acc[i][1][r]);
      }
  });
  __syncthreads();
  // 16 pieces of 16 bytes per row
  for (int c = threadIdx.x; c < 16 * rows; c += 256) {
    const int m = c >> 4, pc = c & 15;
    *reinterpret_cast<moeq_u32x4*>(h + (size_t)(base + m) * I + ft * 128 + 8 * pc) =
        *reinterpret_cast<const moeq_u32x4*>(lds + m * Out::PITCH + 16 * pc);
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
                                                           const int32_t* __restrict__ sched, int xrun,
                                                           uint16_t* __restrict__ y) {
  static_assert(BM == 128, "tile");
  using Out = OutTile<256>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[cmax(lds_bytes<BITS, BM>(), Out::BYTES)];
  int wi, ft;
  block_tile(H / 256, xrun, wi, ft);
  if (wi >= sched[0]) return;
  const int e = sched[2 + 2 * wi], mt = sched[3 + 2 * wi];
  const int base = offsets[e] + mt * BM;
  const int rows = min(BM, counts[e] - mt * BM);
  const int lane = threadIdx.x & 63, hh = lane >> 5;
  const int wv = uniform(threadIdx.x >> 6);
  BDma<BITS> bd;
  {
    const uint8_t* const q[2] = {dq, dq};
    const uint32_t* const sz[2] = {dsz, dsz};
    const size_t row0 = (size_t)e * H + ft * 256 + 64 * wv;   // the wavefront's two 32-row blocks
    const size_t row[2] = {row0, row0 + 32};
    bd.init(q, sz, row, I);
  }
  with_mtiles(rows, [&](auto mta) {
    constexpr int MTA = decltype(mta)::value;
    using ML = Mainloop<BITS, BM, MTA>;
    typename ML::AD ad;
    {
      const uint16_t* rowp[ML::AD::N];
#pragma unroll
      for (int j = 0; j < ML::AD::N; ++j) rowp[j] = h + (size_t)(base + min(ML::AD::row_of(j), rows - 1)) * I;
      ad.init(rowp);
    }
    f32x16_t acc[BM / 32][2];
    ML(ad, bd, I / 64, acc, lds).run();
#pragma unroll
    for (int i = 0; i < MTA; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
        uint8_t* o = lds + m * Out::PITCH + 2 * (64 * wv + (lane & 31));
        *reinterpret_cast<uint16_t*>(o) = (uint16_t)f32_to_bf16_bits(acc[i][0][r]);
        *reinterpret_cast<uint16_t*>(o + 64) = (uint16_t)f32_to_bf16_bits(acc[i][1][r]);
      }
  });
  __syncthreads();
  // 32 pieces of 16 bytes per row, each row to its assignment
  for (int c = threadIdx.x; c < 32 * rows; c += 256) {
    const int m = c >> 5, pc = c & 31;
    *reinterpret_cast<moeq_u32x4*>(y + (size_t)sorted[base + m] * H + ft * 256 + 8 * pc) =
        *reinterpret_cast<const moeq_u32x4*>(lds + m * Out::PITCH + 16 * pc);
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

// Router logits for large batches and expert counts: 128 x BN output tiles
// (BN 128, or 64 where 128-wide tiles would leave CUs with one block), both
// operands staged through double-buffered LDS tiles in K-slices of 64;
// wavefront (wm, wn) owns a (128 / WM) x 64 sub-tile.  Every output element
// is summed over the K-slices in ascending order whatever BN is.  Rows past
// M or N read row M - 1 or N - 1 and are not stored.
template <int BN>
__global__ __launch_bounds__(256) void gemm_nt_tiled_kernel(const uint16_t* __restrict__ A,
                                                            const uint16_t* __restrict__ B,
                                                            const float* __restrict__ bias, int M, int N, int K,
                                                            float* __restrict__ C) {
  constexpr int WN = BN / 64, WM = 4 / WN, MI = 128 / WM / 32;
  __shared__ __attribute__((aligned(16))) uint16_t As[2][128 * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * kLds];
  const int m0 = blockIdx.x * 128, n0 = blockIdx.y * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave / WN, wn = wave % WN, hh = lane >> 5;
  const uint16_t* arow[ATile<128>::N];
  const uint16_t* brow[ATile<BN>::N];
#pragma unroll
  for (int j = 0; j < ATile<128>::N; ++j) {
    const int r = (threadIdx.x >> 3) + 32 * j;
    arow[j] = A + (size_t)min(m0 + r, M - 1) * K;
  }
#pragma unroll
  for (int j = 0; j < ATile<BN>::N; ++j) {
    const int r = (threadIdx.x >> 3) + 32 * j;
    brow[j] = B + (size_t)min(n0 + r, N - 1) * K;
  }
  f32x16_t acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) { acc[i][0][r] = 0.0f; acc[i][1][r] = 0.0f; }
  // K-slices reach registers two slices ahead of their LDS store: at the
  // start of slice s, LDS[s & 1] holds slice s, ra/rb[(s + 1) & 1] slice
  // s + 1 and ra/rb[s & 1] slice s + 2 (loads in flight or arrived).  Past
  // the end the last slice is loaded and stored again (never read), so that
  // every load and store is unconditional and the compiler's counts of the
  // loads in flight are exact: a slice's stores wait only for its own loads.
  ATile<128> ra[2];
  ATile<BN> rb[2];
  const int ns = K / 64;
  ra[0].load(arow, 0);
  rb[0].load(brow, 0);
  ra[0].store(As[0]);
  rb[0].store(Bs[0]);
  ra[1].load(arow, min(1, ns - 1) * 64);
  rb[1].load(brow, min(1, ns - 1) * 64);
  ra[0].load(arow, min(2, ns - 1) * 64);
  rb[0].load(brow, min(2, ns - 1) * 64);
  auto step = [&](int s, ATile<128>& na, ATile<BN>& nb) {   // na, nb: slice s + 1
    __syncthreads();
    const uint16_t* a_s = As[s & 1] + (32 * MI * wm + (lane & 31)) * kLds + 8 * hh;
    const uint16_t* b_s = Bs[s & 1] + (64 * wn + (lane & 31)) * kLds + 8 * hh;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8_t a[MI], b[2];
#pragma unroll
      for (int i = 0; i < MI; ++i) a[i] = *reinterpret_cast<const bf16x8_t*>(a_s + 32 * i * kLds + 16 * t);
#pragma unroll
      for (int i = 0; i < 2; ++i) b[i] = *reinterpret_cast<const bf16x8_t*>(b_s + 32 * i * kLds + 16 * t);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    na.store(As[(s + 1) & 1]);
    nb.store(Bs[(s + 1) & 1]);
    const int nx = min(s + 3, ns - 1);
    na.load(arow, nx * 64);
    nb.load(brow, nx * 64);
  };
  int s = 0;
  for (; s + 1 < ns; s += 2) {
    step(s, ra[1], rb[1]);
    step(s + 1, ra[0], rb[0]);
  }
  if (s < ns) step(s, ra[1], rb[1]);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + 64 * wn + 32 * j + (lane & 31);
    if (n >= N) continue;
    const float bn = bias ? bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 32 * MI * wm + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
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
#ifndef MOEQ_ROUTER_BN64_BELOW
#define MOEQ_ROUTER_BN64_BELOW 512
#endif
    if (tiles128 < MOEQ_ROUTER_BN64_BELOW) {   // 64-wide tiles: two blocks per CU
      dim3 grid((M + 127) / 128, (N + 63) / 64);
      gemm_nt_tiled_kernel<64><<<grid, 256, 0, stream>>>(A, B, bias, M, N, K, C);
    } else {
      dim3 grid((M + 127) / 128, (N + 127) / 128);
      gemm_nt_tiled_kernel<128><<<grid, 256, 0, stream>>>(A, B, bias, M, N, K, C);
    }
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
  int w_gu, cw_gu, w_dn, cw_dn;
  if (!pick_shape(L->H, L->gate.bits, MOEQ_LIST_GATEUP_RUN, w_gu, cw_gu) ||
      !pick_shape(L->I, L->down.bits, MOEQ_LIST_DOWN_RUN, w_dn, cw_dn))
    return set_error(MOEQ_ERR_UNSUPPORTED, "moe_qgemm_prefill: no GEMV kernel for H=%d/I=%d at these bit widths",
                     L->H, L->I);
  char* w = static_cast<char*>(ws);
  int32_t* sched = reinterpret_cast<int32_t*>(w + wl.sched);
  int32_t* gemv = reinterpret_cast<int32_t*>(w + wl.gemv);
  uint16_t* h = reinterpret_cast<uint16_t*>(w + wl.h);
  const int nexp = L->E + L->S, kS = L->k + L->S;
  const long A = (long)T * kS;
  const long max_tiles = prefill_max_tiles(A, nexp);
  schedule_kernel<<<1, 256, 0, stream>>>(counts, nexp, L->E, sched, gemv);
  if ((rc = check_launch("moe_qgemm_prefill (schedule)")) != MOEQ_OK) return rc;
  const int xrun = A / BM >= kXcdRunMinTiles ? 8 : 1;
  const unsigned nw = (unsigned)((max_tiles + 8 * xrun - 1) / (8 * xrun) * (8 * xrun));   // work items, padded for the XCD mapping
  const unsigned g1 = nw * (unsigned)(L->I / 128), g2 = nw * (unsigned)(L->H / 256);
  switch (L->gate.bits) {
    case 4: mfma_gateup_kernel<4, BM><<<g1, 256, 0, stream>>>(L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, kS, counts, offsets, sorted, sched, xrun, h); break;
    case 6: mfma_gateup_kernel<6, BM><<<g1, 256, 0, stream>>>(L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, kS, counts, offsets, sorted, sched, xrun, h); break;
    default: mfma_gateup_kernel<8, BM><<<g1, 256, 0, stream>>>(L->gate.q, L->gate.sz, L->up.q, L->up.sz, x, L->H, L->I, kS, counts, offsets, sorted, sched, xrun, h); break;
  }
  if ((rc = check_launch("moe_qgemm_prefill (gate/up)")) != MOEQ_OK) return rc;
  switch (L->down.bits) {
    case 4: mfma_down_kernel<4, BM><<<g2, 256, 0, stream>>>(L->down.q, L->down.sz, h, L->H, L->I, counts, offsets, sorted, sched, xrun, y); break;
    case 6: mfma_down_kernel<6, BM><<<g2, 256, 0, stream>>>(L->down.q, L->down.sz, h, L->H, L->I, counts, offsets, sorted, sched, xrun, y); break;
    default: mfma_down_kernel<8, BM><<<g2, 256, 0, stream>>>(L->down.q, L->down.sz, h, L->H, L->I, counts, offsets, sorted, sched, xrun, y); break;
  }
  if ((rc = check_launch("moe_qgemm_prefill (down)")) != MOEQ_OK) return rc;
  // the experts of the GEMV list (shared experts take every token: never on it)
  switch (L->gate.bits) {
    case 4: rc = list_gateup_b4(L, x, offsets, sorted, gemv, w_gu, cw_gu, h, stream); break;
    case 6: rc = list_gateup_b6(L, x, offsets, sorted, gemv, w_gu, cw_gu, h, stream); break;
    default: rc = list_gateup_b8(L, x, offsets, sorted, gemv, w_gu, cw_gu, h, stream); break;
  }
  if (rc != MOEQ_OK) return rc;
  switch (L->down.bits) {
    case 4: rc = list_down_b4(L, h, offsets, sorted, gemv, w_dn, cw_dn, y, stream); break;
    case 6: rc = list_down_b6(L, h, offsets, sorted, gemv, w_dn, cw_dn, y, stream); break;
    default: rc = list_down_b8(L, h, offsets, sorted, gemv, w_dn, cw_dn, y, stream); break;
  }
  return rc;
}
