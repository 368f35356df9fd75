/*
 * moeq.h -- C ABI of libmoeq, the forward pass of a Mixture-of-Experts FFN
 * layer whose expert weights are low-bit group-quantised, on AMD MI355X
 * (gfx950).
 *
 * The layer: router logits -> top-k routing with renormalised softmax
 * weights -> grouping of (token, expert) assignments by expert -> per expert
 * a SwiGLU FFN, h = silu(Wg x) * (Wu x), y = Wd h, with weights dequantised
 * on the fly as (q - z) * s -> routing-weighted combine.  Prefill and decode
 * are separate code paths (Krasis update, "Overview"): decode is a grouped
 * GEMV over only the routed experts' weights, prefill a grouped GEMM over
 * expert-sorted tokens (Qwen-tin, "Memory layout and performance": a long
 * prompt touches nearly every expert).  Expert weights are HQQ-style 4-, 6-
 * or 8-bit codes (Krasis update, "Latest results (v1.0)").
 *
 * Conventions for every entry point
 *   - Pointers marked "device" point to GPU memory that the caller allocated
 *     and owns; the library keeps no pointer after the call returns.  It
 *     allocates no memory: scratch space comes in through a caller-owned
 *     workspace whose size moe_workspace_bytes() reports.
 *   - All GPU work is enqueued on the caller's stream; no call synchronises
 *     or copies data to the host, except moe_read_status().
 *   - bf16 and fp16 values travel as uint16_t bit patterns.
 *   - Arguments are validated on the host before anything is enqueued.  On
 *     error nothing is enqueued, a negative MOEQ_ERR_* code is returned and
 *     moe_last_error() (thread-local) describes the problem.  No exception
 *     crosses the ABI and the library never aborts the process.
 *   - Calls that share a workspace must not run concurrently.
 *   - Weights/activations pointers (q, sz, x) must be 16-byte aligned.
 */
#ifndef MOEQ_H
#define MOEQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

#define MOEQ_OK               0
#define MOEQ_ERR_INVALID_ARG (-1)  /* null pointer, bad size, k > E, ...        */
#define MOEQ_ERR_UNSUPPORTED (-2)  /* bits not in {4,6,8}, K not a multiple of 64, shape without a kernel */
#define MOEQ_ERR_MISALIGNED  (-3)  /* a pointer that must be 16-byte aligned is not */
#define MOEQ_ERR_WORKSPACE   (-4)  /* workspace missing or smaller than required */
#define MOEQ_ERR_HIP         (-5)  /* a HIP runtime call failed (launch, memcpy) */

#define MOEQ_GROUP 64              /* quantisation group along the input dim  */

/* One quantised projection of all experts.  For a projection mapping K inputs
 * to N outputs (N a multiple of 64), expert e's weight is an N x K matrix; the
 * rows r = e*N + n of all experts are stored together:
 *   q  bytes, K*bits/8 per row as in plain packing, laid out in tiles of 64
 *      rows.  A "chunk" is 32 codes in 16 bytes (4-bit), 16 codes in 12 bytes
 *      (6-bit) or 16 codes in 16 bytes (8-bit); chunk c of row r starts at
 *      byte ((r / 64) * CPR + c) * 64 * BYTES + (r % 64) * BYTES, CPR =
 *      K / codes-per-chunk, BYTES = bytes per chunk.  Inside a chunk, field n
 *      (4-bit: nibble n = low nibble of byte n/2 for even n, high for odd;
 *      6-bit: bits 6n..6n+5 of the 96-bit little-endian chunk; 8-bit: byte
 *      n) holds code F(n) of the chunk:
 *        4-bit: F(n) = 8*(n/8) + 2*(n%4) + (n/4)%2
 *        6-bit: F(0..15) = 0 2 12 1 3 4 6 13 5 7 8 10 14 9 11 15
 *        8-bit: F(n) = n
 *   sz uint32 words: bits 0-15 the fp16 scale s, bits 16-31 the fp16 zero z
 *      of group g (64 consecutive inputs) of row r, at word
 *      ((r / 64) * (K / 64) + g) * 64 + r % 64.
 * A wavefront whose lane l handles row 64 t + l thus reads every chunk as one
 * contiguous block, and the field order turns every two consecutive codes
 * into a bf16 pair with one AND-OR.  moe_quantize writes this layout and
 * moe_unpack reads it.  The dequantised weight is (q - z) * s, in fp32. */
typedef struct moe_qweight {
  const uint8_t*  q;    /* device */
  const uint32_t* sz;   /* device */
  int             bits; /* 4, 6 or 8 */
} moe_qweight;

/* One MoE layer: E routed experts (ids 0..E-1) and S always-on shared experts
 * (ids E..E+S-1), each a SwiGLU FFN with hidden size H and intermediate size
 * I; k experts are routed per token.  gate and up map H -> I (N = I, K = H),
 * down maps I -> H (N = H, K = I); n_mats = E + S.  The three projections may
 * use different bit widths.
 * An assignment is one (token, slot) pair: a = t*(k+S) + j, where slots
 * j < k are the token's routed experts in routing order and slots j >= k
 * its shared experts (weight one).
 * Every call taking a descriptor requires H and I multiples of 64,
 * E + S <= 4096 and H * I < 2^31 (MOEQ_ERR_UNSUPPORTED otherwise). */
typedef struct moe_layer_desc {
  int H, I, E, S, k;
  moe_qweight gate, up, down;
} moe_layer_desc;

/* Size in bytes of the workspace the calls below need for batches of up to
 * T_max tokens of layer L (decode and prefill alike).  0 if L is invalid.
 * The workspace must be zero-filled before its first use; the library keeps
 * the control words it relies on at zero between calls. */
size_t moe_workspace_bytes(const moe_layer_desc* L, int T_max);

/* Byte offset, in a workspace of moe_workspace_bytes(L, T_max) bytes, of the
 * intermediate h = silu(Wg x) * (Wu x) the expert calls leave there: bf16
 * [T*(k+S)][I], rows in expert-sorted order (the order of moe_permute's
 * sorted) after moe_qgemv_decode and moe_qgemm_prefill, in assignment order
 * after moe_decode_forward.  h is what the two projections of a SwiGLU expert
 * hand each other (Raon-1-mini, optimisation table: the projections that share
 * an input run together, the down projection waits for their result); the
 * call exists to inspect it.  Valid until the next call on the workspace. */
int moe_workspace_h(const moe_layer_desc* L, int T_max, size_t* offset);

/* Description of the last error raised on this thread ("" if none). */
const char* moe_last_error(void);

/* ------------------------------------------------------------------------
 * Quantisation format (the step before the forward path)
 * ------------------------------------------------------------------------ */

/* Quantise fp32 weights w [rows][K] (device, rows = n_mats*N) into codes and
 * fp16 scale/zero per group of 64 along K, min-max affine (the starting point
 * of HQQ; Krasis update, "Latest updates", names HQQ 4/6/8-bit weights), in
 * fp32 with IEEE division and round-to-nearest-even:
 *   s16 = fp16(fp32(max - min) / (2^bits - 1)),  z16 = fp16(-min / s16),
 *   q   = clamp(rint(w / s16 + z16), 0, 2^bits - 1).
 * A group whose s16 is zero stores s16 = 1, z16 = fp16(-min), q = 0.
 * Writes q (rows*K*bits/8 bytes) and sz (rows*K/64 words) in the layout of
 * moe_qweight (device); rows must be a multiple of 64.  w must be 16-byte
 * aligned; w must hold finite values. */
int moe_quantize(const float* w, long rows, int K, int bits,
                 uint8_t* q, uint32_t* sz, hipStream_t stream);

/* Pack codes (host, one byte per code, codes [N][K], each < 2^bits) into the
 * plain row form an offline quantiser stores (host, packed [N][K*bits/8]):
 *   4-bit: byte i of a row = code 2i | code 2i+1 << 4 (two nibbles a byte);
 *   6-bit: bytes 3i..3i+2 = the 24-bit little-endian word
 *          code 4i | code 4i+1 << 6 | code 4i+2 << 12 | code 4i+3 << 18
 *          (groups of four values in three bytes);
 *   8-bit: one byte per code.
 * HQQ weights are made once by a preprocessing stage before the hot path
 * (Krasis update, "Latest updates"); this is their storage form.  K must be
 * a multiple of 4; a code >= 2^bits is MOEQ_ERR_INVALID_ARG (nothing past
 * the check is written).  Host memory only; no GPU work. */
int moe_pack(const uint8_t* codes, long N, int K, int bits, uint8_t* packed);

/* Lay weights in moe_pack's plain form (device packed [rows][K*bits/8]) with
 * their fp16 scales and zeros (device scale [rows][K/64], zero [rows][K/64],
 * group g = inputs 64g .. 64g+63 of a row) out into the layout of
 * moe_qweight (device q, rows*K*bits/8 bytes, and sz, rows*K/64 words;
 * 16-byte aligned).  The dequantised weight of the result is
 * (code - zero) * scale exactly as given: this is how weights quantised
 * elsewhere (HQQ assets, Krasis update, "Latest updates") enter the forward
 * path.  rows and K multiples of 64; the inputs need no alignment beyond
 * their element types.  Enqueued on stream; allocates nothing. */
int moe_qweight_load(const uint8_t* packed, const uint16_t* scale, const uint16_t* zero, long rows, int K,
                     int bits, uint8_t* q, uint32_t* sz, hipStream_t stream);

/* moe_quantize followed by HQQ's zero-point refinement of every group, the
 * half-quadratic solver of Badri & Shaji ("Half-Quadratic Quantization of
 * Large Machine Learning Models", 2023) with the scale held (the pages name
 * HQQ weights -- Krasis update, "Latest results (v1.0)" -- but no solver).
 * Per group, from the min-max zero z (an fp16 value), up to iters rounds of:
 *   q = clamp(rint(w / s16 + z), 0, 2^bits - 1)      (fp32, as moe_quantize)
 *   r = w - (q - z) * s16;  E = mean |r|;  stop if E is not below the
 *   group's best, else keep z as its best;
 *   e = sign(r) * max(|r| - |r|^(lp - 1) / beta, 0);
 *   z = fp16(mean(q - (w - e) / s16));  beta = beta * kappa;
 * then the kept z and its codes are stored, so a group's mean absolute error
 * never exceeds the min-max one.  r is exact in fp64; E, e and the zero
 * update are evaluated in fp64 (lp, beta and kappa taken as given, in fp32)
 * and a mean is the fp64 sum over 64, rounded once to fp16 for z: the stored
 * zero does not depend on the order of the additions.  The stopping test is
 * per group (the objective is a sum over groups with disjoint variables).
 * Groups whose fp16 scale is zero keep the min-max result.  lp in (0, 1]
 * (0.7 and 1 are the usual choices), beta > 0, kappa >= 1, 0 <= iters <=
 * 1000 (0 gives moe_quantize's result); other arguments, layout and errors
 * as moe_quantize. */
int moe_quantize_hqq(const float* w, long rows, int K, int bits,
                     float lp, float beta, float kappa, int iters,
                     uint8_t* q, uint32_t* sz, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Stacked decode in one launch (Raon-1-mini, optimisation table: a persistent
 * per-layer MoE megakernel instead of many small launches)
 * ------------------------------------------------------------------------ */

/* Bytes of the device table moe_stack_table_write fills for nlayers layers:
 * a 64-byte header (layer count, H, I, E, k) and 64 bytes per layer; 0 if
 * nlayers <= 0. */
size_t moe_stack_table_bytes(int nlayers);

/* Write the device table of nlayers MoE layers (host array layers[], each
 * with its own weights and bit widths but the same H, I, E, k and S = 0;
 * gate and up of a layer share a bit width) and their bf16 router weights
 * (host array of device pointers w_router[l], [E][H], 16-byte aligned) into
 * table (device, table_bytes >= moe_stack_table_bytes(nlayers), 16-byte
 * aligned).  A setup call: it copies synchronously (hipMemcpy).  The weights
 * must stay allocated while the table is used. */
int moe_stack_table_write(const moe_layer_desc* layers, const uint16_t* const* w_router, int nlayers,
                          void* table, size_t table_bytes);

/* Workspace bytes moe_stack_decode needs for layers of the dimensions of L
 * on the current device (it depends on the device's CU count); 0 if L is
 * not supported (H a multiple of 512 up to 8192, I a multiple of 64 with
 * k * I <= 16384, k <= 16, k <= E <= 1024, S = 0).  Zero-fill it once. */
size_t moe_stack_workspace_bytes(const moe_layer_desc* L);

/* One batch-1 token through the first nlayers layers of table (the layer
 * sequence of a model's decode step, each block RMSNorm -> MoE -> residual;
 * Raon-1-mini, optimisation table: a persistent per-layer MoE megakernel
 * instead of many small launches): for each layer, n = RMSNorm(x) (as
 * moe_rmsnorm, gamma = 1, eps), routed MoE of n (top-k, renormalised
 * weights, SwiGLU experts with h rounded to bf16, fp32 accumulation),
 * x = bf16(x + bf16(moe)).  x: device bf16 [H], updated in place.  dims: any
 * layer's descriptor (only H, I, E, k, S are read); table_bytes: the size
 * of table; nlayers <= 1024.  A one-thread kernel that advances the
 * workspace's call number, then one cooperative launch whose wavefronts
 * hand values to each other through tagged words in the workspace (no
 * barriers); it fails (MOEQ_ERR_HIP) if the device cannot hold the grid at
 * once.  The kernel checks the table's header against dims and nlayers and,
 * on a mismatch, leaves x untouched and sets bit 2 of the workspace's error
 * word; a wait that polls for a fraction of a second gives up and sets bit 1
 * (x is then wrong).  Read the word with moe_stack_read_status.  Calls that
 * share a workspace must not overlap; a workspace serves one set of
 * dimensions.
 * Each row's K sum is split over the lanes and wavefronts of one
 * workgroup and the down rows take their k slots' weighted sums together,
 * in a fixed order, so results equal moe_rmsnorm + moe_decode_forward to
 * rounding, not bit for bit, and are the same from run to run. */
int moe_stack_decode(const moe_layer_desc* dims, const void* table, size_t table_bytes, int nlayers, float eps,
                     uint16_t* x, void* ws, size_t ws_bytes, hipStream_t stream);

/* Synchronise `stream` and return in *err the error word of a
 * moe_stack_decode workspace (0: no error since the last read; bit 1: a
 * wait gave up; bit 2: the table did not match) and clear it.  The next call
 * needs no other reset: it waits for words tagged with its own call number.
 * dims as for moe_stack_workspace_bytes. */
int moe_stack_read_status(void* ws, size_t ws_bytes, const moe_layer_desc* dims, int* err, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Group-quantised KV cache (the same codec on cache rows; Krasis update,
 * "Latest updates", keeps the KV cache in 4- and 6-bit form)
 * ------------------------------------------------------------------------ */

/* Encode bf16 cache rows x [rows][D] (device; one row = one token's vector of
 * one head, D a multiple of 64) group by group with moe_quantize's min-max
 * formulas (on the exact fp32 values of the bf16 inputs).  Writes, row after
 * row, the packed codes in natural order into q [rows][D*bits/8] (4-bit: code
 * 2i in the low nibble of byte i; 6-bit: code c at bits 6c..6c+5 of the row's
 * little-endian bit string; 8-bit: one byte per code) and the scale/zero
 * words (fp16 s | fp16 z << 16) into sz [rows][D/64].  x and q must be
 * 16-byte aligned, sz 4-byte aligned; rows >= 0; bits in {4,6,8}.  x must
 * hold finite values. */
int moe_kv_encode(const uint16_t* x, long rows, int D, int bits,
                  uint8_t* q, uint32_t* sz, hipStream_t stream);

/* Decode what moe_kv_encode wrote: out[r][i] = bf16((q - z) * s) with the
 * difference and the product each rounded in fp32 (no fused multiply-add) and
 * the result rounded to bf16, ties to even.  q and out 16-byte aligned, sz
 * 4-byte aligned; sizes as moe_kv_encode. */
int moe_kv_decode(const uint8_t* q, const uint32_t* sz, long rows, int D, int bits,
                  uint16_t* out, hipStream_t stream);

/* Unpack codes q (rows*K*bits/8 bytes in the layout of moe_qweight, rows a
 * multiple of 64, device) into one byte per code, codes [rows][K] (device,
 * natural order): the inverse of the packing (two nibbles a byte at 4 bits,
 * four values in three bytes at 6 bits; Krasis update, "Latest results
 * (v1.0)": HQQ 4/6/8-bit weights).  It runs the same in-register unpacking
 * the decode kernels use, so it tests their view of the format bit for
 * bit. */
int moe_unpack(const uint8_t* q, long rows, int K, int bits,
               uint8_t* codes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The five steps of the forward pass
 * ------------------------------------------------------------------------ */

/* Router and top-k routing.
 * If w_router (device, bf16 [E][H]) is non-NULL: logits[t][e] =
 * fp32(sum_h x[t][h]*w_router[e][h]) + bias[e] (bias device fp32 [E], may be
 * NULL), accumulated in fp32, written to logits (device fp32 [T][E]).
 * If w_router is NULL, logits is read as given (bias must be NULL) and x may
 * be NULL.  Then, per token, the k largest logits are selected -- larger
 * first, equal values lower expert index first, -0.0 equal to +0.0 -- into
 * topk_idx (device int32 [T][k]), and topk_w (device fp32 [T][k]) receives a
 * softmax over the selected logits, i.e. the softmax over all experts kept on
 * the selected k and renormalised (Qwen 3.8 Flash Next on an RTX 3060,
 * introduction: top-10 of 512 experts).  Logits must not be NaN.
 * 1 <= k <= E <= 4096; T >= 0 (T = 0 enqueues nothing). */
int moe_route_topk(const uint16_t* x, const uint16_t* w_router, const float* bias,
                   int T, int H, int E, int k,
                   float* logits, int32_t* topk_idx, float* topk_w,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Group the T*(k+S) assignments by expert: histogram, exclusive scan and a
 * stable scatter, so that each expert's tokens are contiguous for its GEMV
 * or GEMM (a prefill chunk spreads over nearly every expert -- Qwen-tin,
 * "Memory layout and performance" -- and each expert's weights are then
 * read once per token tile).  Outputs (device int32):
 *   counts  [E+S]    assignments per expert,
 *   offsets [E+S+1]  exclusive prefix sum of counts,
 *   sorted  [T*(k+S)] assignment ids grouped by expert, ascending within one,
 *   inverse [T*(k+S)] position of each assignment in sorted,
 *   active  [E+S+1]  active[0] = number of experts with counts > 0,
 *                    active[1..] those expert ids, ascending.
 * Shared-expert slots get ids E..E+S-1.  A routed id outside [0, E) is
 * skipped (its assignment is missing from sorted, its inverse is -1) and
 * counted; moe_read_status() reports the count.  Results are identical from
 * run to run (no atomics decide an order). */
int moe_permute(const int32_t* topk_idx, int T, int k, int E, int S,
                int32_t* counts, int32_t* offsets, int32_t* sorted,
                int32_t* inverse, int32_t* active,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* Decode-batch routing: the results of moe_route_topk (with router weights)
 * followed by moe_permute, bit for bit, from two small launches tuned for
 * latency: a router kernel with one wavefront per router row, then a single
 * block that selects every token's top k and groups the assignments.
 * Removing dependent small launches is the decode lever the pages report
 * (Raon-1-mini on an RTX 5070 Ti, optimisation table).
 * Limits: T*(k+S) <= 1024, E+S <= 1024, k <= 64, H in {512, 1024, 2048,
 * 4096}; MOEQ_ERR_UNSUPPORTED otherwise.  ws: at least 256 bytes (its first
 * word receives the bad-id count, always 0 here). */
int moe_route_permute_decode(const uint16_t* x, const uint16_t* w_router, const float* bias,
                             int T, int H, int E, int k, int S,
                             float* logits, int32_t* topk_idx, float* topk_w,
                             int32_t* counts, int32_t* offsets, int32_t* sorted,
                             int32_t* inverse, int32_t* active,
                             void* ws, size_t ws_bytes, hipStream_t stream);

/* Decode path (small T): for every assignment a, y[a] = Wd h with
 * h = silu(Wg x_t) * (Wu x_t), t = a / (k+S), using expert sorted-order data
 * from moe_permute.  Decode streams only the routed experts' weights, and
 * that stream sets its speed (Raon-1-mini on an RTX 5070 Ti, result
 * paragraph: decode at about two thirds of the card's bandwidth).  Only the experts in `active` are read, each once per
 * batch, as a grouped GEMV: codes are unpacked in registers and dot products
 * accumulated in fp32 with the group scale/zero applied per group in fp32;
 * h is rounded to bf16 between the two projections (as on the prefill path).
 * y is device fp32 [T*(k+S)][H], rows in assignment order.  Intended for
 * T <= 64; correct for any T. */
int moe_qgemv_decode(const moe_layer_desc* L, const uint16_t* x, int T,
                     const int32_t* offsets, const int32_t* sorted,
                     const int32_t* active, float* y,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* The whole decode layer (router, top-k, expert FFNs, combine) in three
 * launches instead of five: router logits; then the gate/up GEMV with one
 * block per (routed assignment, row tile), whose first wavefront makes that
 * token's selection from the logits before the block streams its expert
 * (cheaper than a launch between them); then per token the down GEMVs of
 * its k+S experts and their routing-weighted sum, so the expert outputs
 * stay on chip.  Dependent small launches are the decode cost the pages
 * single out (Raon-1-mini on an RTX 5070 Ti, optimisation table).
 * Results: logits [T][E] fp32 and topk_idx/topk_w [T][k] exactly as
 * moe_route_permute_decode gives them; out [T][H] bf16 as moe_combine gives it
 * from moe_qgemv_decode's y, up to fp32 summation order inside each expert
 * dot product (residual: as in moe_combine; may alias out).
 * x, w_router: device bf16, 16-byte aligned; bias: device fp32 [E] or NULL.
 * ws: moe_workspace_bytes(L, T) bytes (holds h, bf16 [T (k+S)][I]).
 * Limits (MOEQ_ERR_UNSUPPORTED otherwise): T <= 64, E <= 1024, k+S <= 16,
 * H in {512, 1024, 2048, 4096}, I in {256, 512, 768} (and 1024 with 4-bit
 * down weights), gate and up at one bit width. */
int moe_decode_forward(const moe_layer_desc* L, const uint16_t* x, const uint16_t* w_router,
                       const float* bias, int T, const uint16_t* residual, float* logits,
                       int32_t* topk_idx, float* topk_w, uint16_t* out,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_decode_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Its scratch (the h rows and the shared
 * experts' partial sums) is a fixed array of
 * moe_decode_forward_noalloc_max_scratch() bytes (8 MiB) in device memory
 * that each GPU holds from the library's load until the process ends; the
 * call allocates nothing.  Every call on one GPU uses that GPU's one array,
 * so calls that overlap on one GPU (other streams, other threads) race and
 * must be serialised by the caller.  Nothing in the array needs to start at
 * zero: the kernels write all they read.  A layer and batch that need more
 * scratch than the array holds (see moe_workspace_bytes(L, T)) are rejected
 * with MOEQ_ERR_WORKSPACE; T <= 64.  Results, other limits and errors as
 * moe_decode_forward. */
int moe_decode_forward_noalloc(const moe_layer_desc* L, const uint16_t* x, const uint16_t* w_router,
                               const float* bias, int T, const uint16_t* residual, float* logits,
                               int32_t* topk_idx, float* topk_w, uint16_t* out, hipStream_t stream);

/* Bytes of moe_decode_forward_noalloc's static scratch. */
size_t moe_decode_forward_noalloc_max_scratch(void);

/* One block of a stacked decode step (fewer launches per block: Raon-1-mini,
 * optimisation table): x <- x + moe(RMSNorm(x)) in place, for
 * a batch of T <= 64 token rows x (device bf16 [T][H]); the RMSNorm is
 * moe_rmsnorm's (gamma = 1, eps), formed inside the router launch by every
 * router block for itself (so the step is three launches, not four), the
 * normalised rows kept in the workspace for the expert launches; the rest is
 * moe_decode_forward with residual = out = x (shared experts, if any, as
 * whole rows in the gate/up launch).  For S = 0 the result equals
 * moe_rmsnorm followed by moe_decode_forward bit for bit.  Limits, logits,
 * topk_idx, topk_w, workspace and errors as moe_decode_forward; eps >= 0. */
int moe_decode_block(const moe_layer_desc* L, uint16_t* x, const uint16_t* w_router, const float* bias,
                     int T, float eps, float* logits, int32_t* topk_idx, float* topk_w,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Prefill path (large T): the same y as moe_qgemv_decode, computed as a
 * grouped GEMM over expert-sorted tokens on the bf16 matrix cores (a prompt
 * touches nearly every expert: Qwen-tin page, "Memory layout and
 * performance").  Codes and scale/zero words are staged in LDS and
 * dequantised in registers into the MFMA operand: each weight is
 * fp32((q - z) s), rounded once to bf16; products accumulate in fp32; h is
 * rounded to bf16 between the two GEMMs.  When the batch has at least 64
 * routed experts with one or two assignments (the tail a skewed router
 * leaves), those experts are computed by the GEMV kernels of
 * moe_qgemv_decode instead (fp32 weights (q - z) s, h rounded to bf16),
 * which stream their weights once.  y is device bf16
 * [T*(k+S)][H], rows in assignment order.
 * Needs I % 128 == 0 and H % 256 == 0 (MOEQ_ERR_UNSUPPORTED otherwise);
 * counts/offsets/sorted as produced by moe_permute. */
int moe_qgemm_prefill(const moe_layer_desc* L, const uint16_t* x, int T,
                      const int32_t* counts, const int32_t* offsets,
                      const int32_t* sorted, uint16_t* y,
                      void* ws, size_t ws_bytes, hipStream_t stream);

#define MOEQ_Y_F32  0
#define MOEQ_Y_BF16 1
/* Weighted combine: out[t] = sum_{j<k} topk_w[t][j] * y[t*(k+S)+j]
 *                          + sum_{j>=k} y[t*(k+S)+j],
 * summed in fp32 in ascending j: each token's output is its routed experts'
 * outputs weighted by the renormalised routing weights (top-10 of 512
 * experts: Qwen 3.8 Flash Next on an RTX 3060, introduction), plus the
 * always-on shared experts with weight one.  If residual (device bf16 [T][H]) is
 * non-NULL, out[t] = bf16(residual[t] + bf16(sum)) instead of bf16(sum).
 * y is device fp32 or bf16 (y_dtype) [T*(k+S)][H]; out device bf16 [T][H]
 * (may alias residual). */
int moe_combine(const void* y, int y_dtype, const float* topk_w,
                const uint16_t* residual, int T, int k, int S, int H,
                uint16_t* out, hipStream_t stream);

/* RMSNorm of bf16 rows, the normalisation in front of each MoE block of a
 * stacked decode step (the per-layer work a persistent decode kernel runs
 * between blocks: Raon-1-mini, optimisation table):
 * out[t] = bf16(x[t] / sqrt(mean(x[t]^2) + eps) * g),
 * g = gamma (device bf16 [H]) or 1 if gamma is NULL; fp32 arithmetic.
 * x, out device bf16 [T][H]; may not alias. */
int moe_rmsnorm(const uint16_t* x, const uint16_t* gamma, int T, int H, float eps,
                uint16_t* out, hipStream_t stream);

/* Synchronise `stream` and report the number of out-of-range expert ids the
 * last moe_permute on this workspace skipped: the routing step's ids must
 * name one of the E routed experts (top-k over the router's E logits;
 * Qwen 3.8 Flash Next on an RTX 3060, introduction), and the permutation
 * counts any that do not instead of reading out of bounds. */
int moe_read_status(const void* ws, size_t ws_bytes, int* n_bad_ids, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOEQ_H */
