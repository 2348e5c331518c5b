/*
 * moe.h -- C ABI of the routed Mixture-of-Experts feed-forward layer for AMD Instinct MI355X
 * (gfx950).  Four calls make one layer: moe_route -> moe_bucket -> moe_expert_ffn -> moe_combine.
 *
 * Sources (cited by page title and section; the pages print no code):
 *  [NV]  same post and section: NVFP4 also stores E2M1 values, with an E4M3 scale per 16 values
 *        and a second, tensor-wide scale.
 *  [MX]  "DeepSeek-V4-Flash on a four-GPU Ampere workstation" (FreeToken blog post), section
 *        "MXFP4 is not NVFP4, and the difference matters on Ampere": packed E2M1 codes with one
 *        unsigned E8M0 scale per 32 values, decoded weight v(c) * 2^(e-127), 4.25 bits/weight,
 *        decode inside the reduction with FP32 accumulation, row-major banks read with no repack.
 *  [BP]  same post, section "Why it would not run": a partition that cuts an FP4 32-value block
 *        is rejected instead of producing garbage; weights and scale grids are sliced together.
 *  [C31] "Cascadia: Resident 975B MoE Inference on Eleven AI PCs", Sec. 3.1: expert weights are
 *        stored expert by expert; each selected expert is a SwiGLU block (two input projections,
 *        the gated activation, one output projection) whose outputs are summed with the routing
 *        coefficients; the router hands the expert path ids plus coefficients, and shared experts
 *        are selections every row carries after its routed ones.
 *  [C32] Cascadia Sec. 3.2: a layer call supplies rows, expert ids and routing weights; the
 *        expert path returns FP32 output (Fig. 2).
 *  [C33] Cascadia Sec. 3.3, Eq. 1: range management across the FP16/FP32 boundary -- a per-layer
 *        power-of-two attenuation of the up projection and a per-row power-of-two factor on the
 *        routing weights, both undone in FP32.
 *  [C34] Cascadia Sec. 3.4, Eq. 2: a dense FFN is the sum of its all-active, unit-weight slices,
 *        cut at quantisation-group boundaries.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers of the current HIP device unless a comment says "host".
 *    The caller owns and allocates every buffer; the library never allocates, frees or keeps
 *    device memory, and keeps no state between calls.
 *  - Calls only validate arguments on the host and enqueue work on `stream` (a hipStream_t, or
 *    NULL for the default stream); they never synchronise and never read device memory on the
 *    host.  Results are ready when the stream has reached that point.
 *  - Validation happens before anything is enqueued; on any error nothing is launched and the
 *    status says why.  T == 0 returns MOE_OK without touching any pointer.
 *  - Inputs are read-only; outputs are overwritten (never accumulated into); buffers must not
 *    alias each other.  Calls that share no output buffer may run concurrently on different
 *    streams.
 *  - Results are deterministic: the same inputs give bit-identical outputs on every run (no
 *    floating-point atomics anywhere).
 */
#ifndef MOE_H
#define MOE_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2
#define MOE_MAX_EXPERTS 1024  /* routed experts E, and buckets / experts E' of the later calls */
#define MOE_MAX_SLOTS_PER_TOKEN 256  /* top_k + n_shared */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,      /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,     /* a size is negative, zero where it must not be, or beyond a limit */
  MOE_ERR_BLOCK = 3,     /* an MXFP4 dimension, slice base or stride cuts a 32-value block [BP] */
  MOE_ERR_ALIGN = 4,     /* a pointer or byte stride is not aligned (activations, outputs, FP16) */
  MOE_ERR_DTYPE = 5,     /* an unknown enum value, or an activation dtype the format cannot take */
  MOE_ERR_TOPK = 6,      /* top_k < 1 or top_k > E */
  MOE_ERR_WORKSPACE = 7, /* workspace NULL or smaller than the size query returns */
  MOE_ERR_HIP = 8        /* a kernel launch failed (the HIP error is lost; nothing else ran) */
} moe_status;

typedef enum { MOE_ACT_BF16 = 0, MOE_ACT_FP16 = 1 } moe_act_dtype;
typedef enum { MOE_W_MXFP4 = 0, MOE_W_FP16 = 1, MOE_W_INT4_G32 = 2, MOE_W_NVFP4 = 3 } moe_w_format;

/* One projection of every expert: logical [n_experts][N][K], K contiguous within a row [MX].
 *  MXFP4: `w` holds two E2M1 codes per byte, element k of a row in byte k/2 with even k in the
 *         low nibble (bits 3..0) and odd k in the high nibble; bit 3 of a code is its sign.
 *         `scales` holds one E8M0 byte per 32 elements: scale of element k at byte k/32 of the
 *         row.  Decoded weight = v(code) * 2^(scale - 127) [MX].  Scale codes 0..252 are
 *         supported (every decoded value is then finite in fp32 and bf16); at 253 and 254 the
 *         largest magnitudes overflow bf16, and 255 is outside the contract.
 *  FP16:  `w` holds IEEE binary16 values; `scales` must be NULL.
 *  INT4_G32 [C31] (Cascadia Sec. 3.1 and 3.5): `w` holds unsigned 4-bit codes packed as for
 *         MXFP4; group g = k/32 of a row has a binary16 scale (little-endian bytes 2g, 2g+1 of the
 *         scale row) and an unsigned 4-bit zero point (zero row byte g/2, even g in the low
 *         nibble); decoded weight = (code - zero) * scale (4.625 bits per weight).
 *  NVFP4 [NV] (FreeToken post, "MXFP4 is not NVFP4"): `w` holds E2M1 codes packed as for MXFP4;
 *         block b = k/16 has an E4M3 scale byte (byte b of the scale row; the two NaN codes are
 *         outside the contract) and every expert one fp32 tensor scale; decoded weight =
 *         v(code) * e4m3(scale) * tensor_scale[e] (4.5 bits per weight plus the tensor scale).
 *  INT4_G32 and NVFP4 run on the K-split kernels with bf16 activations; their weights are exact
 *  MFMA operands (INT4 as a bf16 high + low pair, NVFP4 in one bf16), the NVFP4 tensor scale
 *  multiplies the fp32 sums.
 *  Strides are in bytes between consecutive experts / rows, so a projection may be a slice of a
 *  larger matrix [C34] -- e.g. columns [j*I, (j+1)*I) of a dense [H][8*I] down projection have
 *  w = base + j*I*(bytes per element), w_expert_stride = I*(bytes per element),
 *  w_row_stride = 8*I*(bytes per element).  w, w_expert_stride and w_row_stride must be
 *  multiples of 16 bytes: for MXFP4 that is exactly one 32-code block, so a base or stride off
 *  that grid would start inside a block and is refused with MOE_ERR_BLOCK [BP]; for FP16 it is
 *  the 128-bit load alignment (MOE_ERR_ALIGN).  Scale pointers and strides have no alignment rule. */
typedef struct {
  const void *w;
  const uint8_t *scales;
  int64_t w_expert_stride, w_row_stride;
  int64_t s_expert_stride, s_row_stride;
  const uint8_t *zeros;        /* INT4_G32 zero points (NULL for the other formats) */
  int64_t z_expert_stride, z_row_stride;
  const float *tensor_scale;   /* NVFP4: [n_experts] fp32 (NULL for the other formats) */
} moe_proj;

/* All expert weights of a layer [C31].  gate and up: N = inter, K = hidden; down: N = hidden,
 * K = inter.  n_experts = E' = routed + shared experts (one bucket each).  hidden and inter must
 * be positive multiples of 32.  The struct itself is a HOST struct holding device pointers. */
typedef struct {
  moe_w_format fmt;
  int n_experts;
  int hidden;
  int inter;
  moe_proj gate, up, down;
} moe_expert_weights;

/* ---------------------------------------------------------------------------------------------
 * moe_route -- router logits, softmax, top-k, renormalised weights, shared slots.
 *
 * Per token t (reading of [C31]; the pages print no softmax router, the order below is the
 * method's statement): L[t,e] = sum_h x[t,h] * w_router[e,h] + logit_bias[e] (fp32 accumulation),
 * p = softmax(L[t,:]); the top_k experts by (L descending, index ascending) -- i.e. by p with the
 * lowest index winning exact ties -- fill slots j = 0..top_k-1 in that order with
 * weights[t,j] = p_j / sum_{j'<top_k} p_j'; slots top_k .. top_k+n_shared-1 get the shared
 * experts E .. E+n_shared-1 with weight 1.0.
 *   x          [T][H] bf16 or fp16 (x_dtype), rows contiguous, 16-byte aligned
 *   w_router   [E][H] fp32 (4-byte aligned, like every int32/fp32 array below)
 *   logit_bias [E] fp32 added to the logits before the softmax, or NULL
 *   ids        [T][top_k+n_shared] int32 out;  weights [T][top_k+n_shared] fp32 out
 *   probs      [T][E] fp32 out (the full softmax), or NULL
 *   workspace  moe_route_workspace_bytes(T, H, E) bytes, 16-byte aligned (NULL if that is 0)
 * Errors: NULL, SHAPE (T<0, H<1, E<1, E>MOE_MAX_EXPERTS, n_shared<0), TOPK (also
 * top_k+n_shared > MOE_MAX_SLOTS_PER_TOKEN), DTYPE, ALIGN, WORKSPACE, HIP. */
size_t moe_route_workspace_bytes(int T, int H, int E);
moe_status moe_route(const void *x, moe_act_dtype x_dtype, int T, int H, const float *w_router,
                     const float *logit_bias, int E, int top_k, int n_shared, int32_t *ids,
                     float *weights, float *probs, void *workspace, size_t workspace_bytes,
                     void *stream);

/* moe_route_sigmoid -- the sigmoid router of [C31] (Cascadia Sec. 3.1: sigmoid scores, a
 * bias-adjusted top-k selection, normalisation of the selected weights and a model scale factor;
 * the page names these steps without formulas, and the plainest forms are taken):
 *   L[t,e] = sum_h x[t,h] * w_router[e,h] (fp32 accumulation), s[t,e] = 1 / (1 + e^-L[t,e]);
 *   the top_k experts by (s[t,e] + selection_bias[e] descending, index ascending) fill slots
 *   j = 0..top_k-1 in that order with weights[t,j] = routed_scale * s_j / sum_{j'<top_k} s_j'
 *   (the bias moves the selection only, never a weight); slots top_k .. top_k+n_shared-1 hold
 *   the shared experts E .. E+n_shared-1 with weight shared_weight (Cascadia's rows carry six
 *   routed and two shared selections, ids 256 and 257).
 *   scores [T][E] fp32 out (the sigmoid scores s), or NULL; other arguments as for moe_route,
 *   with the same workspace size.
 * Errors: as moe_route, and SHAPE for a non-finite routed_scale or shared_weight. */
moe_status moe_route_sigmoid(const void *x, moe_act_dtype x_dtype, int T, int H, const float *w_router,
                             const float *selection_bias, int E, int top_k, int n_shared,
                             float routed_scale, float shared_weight, int32_t *ids, float *weights,
                             float *scores, void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Fixed row shapes [C32] (Cascadia Sec. 3.2: a call's rows are run at one of the row shapes the
 * compiled layer supports, the extra rows padded with zero routing weights, and only the real
 * rows are handed back).  Here a row shape is a T for which the caller has buffers (and, say, a
 * captured HIP graph of the layer's calls); the real row count n lives in device memory, so one
 * graph serves every n up to its shape:
 *   moe_route(..., T_shape, ...) -> moe_pad_rows(n_rows, T_shape, ...) -> moe_bucket ->
 *   moe_expert_ffn -> moe_combine, then read rows [0, n) of y.
 *
 * moe_row_shape (host): the smallest entry of shapes[0 .. n_shapes) that is >= T (entries <= 0
 * are ignored; the array need not be sorted); -1 when none is, or for T < 0, shapes NULL or
 * n_shapes < 1. */
int moe_row_shape(int T, const int *shapes, int n_shapes);
/* moe_pad_rows: with n = *n_rows (a device int32, clamped to [0, T_shape]), every slot of rows
 * t >= n gets weights[t,j] = 0 and ids[t,j] = -1 -- the invalid id makes moe_bucket drop it, so no
 * expert runs on padding.  Rows < n are untouched.  Padding changes no real row's result: every
 * kernel computes each token from its own x row and weights only (the rows past n of y_slots and
 * y are left unspecified).  ids, weights [T_shape][k_total] in/out.
 * Errors: NULL, SHAPE (T_shape < 0, k_total outside [1, MOE_MAX_SLOTS_PER_TOKEN]), ALIGN, HIP. */
moe_status moe_pad_rows(const int32_t *n_rows, int T_shape, int k_total, int32_t *ids, float *weights,
                        void *stream);

/* ---------------------------------------------------------------------------------------------
 * moe_route_bucket -- moe_route, then moe_bucket of its ids over n_buckets = E + n_shared, then
 * (W non-NULL) moe_expert_ffn_plan into ffn_workspace, with the same results bit for bit: for
 * T <= 8 in two launches instead of four (one workgroup selects, buckets and writes the tile
 * table), up to 2048 slots in three (the bucketing workgroup also writes the tile table), beyond
 * that as the separate kernels.  Arguments as for those calls; W->n_experts must
 * equal E + n_shared; ffn_workspace then is the workspace that the following
 * moe_expert_ffn_gateup / moe_expert_ffn_down calls use.  workspace:
 * moe_route_bucket_workspace_bytes(T, H, E, top_k, n_shared) bytes, 16-byte aligned (it holds
 * the router's partial sums and the bucketing's scratch).
 * Errors: as for the three calls. */
size_t moe_route_bucket_workspace_bytes(int T, int H, int E, int top_k, int n_shared);
moe_status moe_route_bucket(const void *x, moe_act_dtype x_dtype, int T, int H, const float *w_router,
                            const float *logit_bias, int E, int top_k, int n_shared, int32_t *ids,
                            float *weights, float *probs, int32_t *counts, int32_t *offsets,
                            int32_t *sorted_slot, int32_t *slot_pos, const moe_expert_weights *W,
                            void *ffn_workspace, size_t ffn_workspace_bytes, void *workspace,
                            size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * moe_bucket -- group slots by expert (the fused path runs only the selected experts' work
 * [C31]).  Slot s = t*k_total + j.
 *   counts[b]      number of slots with ids[s] == b                         ([n_buckets])
 *   offsets[b]     exclusive prefix sum of counts; offsets[n_buckets] = number of valid slots
 *   sorted_slot[r] slot indices bucket by bucket, ascending slot index within a bucket (stable)
 *   slot_pos[s]    inverse permutation: sorted_slot[slot_pos[s]] == s           (or NULL)
 * A slot whose id is outside [0, n_buckets) is dropped: slot_pos = -1 and it is not counted;
 * entries of sorted_slot past offsets[n_buckets] are -1.  (Ids live on the device, so this is
 * the only possible check; the expert FFN then leaves that slot's y_slots row unwritten.)
 *   workspace  moe_bucket_workspace_bytes(n_slots, n_buckets) bytes (NULL if that is 0)
 * Errors: NULL, SHAPE (n_slots<0, n_buckets<1 or >MOE_MAX_EXPERTS), ALIGN, WORKSPACE, HIP. */
size_t moe_bucket_workspace_bytes(int n_slots, int n_buckets);
moe_status moe_bucket(const int32_t *ids, int n_slots, int n_buckets, int32_t *counts,
                      int32_t *offsets, int32_t *sorted_slot, int32_t *slot_pos, void *workspace,
                      size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * moe_expert_ffn -- grouped SwiGLU experts over the buckets [C31], decode inside the reduction
 * with FP32 accumulation [MX].
 * For every expert e and sorted row r in [offsets[e], offsets[e+1]) with slot s = sorted_slot[r]
 * and token t = s / k_total:
 *   g = W_gate[e] x_t,  u = W_up[e] x_t  (fp32 accumulation of exact products),
 *   h = SiLU(g) * u     (fp32; fed to the down projection as a high + low pair: bf16 for MXFP4
 *                        weights, about 16 significant bits over the whole fp32 range; binary16
 *                        for FP16 weights, which holds only |h| <= 65504 -- larger h overflows
 *                        to infinity, see moe_expert_ffn_f16 [C33] -- and keeps about 22 bits
 *                        for |h| >= 2^-3, below which the low part is subnormal and the pair's
 *                        error stays under 2^-25 absolute),
 *   y_slots[s,:] = W_down[e] h   (fp32).
 *   x        [T][hidden] activations; MXFP4 weights need MOE_ACT_BF16, FP16 weights MOE_ACT_FP16
 *   W        host pointer to the weight description (device pointers inside)
 *   offsets  [W->n_experts + 1], sorted_slot [T*k_total] as written by moe_bucket
 *   y_slots  [T*k_total][hidden] fp32 out; rows of dropped slots are left unwritten
 *   workspace moe_expert_ffn_workspace_bytes(T, k_total, W) bytes, 16-byte aligned
 * Sorted rows whose slot lies outside [0, T*k_total) are skipped, so corrupt device-side indices
 * cannot cause out-of-bounds accesses.
 * Errors: NULL, SHAPE, BLOCK (MXFP4 hidden or inter not a multiple of 32, or a weight base or
 * stride that cuts a 32-value block), ALIGN, DTYPE, WORKSPACE, HIP. */
size_t moe_expert_ffn_workspace_bytes(int T, int k_total, const moe_expert_weights *W);
moe_status moe_expert_ffn(const void *x, moe_act_dtype x_dtype, int T, int k_total,
                          const moe_expert_weights *W, const int32_t *offsets,
                          const int32_t *sorted_slot, float *y_slots, void *workspace,
                          size_t workspace_bytes, void *stream);

/* moe_expert_ffn_static -- moe_expert_ffn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels
 * and the same results, bit for bit, with the workspace taken from a fixed array of
 * MOE_FFN_STATIC_SCRATCH_BYTES bytes inside the library's device code (one per GPU, held until the
 * process ends) instead of a caller buffer.  The call allocates nothing.  Limit: calls whose
 * moe_expert_ffn_workspace_bytes(T, k_total, W) exceeds MOE_FFN_STATIC_SCRATCH_BYTES are refused
 * with MOE_ERR_WORKSPACE (with inter 2048 and top-8 that is T = 256 and above).  Every call on
 * a GPU shares that GPU's array: calls that overlap in time on one GPU (different streams, or
 * several host threads) race and give wrong results; calls ordered on one stream are safe.
 * Arguments and other errors as for moe_expert_ffn; HIP also when the array's device address
 * cannot be looked up. */
#define MOE_FFN_STATIC_SCRATCH_BYTES ((size_t)16 << 20)
moe_status moe_expert_ffn_static(const void *x, moe_act_dtype x_dtype, int T, int k_total,
                                 const moe_expert_weights *W, const int32_t *offsets,
                                 const int32_t *sorted_slot, float *y_slots, void *stream);

/* The three steps of moe_expert_ffn as separate calls, for callers that time or overlap them.
 * moe_expert_ffn_plan writes the tile schedule (which expert and sorted rows each 16-row tile
 * covers, from offsets) into the workspace; moe_expert_ffn_gateup computes
 * h = SiLU(W_gate x) * (W_up x) for every sorted row into the workspace; moe_expert_ffn_down
 * turns the workspace's h into y_slots.  Both phases read the schedule, so the plan must run first
 * on the same workspace with the same T, k_total, W->n_experts and offsets contents; a schedule
 * left from other arguments gives wrong rows, but the kernels check every schedule entry against
 * the call's bounds and never access memory outside the buffers described.  Calling plan, gateup
 * and down on one stream with the same arguments gives exactly moe_expert_ffn's result (it
 * launches the same kernels).  x_dtype of the plan and down calls only selects the format check
 * (it must match W->fmt as in moe_expert_ffn); the plan reads only W's sizes.  Errors as for
 * moe_expert_ffn. */
moe_status moe_expert_ffn_plan(moe_act_dtype x_dtype, int T, int k_total,
                               const moe_expert_weights *W, const int32_t *offsets, void *workspace,
                               size_t workspace_bytes, void *stream);
moe_status moe_expert_ffn_gateup(const void *x, moe_act_dtype x_dtype, int T, int k_total,
                                 const moe_expert_weights *W, const int32_t *offsets,
                                 const int32_t *sorted_slot, void *workspace,
                                 size_t workspace_bytes, void *stream);
moe_status moe_expert_ffn_down(moe_act_dtype x_dtype, int T, int k_total,
                               const moe_expert_weights *W, const int32_t *offsets,
                               const int32_t *sorted_slot, float *y_slots, void *workspace,
                               size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * Range-managed FP16 path [C33] (Cascadia Sec. 3.3, Eq. 1).  For a layer with attenuation
 * A = 2^attenuation_log2 applied to its up projection, the expert path works on E(x) / A and
 * crosses the FP16 boundary in binary16; every row i is combined with its weights divided by
 * F_i = 2^ceil(log2 max(1, sum_j |w_ij|)) and restored as y_i = A F_i y~_i in FP32.  In real
 * arithmetic the result is the plain layer's; the attenuation keeps h, the expert outputs and
 * the combination inside the binary16 range (the configuration recorded for layer 8 uses A = 16),
 * and the factors, being powers of two, are applied and removed exactly.
 *
 * moe_expert_ffn_f16: for every sorted row as in moe_expert_ffn,
 *   u~ = (W_up[e] x_t) / A,  h~ = binary16(SiLU(W_gate[e] x_t) * u~)   (fp32, then rounded),
 *   y_slots[s,:] = binary16(W_down[e] h~)                              (fp32 accumulation)
 * i.e. binary16 expert outputs E(x) / A (IEEE half bits; values past 65504 become infinite, which
 * is what the attenuation is for).  Weights MXFP4 (bf16 x) or FP16 (fp16 x), as for
 * moe_expert_ffn; runs the K-split kernels.  y_slots [T*k_total][hidden] binary16, 2-byte aligned;
 * dropped slots' rows are left unwritten.  workspace: moe_expert_ffn_f16_workspace_bytes bytes,
 * 16-byte aligned.  Errors as for moe_expert_ffn, plus SHAPE for attenuation_log2 outside
 * [0, MOE_MAX_ATTENUATION_LOG2]. */
#define MOE_MAX_ATTENUATION_LOG2 30
size_t moe_expert_ffn_f16_workspace_bytes(int T, int k_total, const moe_expert_weights *W);
moe_status moe_expert_ffn_f16(const void *x, moe_act_dtype x_dtype, int T, int k_total,
                              const moe_expert_weights *W, int attenuation_log2,
                              const int32_t *offsets, const int32_t *sorted_slot, uint16_t *y_slots,
                              void *workspace, size_t workspace_bytes, void *stream);
/* moe_combine_restore: per token t with F_t = 2^ceil(log2 max(1, sum_j |weights[t,j]|)) (fp32 sum
 * in ascending j),
 *   y~[t,:] = binary16(sum_{j ascending} (weights[t,j] / F_t) * y_slots[t*k_total+j,:])  (fp32 sum)
 *   y[t,:]  = A * F_t * y~[t,:]                                                      (fp32, exact)
 * y_slots [T*k_total][H] binary16 (8-byte aligned), weights [T][k_total] fp32, y [T][H] fp32 out
 * (16-byte aligned), H % 4 == 0.  Errors: NULL, SHAPE (also attenuation_log2 out of range), ALIGN,
 * HIP. */
moe_status moe_combine_restore(const uint16_t *y_slots, const float *weights, int T, int k_total, int H,
                               int attenuation_log2, float *y, void *stream);

/* ---------------------------------------------------------------------------------------------
 * MX mode (prefill).  Not on the pages, which define only the MXFP4 weight block [MX]: the
 * activations are quantised to an OCP Microscaling element format, one E8M0 scale per 32
 * consecutive values along K, so that the expert FFN can run the FP4 weights on the matrix
 * cores' scaled FP4 x FP8/FP6/FP4 instructions.  The result is NOT the exact layer: it differs
 * from moe_expert_ffn by the quantisation of x and h (use moe_expert_ffn for exact results).
 *
 * Element formats (sign | exponent | fraction, subnormals at exponent field 0):
 *   MOE_MX_FP8_E4M3  8-bit, bias 7, largest 448 (S.1111.111 is NaN and never produced)
 *   MOE_MX_FP4_E2M1  4-bit, bias 1, largest 6 (the weights' E2M1 codes)
 *   MOE_MX_FP6_E2M3  6-bit, bias 1, largest 7.5
 * Quantisation of a block of 32 values v_i with amax = max |v_i|: scale code
 * c = clamp(floor(log2 amax) - emax + 127, 0, 254) (emax = 8, 2, 2; c = 0 for an all-zero block),
 * X = 2^(c - 127), and code_i = the element value nearest to v_i / X, ties to the even code,
 * saturating at the largest value, with the sign of v_i (so -0 and tiny negative values give the
 * negative-zero code).
 * Packed codes: a block takes 4 * bits bytes -- FP8 one code per byte; FP4 two per byte, element
 * 2j in the low nibble of byte j; FP6 element j in bits 6j .. 6j+5 of the block's little-endian
 * 192-bit string.  A row of K values is K/32 consecutive blocks, rows are consecutive. */
typedef enum { MOE_MX_FP8_E4M3 = 1, MOE_MX_FP4_E2M1 = 2, MOE_MX_FP6_E2M3 = 3 } moe_mx_format;

/* Bytes of one packed row of K values (K/32 * 4 * bits); 0 for an unknown format or K % 32 != 0. */
size_t moe_mx_row_bytes(moe_mx_format fmt, int K);

/* moe_mx_quantize -- the activation quantiser of the MX mode on its own:
 *   x [n_rows][K] bf16 or fp16 (contiguous, 16-byte aligned), codes [n_rows][row bytes] out
 *   (16-byte aligned), scales [n_rows][K/32] E8M0 out.
 * Errors: NULL, SHAPE (n_rows < 0, K < 1), BLOCK (K % 32), DTYPE (format or x dtype), ALIGN, HIP. */
moe_status moe_mx_quantize(const void *x, moe_act_dtype x_dtype, int n_rows, int K, moe_mx_format fmt,
                           uint8_t *codes, uint8_t *scales, void *stream);

/* moe_expert_ffn_mx -- moe_expert_ffn with MX activations: for every sorted row r of expert e
 * with slot s and token t = s / k_total,
 *   xq = dequant(quant(x[t,:])),  g = W_gate[e] xq,  u = W_up[e] xq  (fp32 accumulation),
 *   h = SiLU(g) * u (fp32),  hq = dequant(quant(h)),  y_slots[s,:] = W_down[e] hq  (fp32),
 * quant/dequant being the block quantisation above along hidden (x) and inter (h).  Weights must
 * be MXFP4 and x bf16.  hidden and inter must be multiples of 256; scale pointers and strides
 * multiples of 8 bytes.  Arguments otherwise as for moe_expert_ffn, with the workspace from
 * moe_expert_ffn_mx_workspace_bytes (it holds the x and h codes and the tile table).
 * Errors: NULL, SHAPE (also hidden or inter not a multiple of 256, or buffers past 2^31 bytes),
 * BLOCK, ALIGN, DTYPE (weights not MXFP4, x not bf16, unknown format), WORKSPACE, HIP. */
size_t moe_expert_ffn_mx_workspace_bytes(int T, int k_total, const moe_expert_weights *W,
                                         moe_mx_format fmt);
moe_status moe_expert_ffn_mx(const void *x, moe_act_dtype x_dtype, int T, int k_total,
                             const moe_expert_weights *W, moe_mx_format fmt, const int32_t *offsets,
                             const int32_t *sorted_slot, float *y_slots, void *workspace,
                             size_t workspace_bytes, void *stream);
/* Where moe_expert_ffn_mx leaves its quantised activations in the workspace, for inspection:
 * offsets[0] x codes ([T] packed rows of `hidden` values), offsets[1] x scales ([T][hidden/32]),
 * offsets[2] h codes ([T*k_total] packed rows of `inter` values, row r belonging to sorted row r,
 * i.e. slot sorted_slot[r]; rows of empty slots are unspecified), offsets[3] h scales
 * ([T*k_total][inter/32]).  offsets is a host array of 4.  Errors: NULL, SHAPE, DTYPE. */
moe_status moe_expert_ffn_mx_workspace_layout(int T, int k_total, const moe_expert_weights *W,
                                              moe_mx_format fmt, size_t *offsets);

/* ---------------------------------------------------------------------------------------------
 * moe_combine -- weighted reduction [C31] with FP32 output [C32]:
 *   y[t,:] = sum_{j = 0 .. k_total-1, in ascending j} weights[t,j] * y_slots[t*k_total+j,:]
 * Every output element has exactly one owner (no atomics).
 *   y_slots [T*k_total][H] fp32, weights [T][k_total] fp32, y [T][H] fp32 out; H % 4 == 0,
 *   y_slots and y 16-byte aligned.
 * Errors: NULL, SHAPE, ALIGN, HIP. */
moe_status moe_combine(const float *y_slots, const float *weights, int T, int k_total, int H,
                       float *y, void *stream);

/* ---------------------------------------------------------------------------------------------
 * moe_mxfp4_dequant -- the device decode primitive of the expert FFN, exposed on its own: writes
 * out[n][k] = bf16(v(code) * 2^(scale-127)) for an [n_rows][K] MXFP4 matrix [MX].  The value is
 * exact in bf16 whenever it is finite (all scale codes 0..252; larger codes can overflow).
 *   codes [n_rows] rows of K/2 bytes at code_row_stride; scales [n_rows] rows of K/32 bytes at
 *   scale_row_stride; out [n_rows][K] bf16 (uint16 bits), 16-byte aligned.
 * Errors: NULL, SHAPE, BLOCK (K % 32, or codes / code_row_stride off the 16-byte block grid),
 * ALIGN (out), HIP. */
moe_status moe_mxfp4_dequant(const uint8_t *codes, const uint8_t *scales, int n_rows, int K,
                             int64_t code_row_stride, int64_t scale_row_stride, uint16_t *out,
                             void *stream);

/* moe_stream_read -- a measurement utility, not a step of the layer: reads `bytes` of device memory
 * at `buf` once, with 16-byte nontemporal loads in which consecutive lanes take consecutive 16-byte
 * pieces (every wave load covers whole 128-byte lines, the shape in which the streaming FFN
 * kernels read their weights), and folds them into a checksum.  Timed over a buffer much larger
 * than the caches, it gives the practical HBM read rate that those kernels are compared with.
 *   buf device memory, 16-byte aligned, read only; bytes a multiple of 16 (0 is a no-op);
 *   sink one device uint32, written only when the checksum takes one fixed value, so its
 *   contents are meaningless (it exists so that the loads cannot be removed).
 * Errors: NULL, ALIGN (buf or bytes), HIP. */
moe_status moe_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

/* Short text for a status code (host, static storage). */
const char *moe_status_str(moe_status status);
/* MOE_ABI_VERSION of the built library. */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
