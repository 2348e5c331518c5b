/*
 * moe_oracle.h -- plain, slow fp64 CPU oracle of the routed Mixture-of-Experts FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's CPU-baseline leg
 * may load or call it.  It shares no code, header, table or helper with the HIP library, and the
 * library never calls it.
 *
 * Sources (cited by page title and section):
 *  [MX]  "DeepSeek-V4-Flash on a four-GPU Ampere workstation" (FreeToken blog post), section
 *        "MXFP4 is not NVFP4, and the difference matters on Ampere": E2M1 codes, E8M0 block
 *        scales, decoded weight v(c) 2^(e-127), 4.25 bits per weight, the decode-in-reduction
 *        sum z_n, row-major packed banks.
 *  [BP]  same post, section "Why it would not run": quantised partitioning must preserve blocks.
 *  [C31] "Cascadia: Resident 975B MoE Inference on Eleven AI PCs", Sec. 3.1: expert-major banks,
 *        gate/up projections, SwiGLU, down projection, weighted reduction; routing yields expert
 *        ids and routing weights; shared experts are always-included selections.
 *  [C32] Cascadia Sec. 3.2: a call supplies rows, expert ids and weights; FP32 output.
 *  [C33] Cascadia Sec. 3.3, Eq. 1: a layer attenuation A = 2^n on the up projection and a row
 *        factor F_i on the routing weights keep the FP16 expert path in range; both are restored
 *        in FP32 afterwards.
 *  [C34] Cascadia Sec. 3.4, Eq. 2: a dense FFN equals the sum of its all-active slices.
 *
 * Where the pages leave a step open the reading used here is stated next to the function.
 * Every floating-point value is computed in IEEE binary64 with plain loops in index order.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stddef.h>
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_W_MXFP4 = 0, ORC_W_FP16 = 1, ORC_W_INT4_G32 = 2, ORC_W_NVFP4 = 3 };
enum { ORC_X_BF16 = 0, ORC_X_FP16 = 1 };

/* One projection of every expert, logical [n_experts][N][K] with K contiguous.
 * MXFP4: w holds bytes, element k of a row in byte k/2, even k in the low nibble; scales hold one
 *        E8M0 byte per 32 elements along K.  FP16: w holds binary16 words, scales unused.
 * INT4_G32 (Cascadia Sec. 3.1 and 3.5): w holds unsigned 4-bit codes packed as for MXFP4; group
 *        g = k/32 has a binary16 scale (little-endian bytes 2g, 2g+1 of the scale row) and an
 *        unsigned 4-bit zero point (nibble g%2 of byte g/2 of the zero row, low nibble first);
 *        weight = (code - zero) * scale.
 * NVFP4 (FreeToken post, "MXFP4 is not NVFP4"): w holds E2M1 codes packed as for MXFP4; block
 *        b = k/16 has an E4M3 scale byte (byte b of the scale row); each expert has one fp32
 *        tensor scale; weight = v(code) * e4m3(scale) * tensor_scale[e].
 * Strides are in bytes, so slices of a larger matrix can be described. */
typedef struct {
  const void *w;
  const uint8_t *scales;
  int64_t w_expert_stride, w_row_stride, s_expert_stride, s_row_stride;
  const uint8_t *zeros;          /* INT4_G32 zero points */
  int64_t z_expert_stride, z_row_stride;
  const float *tensor_scale;     /* NVFP4: [n_experts] */
} orc_proj;

typedef struct {
  int fmt;        /* ORC_W_MXFP4 or ORC_W_FP16 */
  int n_experts;  /* E' = routed + shared */
  int hidden;     /* H */
  int inter;      /* I */
  orc_proj gate;  /* N = I, K = H */
  orc_proj up;    /* N = I, K = H */
  orc_proj down;  /* N = H, K = I */
} orc_weights;

/* ---- number formats ---- */
double orc_e2m1(int code);                  /* v(c), c in [0,16) */
double orc_e8m0(int e);                     /* 2^(e-127), e in [0,256) */
double orc_mxfp4(int code, int e);          /* v(c) 2^(e-127) */
double orc_bf16(uint16_t bits);
double orc_f16(uint16_t bits);
double orc_weight(const orc_proj *p, int fmt, int e, int n, int k);
double orc_mxfp4_bits_per_weight(void);     /* storage cost of one block, per weight */
double orc_int4g32_bits_per_weight(void);   /* 32 codes + binary16 scale + 4-bit zero point */
double orc_nvfp4_bits_per_weight(void);     /* 16 codes + E4M3 scale (tensor scale not counted) */
int64_t orc_mxfp4_bytes(int64_t n_rows, int64_t k);  /* codes + scales of an [n_rows][k] matrix */

/* ---- the layer ---- */
void orc_route(const uint16_t *x, int x_fmt, int T, int H, const float *w_router, const float *bias,
               int E, int top_k, int n_shared, double tie_eps,
               double *logits, double *probs, int32_t *ids, double *weights, uint8_t *near_tie);
/* Sigmoid router (Cascadia Sec. 3.1): sigmoid scores, top-k by score + sel_bias (bias moves the
 * selection only), selected scores normalised to 1 and multiplied by routed_scale, shared slots
 * with shared_weight.  scores [T][E] (optional) are the sigmoid scores. */
void orc_route_sigmoid(const uint16_t *x, int x_fmt, int T, int H, const float *w_router,
                       const float *sel_bias, int E, int top_k, int n_shared, double routed_scale,
                       double shared_weight, double tie_eps, double *scores, int32_t *ids,
                       double *weights, uint8_t *near_tie);
int orc_bucket(const int32_t *ids, int n_slots, int n_buckets, int32_t *counts, int32_t *offsets,
               int32_t *sorted_slot, int32_t *slot_pos);
void orc_expert_apply(const orc_weights *W, int e, const double *xv, double *out);
void orc_expert_ffn(const uint16_t *x, int x_fmt, int T, int k_total, const orc_weights *W,
                    const int32_t *offsets, const int32_t *sorted_slot, const uint8_t *slot_mask,
                    double *y_slots);
void orc_combine(const double *y_slots, const double *weights, int T, int k_total, int H,
                 const uint8_t *token_mask, double *y);

/* ---- FP16 range management (Cascadia Sec. 3.3, Eq. 1) ----
 * A = 2^att_log2 attenuates the layer's up projection, so each expert returns E(x) / A; each row i
 * takes F_i = 2^ceil(log2 max(1, sum_j |w_ij|)), combines y~_i = sum_j (w_ij / F_i) E_ij / A and is
 * restored as y_i = A F_i y~_i.  All in fp64: with powers of two and no overflow or underflow the
 * result is the plain layer's, bit for bit. */
void orc_expert_ffn_attenuated(const uint16_t *x, int x_fmt, int T, int k_total, const orc_weights *W,
                               int att_log2, const int32_t *offsets, const int32_t *sorted_slot,
                               const uint8_t *slot_mask, double *y_slots);
double orc_row_factor(const double *w, int k_total);
void orc_combine_restore(const double *y_slots_att, const double *weights, int T, int k_total, int H,
                         int att_log2, const uint8_t *token_mask, double *y);

/* ---- MX activation formats (prefill MX mode) ----
 * Not on the pages, which define only the E2M1 + E8M0 weight block [MX].  Reading: the activation
 * blocks of the MX mode follow the OCP Microscaling (MX) v1.0 element formats -- E4M3 (bias 7, no
 * infinities, S.1111.111 is NaN, max 448), E2M3 (bias 1, max 7.5) and E2M1 (the page's codes,
 * max 6) -- with one E8M0 scale per 32 consecutive values along K and the scale rule
 * X = 2^(floor(log2 amax) - emax) of that specification, emax being the exponent of the format's
 * largest normal (8, 2, 2).  Elements are rounded to nearest, ties to the even code, saturating. */
enum { ORC_MX_FP8_E4M3 = 1, ORC_MX_FP4_E2M1 = 2, ORC_MX_FP6_E2M3 = 3 };
int orc_mx_bits(int fmt);                   /* bits per element code: 8, 4, 6 */
int orc_mx_emax(int fmt);                   /* exponent of the largest normal: 8, 2, 2 */
double orc_mx_value(int fmt, int code);     /* element value of a code (NaN for E4M3 NaN codes) */
int orc_mx_encode(int fmt, double q);       /* nearest code to q, ties to even, saturating */
int orc_mx_scale_code(int fmt, double amax);/* E8M0 code of a block with largest magnitude amax */
/* codes [n_rows][K] one element code per byte; scales [n_rows][K/32] */
void orc_mx_quantize(const double *v, int n_rows, int K, int fmt, uint8_t *codes, uint8_t *scales);
void orc_mx_dequantize(const uint8_t *codes, const uint8_t *scales, int n_rows, int K, int fmt,
                       double *out);
/* The grouped expert FFN of the MX mode: like orc_expert_ffn, with the token's x row and each
 * slot's h row replaced by their MX round trip (quantize, then dequantize) before they enter a
 * projection.  Weights stay the exact decoded MXFP4 values; all arithmetic is fp64.
 * h_pre (optional, [n_slots][I] indexed by sorted row): the fp64 h of every computed row before
 * its quantisation. */
void orc_expert_ffn_mx(const uint16_t *x, int x_fmt, int T, int k_total, const orc_weights *W,
                       int act_fmt, const int32_t *offsets, const int32_t *sorted_slot,
                       const uint8_t *slot_mask, double *y_slots, double *h_pre);

/* ---- cross-check forms ---- */
void orc_layer_bruteforce(const uint16_t *x, int x_fmt, int T, int k_total, const orc_weights *W,
                          const int32_t *ids, const double *weights, double *y);
void orc_layer_dense_mixture(const uint16_t *x, int x_fmt, int T, int k_total, const orc_weights *W,
                             const int32_t *ids, const double *weights, double *y);
void orc_dense_ffn_f16(const uint16_t *x, int x_fmt, int T, int H, int I, const uint16_t *wg,
                       const uint16_t *wu, const uint16_t *wd, double *y);
void orc_mxfp4_decode_matrix(const uint8_t *codes, const uint8_t *scales, int n_rows, int k,
                             double *out);
double orc_silu(double z);
int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
