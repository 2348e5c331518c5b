/*
 * moe_oracle.c -- fp64 CPU oracle of the routed MoE FFN layer.  TEST INFRASTRUCTURE ONLY
 * (see moe_oracle.h for who may use it and for the source abbreviations [MX] [BP] [C31] ...).
 *
 * Plain loops, IEEE binary64 throughout, no blocking or reordering beyond what each definition
 * states.  OpenMP only distributes independent output elements over threads; every output element
 * is still produced by one thread in index order, so results do not depend on the thread count.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------------------------ */
/* Number formats                                                                             */
/* ------------------------------------------------------------------------------------------ */

/* [MX]: an E2M1 code is one sign bit plus a magnitude from {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
 * Reading (the page gives the set, not the bit assignment): bit 3 is the sign, bits 2..0 index
 * the magnitudes in ascending order -- the standard E2M1 layout (2 exponent bits, bias 1, one
 * mantissa bit).  Code 8 is negative zero. */
static const double E2M1_MAGNITUDE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1(int code) {
  double mag = E2M1_MAGNITUDE[code & 7];
  return (code & 8) ? -mag : mag;
}

/* [MX]: the block scale is the unsigned E8M0 code e; its value is 2^(e-127). */
double orc_e8m0(int e) { return ldexp(1.0, e - 127); }

/* [MX]: decoded weight w_hat = v(c) * 2^(e-127). */
double orc_mxfp4(int code, int e) { return orc_e2m1(code) * orc_e8m0(e); }

/* [MX]: a 32-weight block stores 32 four-bit codes and one 8-bit scale: 4 + 8/32 bits per weight. */
double orc_mxfp4_bits_per_weight(void) { return (32.0 * 4.0 + 8.0) / 32.0; }

/* Cascadia Sec. 3.1 and 3.5: a group of 32 four-bit codes carries a binary16 scale and (reading)
 * a four-bit zero point: 4 + 16/32 + 4/32 bits per weight. */
double orc_int4g32_bits_per_weight(void) { return (32.0 * 4.0 + 16.0 + 4.0) / 32.0; }

/* FreeToken post, "MXFP4 is not NVFP4": E2M1 codes with one E4M3 scale per 16 values, 4 + 8/16
 * bits per weight before the tensor scale. */
double orc_nvfp4_bits_per_weight(void) { return (16.0 * 4.0 + 8.0) / 16.0; }

int64_t orc_mxfp4_bytes(int64_t n_rows, int64_t k) {
  return n_rows * (k / 2) + n_rows * (k / 32);
}

/* bfloat16: the top 16 bits of an IEEE binary32 value. */
double orc_bf16(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_f16(uint16_t bits) {
  int sign = bits >> 15, ex = (bits >> 10) & 31, fr = bits & 1023;
  double v;
  if (ex == 0)
    v = ldexp((double)fr, -24);                       /* zero and subnormals: fr * 2^-14 * 2^-10 */
  else if (ex == 31)
    v = fr ? NAN : INFINITY;
  else
    v = ldexp(1024.0 + (double)fr, ex - 25);          /* (1 + fr/1024) * 2^(ex-15) */
  return sign ? -v : v;
}

static double act_value(const uint16_t *x, int x_fmt, int64_t i) {
  return x_fmt == ORC_X_FP16 ? orc_f16(x[i]) : orc_bf16(x[i]);
}

/* Element (n, k) of expert e of one projection.  [MX]: element k of a packed row lives in byte
 * k/2 (reading: even k in the low nibble) and uses the scale of block floor(k/32); rows are
 * row-major with K contiguous, read in place with no repack.  The other formats as described in
 * moe_oracle.h. */
double orc_weight(const orc_proj *p, int fmt, int e, int n, int k) {
  const uint8_t *row = (const uint8_t *)p->w + (int64_t)e * p->w_expert_stride + (int64_t)n * p->w_row_stride;
  if (fmt == ORC_W_FP16) {
    uint16_t bits;
    memcpy(&bits, row + 2 * (int64_t)k, 2);
    return orc_f16(bits);
  }
  const uint8_t *srow = p->scales + (int64_t)e * p->s_expert_stride + (int64_t)n * p->s_row_stride;
  uint8_t byte = row[k / 2];
  int code = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
  if (fmt == ORC_W_INT4_G32) {
    /* Cascadia Sec. 3.1: group-32 unsigned INT4 codes with a binary16 scale; zero point (reading:
     * four bits, low nibble first) */
    const int g = k / 32;
    const uint16_t sbits = (uint16_t)(srow[2 * g] | (srow[2 * g + 1] << 8));
    const uint8_t *zrow = p->zeros + (int64_t)e * p->z_expert_stride + (int64_t)n * p->z_row_stride;
    const int zero = (g % 2 == 0) ? (zrow[g / 2] & 0x0F) : (zrow[g / 2] >> 4);
    return (double)(code - zero) * orc_f16(sbits);
  }
  if (fmt == ORC_W_NVFP4) {
    /* FreeToken post: E2M1 value times the E4M3 scale of its 16-value block times the tensor
     * scale */
    return orc_e2m1(code) * orc_mx_value(ORC_MX_FP8_E4M3, srow[k / 16]) * (double)p->tensor_scale[e];
  }
  return orc_mxfp4(code, srow[k / 32]);
}

/* SiLU(z) = z / (1 + e^-z).  For very negative z, e^-z overflows to +inf and the quotient is -0,
 * which is the limit; no NaN can arise for finite z. */
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count for the following calls (timing only: results do not depend on it). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------------------------ */
/* Router: logits, softmax, top-k, renormalise, append shared experts                         */
/* ------------------------------------------------------------------------------------------ */

/* Per token t:
 *   L[t,e] = sum_h x[t,h] W_r[e,h] + b[e]
 *   p      = softmax(L[t,:]) = exp(L - max L) / sum exp(L - max L)
 *   the k experts with the largest p, ordered by (p descending, index ascending)
 *   w_j    = p_j / sum_{j'<k} p_j'      (routing weights renormalised to 1)
 *   slots k .. k+S-1 hold the shared experts E .. E+S-1 with weight 1.
 * [C31] routing produces expert ids and routing weights for the fused expert path, and shared
 * experts are always-included selections after the routed ones.  The softmax -> top-k ->
 * renormalise order, the lowest-index tie-break and the shared weight of 1 (outside the
 * renormalisation) are readings: the pages print no softmax router.
 * near_tie[t] = 1 when two neighbours among the first min(k+1, E) sorted probabilities differ by
 * at most tie_eps; such tokens may legitimately come out in another order. */
void orc_route(const uint16_t *x, int x_fmt, int T, int H, const float *w_router, const float *bias,
               int E, int top_k, int n_shared, double tie_eps,
               double *logits, double *probs, int32_t *ids, double *weights, uint8_t *near_tie) {
  const int k_total = top_k + n_shared;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t) {
    double *L = (double *)malloc(sizeof(double) * (size_t)E);
    double *p = (double *)malloc(sizeof(double) * (size_t)E);
    int *order = (int *)malloc(sizeof(int) * (size_t)E);
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += act_value(x, x_fmt, (int64_t)t * H + h) * (double)w_router[(int64_t)e * H + h];
      L[e] = acc + (bias ? (double)bias[e] : 0.0);
    }
    double mx = L[0];
    for (int e = 1; e < E; ++e)
      if (L[e] > mx) mx = L[e];
    double den = 0.0;
    for (int e = 0; e < E; ++e) {
      p[e] = exp(L[e] - mx);
      den += p[e];
    }
    for (int e = 0; e < E; ++e) p[e] /= den;
    /* Selection: repeatedly take the largest remaining p, lowest index first among equals. */
    for (int e = 0; e < E; ++e) order[e] = e;
    int n_sort = top_k + 1 < E ? top_k + 1 : E;
    for (int j = 0; j < n_sort; ++j) {
      int best = j;
      for (int i = j + 1; i < E; ++i) {
        int a = order[i], b = order[best];
        if (p[a] > p[b] || (p[a] == p[b] && a < b)) best = i;
      }
      int tmp = order[j];
      order[j] = order[best];
      order[best] = tmp;
    }
    double sel = 0.0;
    for (int j = 0; j < top_k; ++j) sel += p[order[j]];
    for (int j = 0; j < top_k; ++j) {
      ids[(int64_t)t * k_total + j] = order[j];
      weights[(int64_t)t * k_total + j] = p[order[j]] / sel;
    }
    for (int s = 0; s < n_shared; ++s) {
      ids[(int64_t)t * k_total + top_k + s] = E + s;
      weights[(int64_t)t * k_total + top_k + s] = 1.0;
    }
    uint8_t tie = 0;
    for (int j = 0; j + 1 < n_sort; ++j)
      if (p[order[j]] - p[order[j + 1]] <= tie_eps) tie = 1;
    if (near_tie) near_tie[t] = tie;
    if (logits) memcpy(logits + (int64_t)t * E, L, sizeof(double) * (size_t)E);
    if (probs) memcpy(probs + (int64_t)t * E, p, sizeof(double) * (size_t)E);
    free(L);
    free(p);
    free(order);
  }
}

/* Sigmoid router of Cascadia Sec. 3.1 (Inkling's gate): per token t
 *   L[t,e] = sum_h x[t,h] W_r[e,h]                 (no bias inside the score)
 *   s[t,e] = 1 / (1 + e^-L[t,e])                   (sigmoid scores)
 *   the k experts with the largest s[t,e] + b[e], ordered by (that key desc, index asc)
 *       (bias-adjusted selection: b moves the choice only)
 *   w_j    = gamma * s_j / sum_{j'<k} s_j'         (selected scores normalised to 1, times the
 *                                                   model's scale factor gamma)
 *   slots k .. k+S-1: shared experts E .. E+S-1 with weight shared_weight.
 * Readings: the page names the steps (sigmoid scores, bias-adjusted top-k, selected/shared
 * normalisation, model-specific scale factors) without their formulas; the normalisation over the
 * selected scores, gamma as one multiplier of the routed weights and a fixed shared weight are the
 * plainest forms of those steps.  near_tie as in orc_route, on the selection keys. */
void orc_route_sigmoid(const uint16_t *x, int x_fmt, int T, int H, const float *w_router,
                       const float *sel_bias, int E, int top_k, int n_shared, double routed_scale,
                       double shared_weight, double tie_eps, double *scores, int32_t *ids,
                       double *weights, uint8_t *near_tie) {
  const int k_total = top_k + n_shared;
#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < T; ++t) {
    double *sc = (double *)malloc(sizeof(double) * (size_t)E);
    double *key = (double *)malloc(sizeof(double) * (size_t)E);
    int *order = (int *)malloc(sizeof(int) * (size_t)E);
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int h = 0; h < H; ++h)
        acc += act_value(x, x_fmt, (int64_t)t * H + h) * (double)w_router[(int64_t)e * H + h];
      sc[e] = 1.0 / (1.0 + exp(-acc));
      key[e] = sc[e] + (sel_bias ? (double)sel_bias[e] : 0.0);
    }
    for (int e = 0; e < E; ++e) order[e] = e;
    int n_sort = top_k + 1 < E ? top_k + 1 : E;
    for (int j = 0; j < n_sort; ++j) {
      int best = j;
      for (int i = j + 1; i < E; ++i) {
        int a = order[i], b = order[best];
        if (key[a] > key[b] || (key[a] == key[b] && a < b)) best = i;
      }
      int tmp = order[j];
      order[j] = order[best];
      order[best] = tmp;
    }
    double sel = 0.0;
    for (int j = 0; j < top_k; ++j) sel += sc[order[j]];
    for (int j = 0; j < top_k; ++j) {
      ids[(int64_t)t * k_total + j] = order[j];
      weights[(int64_t)t * k_total + j] = routed_scale * (sc[order[j]] / sel);
    }
    for (int s = 0; s < n_shared; ++s) {
      ids[(int64_t)t * k_total + top_k + s] = E + s;
      weights[(int64_t)t * k_total + top_k + s] = shared_weight;
    }
    uint8_t tie = 0;
    for (int j = 0; j + 1 < n_sort; ++j)
      if (key[order[j]] - key[order[j + 1]] <= tie_eps) tie = 1;
    if (near_tie) near_tie[t] = tie;
    if (scores) memcpy(scores + (int64_t)t * E, sc, sizeof(double) * (size_t)E);
    free(sc);
    free(key);
    free(order);
  }
}

/* ------------------------------------------------------------------------------------------ */
/* Bucketing: group slots by expert                                                           */
/* ------------------------------------------------------------------------------------------ */

/* [C31]: the fused path executes only the selected experts' work, so slots are grouped by expert.
 * counts[b] = number of slots s with ids[s] == b; offsets = exclusive prefix sum of counts with
 * offsets[n_buckets] = number of valid slots; sorted_slot lists slot indices bucket by bucket,
 * ascending slot index within a bucket (a stable counting sort); slot_pos is its inverse.
 * A slot whose id is outside [0, n_buckets) is dropped: slot_pos = -1, and sorted_slot entries
 * past the valid count are -1.  Returns the number of valid slots. */
int orc_bucket(const int32_t *ids, int n_slots, int n_buckets, int32_t *counts, int32_t *offsets,
               int32_t *sorted_slot, int32_t *slot_pos) {
  for (int b = 0; b < n_buckets; ++b) counts[b] = 0;
  for (int s = 0; s < n_slots; ++s)
    if (ids[s] >= 0 && ids[s] < n_buckets) counts[ids[s]]++;
  offsets[0] = 0;
  for (int b = 0; b < n_buckets; ++b) offsets[b + 1] = offsets[b] + counts[b];
  int32_t *fill = (int32_t *)calloc((size_t)n_buckets + 1, sizeof(int32_t));
  for (int s = 0; s < n_slots; ++s) sorted_slot[s] = -1;
  for (int s = 0; s < n_slots; ++s) {
    int b = ids[s];
    if (b < 0 || b >= n_buckets) {
      if (slot_pos) slot_pos[s] = -1;
      continue;
    }
    int pos = offsets[b] + fill[b]++;
    sorted_slot[pos] = s;
    if (slot_pos) slot_pos[s] = pos;
  }
  free(fill);
  return offsets[n_buckets];
}

/* ------------------------------------------------------------------------------------------ */
/* Expert FFN                                                                                 */
/* ------------------------------------------------------------------------------------------ */

/* One expert applied to one activation vector xv[H] (already in double):
 *   g_n = sum_k W_g[n,k] x_k,  u_n = sum_k W_u[n,k] x_k,  h_n = SiLU(g_n) u_n,
 *   out_m = sum_n W_d[m,n] h_n.
 * [C31] gate/up projections, SwiGLU, down projection.  With MXFP4 weights each sum is the
 * decode-in-reduction sum z_n = sum_k a_k v(c_{n,k}) 2^(e_{n,floor(k/32)}-127) of [MX]. */
void orc_expert_apply(const orc_weights *W, int e, const double *xv, double *out) {
  const int H = W->hidden, I = W->inter;
  double *h = (double *)malloc(sizeof(double) * (size_t)I);
  for (int n = 0; n < I; ++n) {
    double g = 0.0, u = 0.0;
    for (int k = 0; k < H; ++k) {
      g += orc_weight(&W->gate, W->fmt, e, n, k) * xv[k];
      u += orc_weight(&W->up, W->fmt, e, n, k) * xv[k];
    }
    h[n] = orc_silu(g) * u;
  }
  for (int m = 0; m < H; ++m) {
    double acc = 0.0;
    for (int n = 0; n < I; ++n) acc += orc_weight(&W->down, W->fmt, e, m, n) * h[n];
    out[m] = acc;
  }
  free(h);
}

/* Grouped expert FFN over buckets: for every expert e and every row r in
 * [offsets[e], offsets[e+1]), slot s = sorted_slot[r] of token t = s / k_total gets
 * y_slots[s,:] = expert_e(x[t,:]).  Each expert's weight rows are decoded once per row and
 * applied to all of its bucket's rows -- the same sums as orc_expert_apply, in the same k order.
 * slot_mask (optional): only slots with slot_mask[s] != 0 are computed; other rows of y_slots are
 * left untouched. */
static void mx_round_trip(double *v, int K, int fmt);

/* act_fmt = 0: the exact FFN.  act_fmt = an ORC_MX_* format: the MX mode, where the token's x row
 * and each slot's h row go through the MX round trip before entering a projection. */
static void grouped_ffn(const uint16_t *x, int x_fmt, int T, int k_total, const orc_weights *W,
                        int act_fmt, double up_scale, const int32_t *offsets,
                        const int32_t *sorted_slot, const uint8_t *slot_mask, double *y_slots,
                        double *h_pre) {
  const int H = W->hidden, I = W->inter, E2 = W->n_experts;
  const int64_t n_slots = (int64_t)T * k_total;
  for (int e = 0; e < E2; ++e) {
    int r0 = offsets[e], r1 = offsets[e + 1];
    int n_rows = 0;
    int *slot = (int *)malloc(sizeof(int) * (size_t)(r1 - r0 + 1));
    int *srow = (int *)malloc(sizeof(int) * (size_t)(r1 - r0 + 1));
    for (int r = r0; r < r1; ++r) {
      int s = sorted_slot[r];
      if (s < 0 || s >= n_slots) continue;
      if (slot_mask && !slot_mask[s]) continue;
      srow[n_rows] = r;
      slot[n_rows++] = s;
    }
    if (n_rows == 0) {
      free(slot);
      free(srow);
      continue;
    }
    double *xs = (double *)malloc(sizeof(double) * (size_t)n_rows * H);
    double *hs = (double *)malloc(sizeof(double) * (size_t)n_rows * I);
    for (int i = 0; i < n_rows; ++i) {
      int t = slot[i] / k_total;
      for (int k = 0; k < H; ++k) xs[(int64_t)i * H + k] = act_value(x, x_fmt, (int64_t)t * H + k);
      if (act_fmt) mx_round_trip(xs + (int64_t)i * H, H, act_fmt);
    }
#pragma omp parallel for schedule(static)
    for (int n = 0; n < I; ++n) {
      double *wg = (double *)malloc(sizeof(double) * (size_t)H);
      double *wu = (double *)malloc(sizeof(double) * (size_t)H);
      for (int k = 0; k < H; ++k) {
        wg[k] = orc_weight(&W->gate, W->fmt, e, n, k);
        wu[k] = orc_weight(&W->up, W->fmt, e, n, k);
      }
      for (int i = 0; i < n_rows; ++i) {
        const double *xv = xs + (int64_t)i * H;
        double g = 0.0, u = 0.0;
        for (int k = 0; k < H; ++k) {
          g += wg[k] * xv[k];
          u += wu[k] * xv[k];
        }
        hs[(int64_t)i * I + n] = orc_silu(g) * (u * up_scale);
      }
      free(wg);
      free(wu);
    }
    if (h_pre)
      for (int i = 0; i < n_rows; ++i) memcpy(h_pre + (int64_t)srow[i] * I, hs + (int64_t)i * I, sizeof(double) * (size_t)I);
    if (act_fmt) {
#pragma omp parallel for schedule(static)
      for (int i = 0; i < n_rows; ++i) mx_round_trip(hs + (int64_t)i * I, I, act_fmt);
    }
#pragma omp parallel for schedule(static)
    for (int m = 0; m < H; ++m) {
      double *wd = (double *)malloc(sizeof(double) * (size_t)I);
      for (int n = 0; n < I; ++n) wd[n] = orc_weight(&W->down, W->fmt, e, m, n);
      for (int i = 0; i < n_rows; ++i) {
        const double *hv = hs + (int64_t)i * I;
        double acc = 0.0;
        for (int n = 0; n < I; ++n) acc += wd[n] * hv[n];
        y_slots[(int64_t)slot[i] * H + m] = acc;
      }
      free(wd);
    }
    free(xs);
    free(hs);
    free(slot);
    free(srow);
  }
}

void orc_expert_ffn(const uint16_t *x, int x_fmt, int T, int k_total, const orc_weights *W,
                    const int32_t *offsets, const int32_t *sorted_slot, const uint8_t *slot_mask,
                    double *y_slots) {
  grouped_ffn(x, x_fmt, T, k_total, W, 0, 1.0, offsets, sorted_slot, slot_mask, y_slots, NULL);
}

/* Cascadia Sec. 3.3, Eq. 1, expert side: the layer's up projection is attenuated by
 * A = 2^att_log2, so h~ = SiLU(g) (u / A) and the expert output becomes E(x) / A (the up branch
 * enters SwiGLU as a factor, so the attenuation carries straight through the down projection). */
void orc_expert_ffn_attenuated(const uint16_t *x, int x_fmt, int T, int k_total, const orc_weights *W,
                               int att_log2, const int32_t *offsets, const int32_t *sorted_slot,
                               const uint8_t *slot_mask, double *y_slots) {
  grouped_ffn(x, x_fmt, T, k_total, W, 0, ldexp(1.0, -att_log2), offsets, sorted_slot, slot_mask, y_slots,
              NULL);
}

/* Cascadia Sec. 3.3, Eq. 1, row factor: F = 2^ceil(log2 max(1, sum_j |w_j|)) over the row's
 * selections.  frexp gives m = f 2^ex with f in [0.5, 1): m is a power of two exactly when
 * f == 0.5, and then ceil(log2 m) = ex - 1; otherwise it is ex. */
double orc_row_factor(const double *w, int k_total) {
  double sum = 0.0;
  for (int j = 0; j < k_total; ++j) sum += fabs(w[j]);
  double m = sum > 1.0 ? sum : 1.0;
  int ex;
  double f = frexp(m, &ex);
  return ldexp(1.0, f == 0.5 ? ex - 1 : ex);
}

/* Cascadia Sec. 3.3, Eq. 1, combination and restoration: per row i with factor F_i,
 * y~_i = sum_j (w_ij / F_i) y_slots~[i,j] (ascending j), then y_i = A F_i y~_i, where y_slots~
 * holds the attenuated expert outputs E / A.  In real arithmetic y equals the unscaled combine. */
void orc_combine_restore(const double *y_slots_att, const double *weights, int T, int k_total, int H,
                         int att_log2, const uint8_t *token_mask, double *y) {
  const double A = ldexp(1.0, att_log2);
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    if (token_mask && !token_mask[t]) continue;
    const double *w = weights + (int64_t)t * k_total;
    const double F = orc_row_factor(w, k_total);
    for (int m = 0; m < H; ++m) {
      double acc = 0.0;
      for (int j = 0; j < k_total; ++j) acc += (w[j] / F) * y_slots_att[((int64_t)t * k_total + j) * H + m];
      y[(int64_t)t * H + m] = (A * F) * acc;
    }
  }
}

/* Weighted reduction [C31]: y[t,:] = sum_{j = 0..k_total-1, ascending} w[t,j] * y_slots[t*k_total+j,:].
 * token_mask (optional): only tokens with token_mask[t] != 0 are computed. */
void orc_combine(const double *y_slots, const double *weights, int T, int k_total, int H,
                 const uint8_t *token_mask, double *y) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    if (token_mask && !token_mask[t]) continue;
    for (int m = 0; m < H; ++m) {
      double acc = 0.0;
      for (int j = 0; j < k_total; ++j)
        acc += weights[(int64_t)t * k_total + j] * y_slots[((int64_t)t * k_total + j) * H + m];
      y[(int64_t)t * H + m] = acc;
    }
  }
}

/* ------------------------------------------------------------------------------------------ */
/* MX activation formats and the MX-mode expert FFN (readings stated in moe_oracle.h)          */
/* ------------------------------------------------------------------------------------------ */

int orc_mx_bits(int fmt) { return fmt == ORC_MX_FP8_E4M3 ? 8 : (fmt == ORC_MX_FP6_E2M3 ? 6 : 4); }
int orc_mx_emax(int fmt) { return fmt == ORC_MX_FP8_E4M3 ? 8 : 2; }

/* A code is sign | exponent field | fraction field.  Exponent field 0 gives the subnormal
 * fr * 2^(1 - bias - m_bits); otherwise (2^m_bits + fr) * 2^(ex - bias - m_bits). */
double orc_mx_value(int fmt, int code) {
  int e_bits, m_bits, bias;
  if (fmt == ORC_MX_FP8_E4M3) { e_bits = 4; m_bits = 3; bias = 7; }
  else if (fmt == ORC_MX_FP6_E2M3) { e_bits = 2; m_bits = 3; bias = 1; }
  else return orc_e2m1(code & 15);
  int sign = (code >> (e_bits + m_bits)) & 1;
  int ex = (code >> m_bits) & ((1 << e_bits) - 1), fr = code & ((1 << m_bits) - 1);
  if (fmt == ORC_MX_FP8_E4M3 && ex == 15 && fr == 7) return NAN;
  double v = ex == 0 ? ldexp((double)fr, 1 - bias - m_bits)
                     : ldexp((double)((1 << m_bits) + fr), ex - bias - m_bits);
  return sign ? -v : v;
}

/* Search over every non-negative code (their values ascend with the code): the nearest value to
 * |q| wins, an exact tie goes to the even code.  Past the largest value the largest code is the
 * nearest, which is the saturation.  The sign bit is the sign of q (so -0.0 and tiny negative
 * values give the negative-zero code). */
int orc_mx_encode(int fmt, double q) {
  const int bits = orc_mx_bits(fmt);
  const int n_pos = fmt == ORC_MX_FP8_E4M3 ? 127 : (1 << (bits - 1)); /* E4M3: 0x7F is NaN */
  const double a = fabs(q);
  int best = 0;
  double best_d = a;
  for (int c = 1; c < n_pos; ++c) {
    double d = fabs(a - orc_mx_value(fmt, c));
    if (d < best_d || (d == best_d && c % 2 == 0)) {
      best = c;
      best_d = d;
    }
  }
  return signbit(q) ? (best | (1 << (bits - 1))) : best;
}

/* X = 2^(floor(log2 amax) - emax), as the E8M0 code floor(log2 amax) - emax + 127 clamped to
 * [0, 254]; a block of zeros takes code 0.  frexp gives amax = f 2^ex with f in [0.5, 1), so
 * floor(log2 amax) = ex - 1 exactly. */
int orc_mx_scale_code(int fmt, double amax) {
  if (!(amax > 0.0)) return 0;
  int ex;
  frexp(amax, &ex);
  int c = (ex - 1) - orc_mx_emax(fmt) + 127;
  return c < 0 ? 0 : (c > 254 ? 254 : c);
}

void orc_mx_quantize(const double *v, int n_rows, int K, int fmt, uint8_t *codes, uint8_t *scales) {
  for (int r = 0; r < n_rows; ++r)
    for (int b = 0; b < K / 32; ++b) {
      const double *blk = v + (int64_t)r * K + 32 * b;
      double amax = 0.0;
      for (int i = 0; i < 32; ++i)
        if (fabs(blk[i]) > amax) amax = fabs(blk[i]);
      const int sc = orc_mx_scale_code(fmt, amax);
      scales[(int64_t)r * (K / 32) + b] = (uint8_t)sc;
      const double X = orc_e8m0(sc);
      for (int i = 0; i < 32; ++i) codes[(int64_t)r * K + 32 * b + i] = (uint8_t)orc_mx_encode(fmt, blk[i] / X);
    }
}

void orc_mx_dequantize(const uint8_t *codes, const uint8_t *scales, int n_rows, int K, int fmt,
                       double *out) {
  for (int r = 0; r < n_rows; ++r)
    for (int k = 0; k < K; ++k)
      out[(int64_t)r * K + k] =
          orc_mx_value(fmt, codes[(int64_t)r * K + k]) * orc_e8m0(scales[(int64_t)r * (K / 32) + k / 32]);
}

/* One vector through the MX round trip in place: v <- dequantize(quantize(v)). */
static void mx_round_trip(double *v, int K, int fmt) {
  uint8_t *c = (uint8_t *)malloc((size_t)K);
  uint8_t *s = (uint8_t *)malloc((size_t)K / 32 + 1);
  orc_mx_quantize(v, 1, K, fmt, c, s);
  orc_mx_dequantize(c, s, 1, K, fmt, v);
  free(c);
  free(s);
}

void orc_expert_ffn_mx(const uint16_t *x, int x_fmt, int T, int k_total, const orc_weights *W,
                       int act_fmt, const int32_t *offsets, const int32_t *sorted_slot,
                       const uint8_t *slot_mask, double *y_slots, double *h_pre) {
  grouped_ffn(x, x_fmt, T, k_total, W, act_fmt, 1.0, offsets, sorted_slot, slot_mask, y_slots, h_pre);
}

/* ------------------------------------------------------------------------------------------ */
/* Cross-check forms                                                                          */
/* ------------------------------------------------------------------------------------------ */

/* Dense decode of one packed MXFP4 matrix [n_rows][k], walking bytes rather than elements:
 * byte j of a row gives elements 2j (low nibble) and 2j+1 (high nibble), both in block
 * floor(2j/32). */
void orc_mxfp4_decode_matrix(const uint8_t *codes, const uint8_t *scales, int n_rows, int k,
                             double *out) {
  for (int n = 0; n < n_rows; ++n) {
    const uint8_t *row = codes + (int64_t)n * (k / 2);
    const uint8_t *srow = scales + (int64_t)n * (k / 32);
    for (int j = 0; j < k / 2; ++j) {
      double s = orc_e8m0(srow[(2 * j) / 32]);
      out[(int64_t)n * k + 2 * j] = orc_e2m1(row[j] & 0x0F) * s;
      out[(int64_t)n * k + 2 * j + 1] = orc_e2m1(row[j] >> 4) * s;
    }
  }
}

static void dense_expert(const orc_weights *W, int e, double *g, double *u, double *d) {
  const int H = W->hidden, I = W->inter;
  for (int n = 0; n < I; ++n)
    for (int k = 0; k < H; ++k) {
      g[(int64_t)n * H + k] = orc_weight(&W->gate, W->fmt, e, n, k);
      u[(int64_t)n * H + k] = orc_weight(&W->up, W->fmt, e, n, k);
    }
  for (int m = 0; m < H; ++m)
    for (int n = 0; n < I; ++n) d[(int64_t)m * I + n] = orc_weight(&W->down, W->fmt, e, m, n);
}

static void dense_apply(const double *g, const double *u, const double *d, int H, int I,
                        const double *xv, double *out) {
  double *h = (double *)malloc(sizeof(double) * (size_t)I);
  for (int n = 0; n < I; ++n) {
    double a = 0.0, b = 0.0;
    for (int k = 0; k < H; ++k) {
      a += g[(int64_t)n * H + k] * xv[k];
      b += u[(int64_t)n * H + k] * xv[k];
    }
    h[n] = orc_silu(a) * b;
  }
  for (int m = 0; m < H; ++m) {
    double acc = 0.0;
    for (int n = 0; n < I; ++n) acc += d[(int64_t)m * I + n] * h[n];
    out[m] = acc;
  }
  free(h);
}

/* Form B: per token, decode each selected expert densely and accumulate w * expert(x) -- no
 * bucketing, no slot buffer. */
void orc_layer_bruteforce(const uint16_t *x, int x_fmt, int T, int k_total, const orc_weights *W,
                          const int32_t *ids, const double *weights, double *y) {
  const int H = W->hidden, I = W->inter;
  double *g = (double *)malloc(sizeof(double) * (size_t)I * H);
  double *u = (double *)malloc(sizeof(double) * (size_t)I * H);
  double *d = (double *)malloc(sizeof(double) * (size_t)H * I);
  double *xv = (double *)malloc(sizeof(double) * (size_t)H);
  double *o = (double *)malloc(sizeof(double) * (size_t)H);
  for (int t = 0; t < T; ++t) {
    for (int k = 0; k < H; ++k) xv[k] = act_value(x, x_fmt, (int64_t)t * H + k);
    for (int m = 0; m < H; ++m) y[(int64_t)t * H + m] = 0.0;
    for (int j = 0; j < k_total; ++j) {
      int e = ids[(int64_t)t * k_total + j];
      dense_expert(W, e, g, u, d);
      dense_apply(g, u, d, H, I, xv, o);
      for (int m = 0; m < H; ++m) y[(int64_t)t * H + m] += weights[(int64_t)t * k_total + j] * o[m];
    }
  }
  free(g); free(u); free(d); free(xv); free(o);
}

/* Form C: a dense mixture over every expert, gate g_e = w_j when e = ids[t,j], else 0. */
void orc_layer_dense_mixture(const uint16_t *x, int x_fmt, int T, int k_total, const orc_weights *W,
                             const int32_t *ids, const double *weights, double *y) {
  const int H = W->hidden, E2 = W->n_experts;
  double *xv = (double *)malloc(sizeof(double) * (size_t)H);
  double *o = (double *)malloc(sizeof(double) * (size_t)H);
  for (int t = 0; t < T; ++t) {
    for (int k = 0; k < H; ++k) xv[k] = act_value(x, x_fmt, (int64_t)t * H + k);
    for (int m = 0; m < H; ++m) y[(int64_t)t * H + m] = 0.0;
    for (int e = 0; e < E2; ++e) {
      double gate = 0.0;
      for (int j = 0; j < k_total; ++j)
        if (ids[(int64_t)t * k_total + j] == e) gate = weights[(int64_t)t * k_total + j];
      orc_expert_apply(W, e, xv, o);
      for (int m = 0; m < H; ++m) y[(int64_t)t * H + m] += gate * o[m];
    }
  }
  free(xv); free(o);
}

/* Form D [C34]: the unsliced dense SwiGLU FFN with binary16 weights wg, wu [I][H] and wd [H][I]:
 * y = W_d [SiLU(W_g x) (.) W_u x]. */
void orc_dense_ffn_f16(const uint16_t *x, int x_fmt, int T, int H, int I, const uint16_t *wg,
                       const uint16_t *wu, const uint16_t *wd, double *y) {
  for (int t = 0; t < T; ++t) {
    double *h = (double *)malloc(sizeof(double) * (size_t)I);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < I; ++n) {
      double a = 0.0, b = 0.0;
      for (int k = 0; k < H; ++k) {
        double xv = act_value(x, x_fmt, (int64_t)t * H + k);
        a += orc_f16(wg[(int64_t)n * H + k]) * xv;
        b += orc_f16(wu[(int64_t)n * H + k]) * xv;
      }
      h[n] = orc_silu(a) * b;
    }
#pragma omp parallel for schedule(static)
    for (int m = 0; m < H; ++m) {
      double acc = 0.0;
      for (int n = 0; n < I; ++n) acc += orc_f16(wd[(int64_t)m * I + n]) * h[n];
      y[(int64_t)t * H + m] = acc;
    }
    free(h);
  }
}
