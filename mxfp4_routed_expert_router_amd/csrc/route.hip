// Router: logits, softmax, top-k with renormalised weights, shared-expert slots.
//
// Stage 1 (route_logits_kernel): partial[s][t][e] = sum over the s-th slice of the hidden dim of
//   x[t,h] * w_router[e,h] on the matrix cores.  w_router (fp32) is split exactly into three bf16
//   terms, hi = bf16(w), mid = bf16(w - hi), lo = bf16(w - hi - mid) (each difference is exact, so
//   hi + mid + lo = w for every normal w); x is bf16 (or fp16) and exact; every product is exact in
//   fp32 and v_mfma_f32_16x16x32 accumulates in fp32, so the logits are fp32-accurate.  One wave
//   owns 16 experts x 16*MT tokens x one hidden slice; slices spread the router-weight read over
//   many CUs when T is small.
// Stage 2 (route_select_kernel): one wave per token sums the slices in slice order, adds the
//   bias, takes max / exp / sum over the E logits held across the wave, then picks top_k rounds of
//   (largest logit, lowest index) by wave argmax and writes ids, renormalised weights and probs.
// The selection order and renormalisation follow the routed-MoE statement (softmax, top-k, weights
// renormalised to 1); shared experts are always-included slots after the routed ones (Cascadia,
// Sec. 3.1).
#include "bucket.hpp"
#include "tiles.hpp"

namespace moe {

namespace {
constexpr int kMaxSplits = 32;

// Round to nearest even (v_cvt_pk_bf16_f32, two values per instruction).
__device__ __forceinline__ bf16x8 to_bf16x8_rne(const float (&v)[8]) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)v[j];
  return r;
}

// XF16: activations are fp16 (converted exactly to fp32 and re-split into two bf16 terms, since an
// fp16 value has 11 significant bits).  VEC: 16-byte loads (aligned w_router rows, H % 8 == 0).
// A wave computes one 16-expert x 16-token tile over its K slice, kU k-steps of 32 at a time with
// all of their loads issued first (the kernel is latency-bound: a load-then-use loop would wait a
// full memory latency per k-step): 8 with one token tile per wave (measured 6.7 -> 6.2 us at
// T <= 32), 4 with more (their activation registers grow with the tiles).
template <int MT>
constexpr int route_ku() { return MT == 1 ? 8 : 4; }

// MT: 16-token tiles per wave (more than one when T is large: each router-weight fragment, and its
// three-way split, then serves MT token tiles, which cuts the weight re-reads through L2).
template <int XF16, int VEC, int MT>
__global__ __launch_bounds__(64) void route_logits_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                          const float* __restrict__ w, int E, int ks_per_split,
                                                          float* __restrict__ partial) {
  const int lane = threadIdx.x, l16 = lane & 15, lq = lane >> 4;
  const int e = blockIdx.x * 16 + l16;
  const int split = blockIdx.z;
  const int nks = (H + 31) / 32;
  const int ks0 = split * ks_per_split, ks1 = min(ks0 + ks_per_split, nks);
  const float* wrow = w + (int64_t)(e < E ? e : 0) * H;
  constexpr int kU = route_ku<MT>();
  const uint16_t* xrow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int t = (blockIdx.y * MT + mt) * 16 + l16;
    xrow[mt] = x + (int64_t)(t < T ? t : 0) * H;
  }
  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // kG groups of kU k-steps are loaded before any of them is used (two with one token tile: the
  // 14 k-steps of a small call's slice in one memory round trip; separate arrays keep them in
  // registers)
  constexpr int kG = MT == 1 ? 2 : 1;
  auto load_group = [&](int ks, float (&wv)[kU][8], uint16_t (&xv)[kU][MT][8]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      // k-steps past the slice reload the slice's last step and are skipped below
      const int k = min(ks + u, ks1 - 1) * 32 + 8 * lq;  // this lane's 8 hidden indices
      if (VEC && k + 8 <= H) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(wrow + k);
        const f32x4 b = *reinterpret_cast<const f32x4*>(wrow + k + 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          wv[u][j] = a[j];
          wv[u][4 + j] = b[j];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const u32x4 q = ld16(xrow[mt] + k);
          __builtin_memcpy(xv[u][mt], &q, 16);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          wv[u][j] = (k + j < H) ? wrow[k + j] : 0.f;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) xv[u][mt][j] = (k + j < H) ? xrow[mt][k + j] : 0;
        }
      }
    }
  };
  auto compute_group = [&](int ks, float (&wv)[kU][8], uint16_t (&xv)[kU][MT][8]) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (ks + u >= ks1) break;  // uniform
      float r[8];
      if (e >= E) {
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[u][j] = 0.f;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if ((blockIdx.y * MT + mt) * 16 + l16 >= T) {
#pragma unroll
          for (int j = 0; j < 8; ++j) xv[u][mt][j] = 0;
        }
      const bf16x8 hi = to_bf16x8_rne(wv[u]);
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] = wv[u][j] - (float)hi[j];
      const bf16x8 mid = to_bf16x8_rne(r);
#pragma unroll
      for (int j = 0; j < 8; ++j) r[j] -= (float)mid[j];
      const bf16x8 lo = to_bf16x8_rne(r);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (XF16) {
          // fp16 -> fp32 exactly, then two bf16 terms (8 + 8 >= 11 significant bits)
          float xf[8], xr2[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) xf[j] = (float)bitcast<_Float16>(xv[u][mt][j]);
          const bf16x8 xh = to_bf16x8_rne(xf);
#pragma unroll
          for (int j = 0; j < 8; ++j) xr2[j] = xf[j] - (float)xh[j];
          const bf16x8 xl = to_bf16x8_rne(xr2);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, xh, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, xh, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, xh, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, xl, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, xl, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, xl, acc[mt], 0, 0, 0);
        } else {
          bf16x8 b;
          __builtin_memcpy(&b, xv[u][mt], 16);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, b, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(mid, b, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, b, acc[mt], 0, 0, 0);
        }
      }
    }
  };
  for (int ks = ks0; ks < ks1; ks += kG * kU) {
    float wa[kU][8];
    uint16_t xa[kU][MT][8];
    load_group(ks, wa, xa);
    if constexpr (kG == 2) {
      float wb[kU][8];
      uint16_t xb[kU][MT][8];
      if (ks + kU < ks1) load_group(ks + kU, wb, xb);  // uniform
      compute_group(ks, wa, xa);
      if (ks + kU < ks1) compute_group(ks + kU, wb, xb);
    } else {
      compute_group(ks, wa, xa);
    }
  }
  // D: lane holds experts 16*blockIdx.x + 4*lq + i of token l16 of each token tile
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int t = (blockIdx.y * MT + mt) * 16 + l16;
    if (t < T) {
      float* out = partial + ((int64_t)split * T + t) * E;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ee = blockIdx.x * 16 + 4 * lq + i;
        if (ee < E) out[ee] = acc[mt][i];
      }
    }
  }
}

// Lane l holds experts VPL l .. VPL l + VPL - 1 (contiguous, so with E % VPL == 0 -- VEC -- a
// lane reads each slice's VPL partial logits with one vector load, and writes its probabilities
// together).
//
// SIG selects the sigmoid router of Cascadia Sec. 3.1 instead of the softmax one: scores
// s = 1 / (1 + e^-L), selection by s + bias (the bias moves the choice only), weights
// routed_scale * s / (sum of the selected s), shared slots shared_weight; `probs` receives s.
// select_token: the selection of token t by the calling wave (t wave-uniform, t < T).
template <int VPL, bool VEC, bool SIG>
__device__ __forceinline__ void select_token(const float* __restrict__ partial, int splits, int T, int E,
                                             const float* __restrict__ bias, int top_k, int n_shared,
                                             int32_t* __restrict__ ids, float* __restrict__ weights,
                                             float* __restrict__ probs, float routed_scale, float shared_weight,
                                             int t, int* lds_ids = nullptr) {
  const int lane = threadIdx.x & 63;
  const int e0 = VPL * lane;
  float L[VPL];
  // Sum the hidden-dimension slices in slice order, kSplitChunk slices at a time (the loads of a
  // chunk issued together: all of them with at most 4 experts per lane).  A lane past E reads the
  // last valid lane's values and discards them.
  constexpr int kSplitChunk = VPL <= 4 ? kMaxSplits : 16;
#pragma unroll
  for (int v = 0; v < VPL; ++v) L[v] = 0.0f;
#pragma unroll
  for (int q0 = 0; q0 < kMaxSplits; q0 += kSplitChunk) {
    if (q0 >= splits) break;  // uniform
    float part[kSplitChunk][VPL];
#pragma unroll
    for (int qq = 0; qq < kSplitChunk; ++qq) {
      const int q = q0 + qq;
      if (VEC) {
        const float* src = partial + ((int64_t)min(q, splits - 1) * T + t) * E + min(e0, E - VPL);
        typedef float fv __attribute__((ext_vector_type(VPL)));
        fv val;
        __builtin_memcpy(&val, __builtin_assume_aligned(src, VPL >= 4 ? 16 : 4 * VPL), 4 * VPL);  // workspace: 16-byte aligned
#pragma unroll
        for (int v = 0; v < VPL; ++v) part[qq][v] = (q < splits && e0 < E) ? val[v] : 0.0f;
      } else {
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          const int e = e0 + v;
          part[qq][v] = (q < splits && e < E) ? partial[((int64_t)q * T + t) * E + e] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int qq = 0; qq < kSplitChunk; ++qq) L[v] += part[qq][v];
  }
  if constexpr (SIG) {
    // scores, and the selection keys score + bias; the winner of a round reads its score from the
    // lane that holds it
    float sv[VPL];
    uint32_t kh[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = e0 + v;
      sv[v] = (e < E) ? 1.0f / (1.0f + expf(-L[v])) : 0.0f;
      kh[v] = (e < E) ? f32_order_key(sv[v] + (bias ? bias[e] : 0.0f)) : 0u;
      if (probs && e < E) probs[(int64_t)t * E + e] = sv[v];
    }
    float psum = 0.0f;
    int my_id[4] = {0, 0, 0, 0};
    float my_p[4] = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < top_k; ++j) {
      uint32_t m = kh[0];
#pragma unroll
      for (int v = 1; v < VPL; ++v) m = max(m, kh[v]);
      m = wave_max_u32_dpp(m);
      int bi = INT_MAX;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const uint64_t b = __ballot(kh[v] == m);
        if (b) bi = min(bi, VPL * (__builtin_ffsll((long long)b) - 1) + v);
      }
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        if (e0 + v == bi) kh[v] = 0u;
      const int bv = bi % VPL;  // uniform: every lane offers its score of that register
      float cand = sv[0];
#pragma unroll
      for (int v = 1; v < VPL; ++v) cand = (v == bv) ? sv[v] : cand;
      const float p = __shfl(cand, bi / VPL, kWave);
      psum += p;
      if ((j & 63) == lane) {
        const int q = j >> 6;
#pragma unroll
        for (int z = 0; z < 4; ++z)
          if (z == q) {
            my_id[z] = bi;
            my_p[z] = p;
          }
      }
    }
    const int k_total = top_k + n_shared;
#pragma unroll
    for (int z = 0; z < 4; ++z) {
      const int j = lane + 64 * z;
      if (j >= k_total) break;
      const bool routed = j < top_k;
      ids[(int64_t)t * k_total + j] = routed ? my_id[z] : E + (j - top_k);
      if (lds_ids) lds_ids[t * k_total + j] = routed ? my_id[z] : E + (j - top_k);
      weights[(int64_t)t * k_total + j] = routed ? routed_scale * (my_p[z] / psum) : shared_weight;
    }
    return;
  }
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = e0 + v;
    L[v] = (e < E) ? L[v] + (bias ? bias[e] : 0.0f) : -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < VPL; ++v) mx = fmaxf(mx, L[v]);
  mx = wave_max_dpp(mx);
  float esum = 0.0f;
#pragma unroll
  for (int v = 0; v < VPL; ++v) esum += (e0 + v < E) ? expf(L[v] - mx) : 0.0f;
  const float den = wave_sum_dpp(esum);
  if (probs) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = e0 + v;
      if (e < E) probs[(int64_t)t * E + e] = expf(L[v] - mx) / den;
    }
  }
  // k rounds of wave argmax over (logit desc, index asc).  Each lane first sorts its VPL
  // (order key, expert) pairs, descending by key and, among equal keys, ascending by expert (a
  // stable exchange network on keys that start in expert order); a round is then one 32-bit DPP
  // maximum of the lanes' heads, one ballot for the lowest lane holding it (lanes hold ascending
  // experts, so that is the lowest index with the largest key), a read of that lane's head expert,
  // and the winning lane dropping its head.  Padded experts carry key 0, below every logit's key.
  // The winner of round j is kept by lane j % 64 in register q = j / 64 (k_total <=
  // MOE_MAX_SLOTS_PER_TOKEN = 4 * 64); the probabilities and their sum follow the rounds.
  uint32_t sk[VPL];
  int si[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    sk[v] = (e0 + v < E) ? f32_order_key(L[v]) : 0u;
    si[v] = e0 + v;
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i)
#pragma unroll
    for (int v = VPL - 1; v > i; --v)
      if (sk[v] > sk[v - 1]) {
        const uint32_t tk = sk[v];
        sk[v] = sk[v - 1];
        sk[v - 1] = tk;
        const int ti = si[v];
        si[v] = si[v - 1];
        si[v - 1] = ti;
      }
  int my_id[4] = {0, 0, 0, 0};
  uint32_t my_key[4] = {0u, 0u, 0u, 0u};
  for (int j = 0; j < top_k; ++j) {
    const uint32_t m = wave_max_u32_dpp(sk[0]);
    const int wl = __builtin_ffsll((long long)__ballot(sk[0] == m)) - 1;  // uniform
    const int bi = __builtin_amdgcn_readlane(si[0], wl);
    if (lane == wl) {
#pragma unroll
      for (int v = 0; v + 1 < VPL; ++v) {
        sk[v] = sk[v + 1];
        si[v] = si[v + 1];
      }
      sk[VPL - 1] = 0u;
    }
    if ((j & 63) == lane) {
      const int q = j >> 6;
#pragma unroll
      for (int z = 0; z < 4; ++z)
        if (z == q) {
          my_id[z] = bi;
          my_key[z] = m;
        }
    }
  }
  float my_p[4];
  float psum_l = 0.0f;
#pragma unroll
  for (int z = 0; z < 4; ++z) {
    my_p[z] = (lane + 64 * z < top_k) ? expf(f32_from_order_key(my_key[z]) - mx) / den : 0.0f;
    psum_l += my_p[z];
  }
  const float psum = wave_sum_dpp(psum_l);
  const int k_total = top_k + n_shared;
#pragma unroll
  for (int z = 0; z < 4; ++z) {
    const int j = lane + 64 * z;
    if (j >= k_total) break;
    int id;
    float wgt;
    if (j < top_k) {
      id = my_id[z];
      wgt = my_p[z] / psum;
    } else {
      id = E + (j - top_k);
      wgt = 1.0f;
    }
    ids[(int64_t)t * k_total + j] = id;
    if (lds_ids) lds_ids[t * k_total + j] = id;
    weights[(int64_t)t * k_total + j] = wgt;
  }
}

template <int VPL, bool VEC, bool SIG>
__global__ __launch_bounds__(256) void route_select_kernel(const float* __restrict__ partial, int splits, int T,
                                                           int E, const float* __restrict__ bias, int top_k,
                                                           int n_shared, int32_t* __restrict__ ids,
                                                           float* __restrict__ weights, float* __restrict__ probs,
                                                           float routed_scale, float shared_weight) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave leaves together; no block-wide barrier follows
  select_token<VPL, VEC, SIG>(partial, splits, T, E, bias, top_k, n_shared, ids, weights, probs, routed_scale,
                              shared_weight, t);
}

// The router's selection, the bucketing and the expert FFN's tile table in one workgroup, for calls
// of at most kFusedTokens tokens: wave t selects token t, and after a barrier (which makes the
// workgroup's ids visible to all its waves) the workgroup buckets the slots and builds the tile
// table from the bucket offsets.  (With several selection workgroups the bucketing would wait for
// all of them behind a device-scope release, an atomic ticket and an acquire; measured on the
// sweep layer, that tail was slower than the separate bucketing and plan launches at 32 tokens and
// more, and no faster below, so larger calls take the separate kernels.)
constexpr int kFusedTokens = kBucketChunk / 64;
struct FusedTail {
  int n_buckets;
  int32_t *counts, *offsets, *sorted_slot, *slot_pos;
  TileEntry* table;  // NULL: no tile table
  int rows_per_tile, n_entries;
};

template <int VPL, bool VEC, bool SIG>
__global__ __launch_bounds__(kBucketChunk) void route_select_bucket_kernel(
    const float* __restrict__ partial, int splits, int T, int E, const float* __restrict__ bias, int top_k,
    int n_shared, int32_t* __restrict__ ids, float* __restrict__ weights, float* __restrict__ probs,
    float routed_scale, float shared_weight, FusedTail ft) {
  extern __shared__ int lds[];
  const int t = threadIdx.x >> 6;  // one workgroup: T <= kFusedTokens
  const int n_slots = T * (top_k + n_shared);
  const bool small = n_slots <= kSmallSlots;  // uniform: the ids stay in LDS for the small path
  if (t < T)
    select_token<VPL, VEC, SIG>(partial, splits, T, E, bias, top_k, n_shared, ids, weights, probs, routed_scale,
                                shared_weight, t, small ? lds : nullptr);
  __syncthreads();
  if (small) {
    bucket_small_block(lds, n_slots, ft.n_buckets, ft.counts, ft.offsets, ft.sorted_slot, ft.slot_pos, ft.table,
                       ft.rows_per_tile, ft.n_entries, lds + kSmallSlots);
    return;
  }
  const int total = bucket_fused_block(ids, n_slots, ft.n_buckets, ft.counts, ft.offsets, ft.sorted_slot,
                                       ft.slot_pos, lds);
  if (ft.table)
    tiles_from_offsets_block(fused_base(lds, ft.n_buckets), total, ft.n_buckets, n_slots, ft.rows_per_tile,
                             ft.n_entries, ft.table, lds);
}
}  // namespace

// Each wave computes one 16-expert x 16-token tile over a K slice.  The logits are latency-bound,
// so with few tiles, many small waves (about 2048, one tile each) beat fewer waves that reuse each
// router-weight fragment for more tokens.  From about 128 tiles (e.g. 256 experts and 128 or
// more tokens) two token tiles per wave are faster (measured: 29 -> 24.5 us for 176 tokens x
// 256 experts x 7168), and four from 8192 tiles.
int route_mt(int T, int E) {
  const int64_t g1 = (int64_t)((E + 15) / 16) * ((T + 15) / 16);
  return g1 >= 4 * 2048 ? 4 : (g1 >= 128 ? 2 : 1);
}

int route_splits(int T, int H, int E) {
  const int mt = route_mt(T, E);
  const int64_t groups = (int64_t)((E + 15) / 16) * ((T + 16 * mt - 1) / (16 * mt));
  const int nks = (H + 31) / 32;
  int s = (int)((2048 + groups - 1) / groups);
  const int cap = nks / 4 < 1 ? 1 : nks / 4;  // at least 4 k-steps of 32 per slice
  if (s > cap) s = cap;
  // up to kMaxSplits slices for calls of one 16-expert x 16-token group set (T <= 16 with 256
  // experts: shorter slices shorten the latency-bound waves), half that beyond (at 176 tokens 22
  // slices took the logits from 15.8 to 18.2 us)
  const int smax = groups <= 16 ? kMaxSplits : kMaxSplits / 2;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  return s;
}

template <int XF16, int VEC>
void launch_logits(const void* x, int T, int H, const float* w, int E, int splits, float* partial, hipStream_t st) {
  const int nks = (H + 31) / 32;
  const int per = (nks + splits - 1) / splits;
  const int mt = route_mt(T, E);
  const dim3 g((E + 15) / 16, (T + 16 * mt - 1) / (16 * mt), splits);
  const uint16_t* xx = (const uint16_t*)x;
  if (mt == 4) route_logits_kernel<XF16, VEC, 4><<<g, 64, 0, st>>>(xx, T, H, w, E, per, partial);
  else if (mt == 2) route_logits_kernel<XF16, VEC, 2><<<g, 64, 0, st>>>(xx, T, H, w, E, per, partial);
  else route_logits_kernel<XF16, VEC, 1><<<g, 64, 0, st>>>(xx, T, H, w, E, per, partial);
}

// Logits for every form of the router call.
hipError_t launch_route_logits(const void* x, int x_fp16, int T, int H, const float* w_router, int E, float* partial,
                               int splits, hipStream_t stream) {
  const bool vec = ((uintptr_t)w_router % 16 == 0) && (H % 8 == 0);
  if (x_fp16) {
    if (vec) launch_logits<1, 1>(x, T, H, w_router, E, splits, partial, stream);
    else launch_logits<1, 0>(x, T, H, w_router, E, splits, partial, stream);
  } else {
    if (vec) launch_logits<0, 1>(x, T, H, w_router, E, splits, partial, stream);
    else launch_logits<0, 0>(x, T, H, w_router, E, splits, partial, stream);
  }
  return hipGetLastError();
}

hipError_t launch_route(const void* x, int x_fp16, int T, int H, const float* w_router, const float* bias, int E,
                        int top_k, int n_shared, int32_t* ids, float* weights, float* probs, float* partial,
                        int splits, hipStream_t stream, bool sigmoid, float routed_scale, float shared_weight) {
  hipError_t err = launch_route_logits(x, x_fp16, T, H, w_router, E, partial, splits, stream);
  if (err != hipSuccess) return err;
  dim3 g2((T + 3) / 4);
  const int vpl = (E + 63) / 64;
#define MOE_SEL2(V, SG)                                                                                       \
  {                                                                                                          \
    if (E % V == 0)                                                                                          \
      route_select_kernel<V, true, SG><<<g2, 256, 0, stream>>>(partial, splits, T, E, bias, top_k, n_shared,  \
                                                               ids, weights, probs, routed_scale,            \
                                                               shared_weight);                               \
    else                                                                                                     \
      route_select_kernel<V, false, SG><<<g2, 256, 0, stream>>>(partial, splits, T, E, bias, top_k, n_shared, \
                                                                ids, weights, probs, routed_scale,           \
                                                                shared_weight);                              \
  }
#define MOE_SEL(V)          \
  {                         \
    if (sigmoid)            \
      MOE_SEL2(V, true)     \
    else                    \
      MOE_SEL2(V, false)    \
  }
  if (vpl <= 1) MOE_SEL(1)
  else if (vpl <= 2) MOE_SEL(2)
  else if (vpl <= 4) MOE_SEL(4)
  else if (vpl <= 8) MOE_SEL(8)
  else MOE_SEL(16)
#undef MOE_SEL
#undef MOE_SEL2
  return hipGetLastError();
}

bool route_bucket_fusable(int T, int k_total, int n_buckets) {
  return T <= kFusedTokens && (int64_t)T * k_total <= (int64_t)kFusedChunks * kBucketChunk &&
         n_buckets <= MOE_MAX_EXPERTS;
}

hipError_t launch_route_bucket(const void* x, int x_fp16, int T, int H, const float* w_router, const float* bias,
                               int E, int top_k, int n_shared, int32_t* ids, float* weights, float* probs,
                               float* partial, int splits, int n_buckets, int32_t* counts, int32_t* offsets,
                               int32_t* sorted_slot, int32_t* slot_pos, void* table, int rows_per_tile,
                               int64_t n_entries, hipStream_t stream) {
  if (!route_bucket_fusable(T, top_k + n_shared, n_buckets)) return hipErrorInvalidValue;
  hipError_t err = launch_route_logits(x, x_fp16, T, H, w_router, E, partial, splits, stream);
  if (err != hipSuccess) return err;
  FusedTail ft{n_buckets, counts, offsets, sorted_slot, slot_pos, (TileEntry*)table, rows_per_tile, (int)n_entries};
  const dim3 g(1);
  const size_t lds = sizeof(int) * std::max<size_t>(bucket_fused_lds_ints(n_buckets), kSmallSlots + kSmallLdsInts);
  const int vpl = (E + 63) / 64;
#define MOE_FSEL(V)                                                                                            \
  {                                                                                                            \
    if (E % V == 0)                                                                                            \
      route_select_bucket_kernel<V, true, false><<<g, kBucketChunk, lds, stream>>>(                             \
          partial, splits, T, E, bias, top_k, n_shared, ids, weights, probs, 1.0f, 1.0f, ft);                  \
    else                                                                                                       \
      route_select_bucket_kernel<V, false, false><<<g, kBucketChunk, lds, stream>>>(                            \
          partial, splits, T, E, bias, top_k, n_shared, ids, weights, probs, 1.0f, 1.0f, ft);                  \
  }
  if (vpl <= 1) MOE_FSEL(1)
  else if (vpl <= 2) MOE_FSEL(2)
  else if (vpl <= 4) MOE_FSEL(4)
  else if (vpl <= 8) MOE_FSEL(8)
  else MOE_FSEL(16)
#undef MOE_FSEL
  return hipGetLastError();
}

}  // namespace moe
