// Router: logits, softmax, top-k with renormalised weights, shared-expert slots.
//
// Stage 1 (route_logits_kernel): partial[s][t][e] = sum over the s-th slice of the hidden dim of
//   x[t,h] * w_router[e,h], fp32 FMA.  A workgroup owns a 32-token x 64-expert tile and one
//   hidden slice; both operand tiles are staged through LDS in 32-wide k steps.  Splitting the
//   hidden dimension spreads the router-weight read over many CUs when T is small (decode).
// Stage 2 (route_select_kernel): one wave per token sums the slices in slice order, adds the
//   bias, takes max / exp / sum over the E logits held across the wave, then picks top_k rounds of
//   (largest logit, lowest index) by wave argmax and writes ids, renormalised weights and probs.
// The selection order and renormalisation follow the routed-MoE statement (softmax, top-k, weights
// renormalised to 1); shared experts are always-included slots after the routed ones (Cascadia,
// Sec. 3.1).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {
constexpr int kTT = 32;   // tokens per tile
constexpr int kTE = 64;   // experts per tile
constexpr int kBK = 32;   // hidden elements per LDS step

template <int XF16>
__device__ __forceinline__ float act_to_f32(uint16_t b) {
  if constexpr (XF16) {
    return (float)bitcast<_Float16>(b);
  } else {
    return __uint_as_float((uint32_t)b << 16);
  }
}

template <int XF16>
__global__ __launch_bounds__(256) void route_logits_kernel(const uint16_t* __restrict__ x, int T, int H,
                                                           const float* __restrict__ w, int E, int k_per_split,
                                                           float* __restrict__ partial) {
  __shared__ float xs[kBK][kTT + 1];
  __shared__ float ws[kBK][kTE + 4];
  const int tid = threadIdx.x;
  const int e0 = blockIdx.x * kTE;
  const int t0 = blockIdx.y * kTT;
  const int split = blockIdx.z;
  const int h_begin = split * k_per_split;
  const int h_end = min(H, h_begin + k_per_split);
  const int tx = tid & 15;   // experts tx*4 .. tx*4+3
  const int ty = tid >> 4;   // tokens ty*2, ty*2+1
  float acc[2][4] = {};
  for (int h0 = h_begin; h0 < h_end; h0 += kBK) {
    // x tile: 32 tokens x 32 hidden, 4 elements per thread, k fastest
#pragma unroll
    for (int q = 0; q < (kTT * kBK) / 256; ++q) {
      int idx = tid + q * 256;
      int kk = idx % kBK, tt = idx / kBK;
      int t = t0 + tt, h = h0 + kk;
      xs[kk][tt] = (t < T && h < h_end) ? act_to_f32<XF16>(x[(int64_t)t * H + h]) : 0.0f;
    }
    // w tile: 64 experts x 32 hidden, 8 elements per thread
#pragma unroll
    for (int q = 0; q < (kTE * kBK) / 256; ++q) {
      int idx = tid + q * 256;
      int kk = idx % kBK, ee = idx / kBK;
      int e = e0 + ee, h = h0 + kk;
      ws[kk][ee] = (e < E && h < h_end) ? w[(int64_t)e * H + h] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < kBK; ++kk) {
      float a0 = xs[kk][ty * 2], a1 = xs[kk][ty * 2 + 1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float b = ws[kk][tx * 4 + j];
        acc[0][j] += a0 * b;
        acc[1][j] += a1 * b;
      }
    }
    __syncthreads();
  }
  float* out = partial + (int64_t)split * T * E;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int t = t0 + ty * 2 + i;
    if (t >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = e0 + tx * 4 + j;
      if (e < E) out[(int64_t)t * E + e] = acc[i][j];
    }
  }
}

template <int VPL>
__global__ __launch_bounds__(256) void route_select_kernel(const float* __restrict__ partial, int splits, int T,
                                                           int E, const float* __restrict__ bias, int top_k,
                                                           int n_shared, int32_t* __restrict__ ids,
                                                           float* __restrict__ weights, float* __restrict__ probs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // whole wave leaves together; no block-wide barrier follows
  float L[VPL];
  // Sum the hidden-dimension slices in slice order; the loads of 8 slices are issued together.
#pragma unroll
  for (int v = 0; v < VPL; ++v) L[v] = 0.0f;
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float part[8][VPL];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int e = lane + 64 * v;
        part[q][v] = (s0 + q < splits && e < E) ? partial[((int64_t)(s0 + q) * T + t) * E + e] : 0.0f;
      }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int v = 0; v < VPL; ++v) L[v] += part[q][v];
  }
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = lane + 64 * v;
    L[v] = (e < E) ? L[v] + (bias ? bias[e] : 0.0f) : -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int v = 0; v < VPL; ++v) mx = fmaxf(mx, L[v]);
  mx = wave_max(mx);
  float part = 0.0f;
#pragma unroll
  for (int v = 0; v < VPL; ++v) part += (lane + 64 * v < E) ? expf(L[v] - mx) : 0.0f;
  const float den = wave_sum(part);
  if (probs) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      int e = lane + 64 * v;
      if (e < E) probs[(int64_t)t * E + e] = expf(L[v] - mx) / den;
    }
  }
  // k rounds of wave argmax over (logit desc, index asc).  The winner of round j is kept by lane
  // j % 64 in register q = j / 64 (k_total <= MOE_MAX_SLOTS_PER_TOKEN = 4 * 64).
  uint32_t taken = 0;
  float psum = 0.0f;
  int my_id[4] = {0, 0, 0, 0};
  float my_p[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < top_k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      int e = lane + 64 * v;
      bool free_ = e < E && !((taken >> v) & 1u);
      if (free_ && (L[v] > bv || (L[v] == bv && e < bi))) {
        bv = L[v];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float ov = __shfl_xor(bv, o, kWave);
      int oi = __shfl_xor(bi, o, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    const float p = expf(bv - mx) / den;
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
    weights[(int64_t)t * k_total + j] = wgt;
  }
}
}  // namespace

int route_splits(int T, int H, int E) {
  const int tiles = ((E + kTE - 1) / kTE) * ((T + kTT - 1) / kTT);
  const int max_splits = min(16, (H + 255) / 256);  // at least 256 hidden elements per slice
  int s = (512 + tiles - 1) / tiles;
  if (s > max_splits) s = max_splits;
  if (s < 1) s = 1;
  return s;
}

hipError_t launch_route(const void* x, int x_fp16, int T, int H, const float* w_router, const float* bias, int E,
                        int top_k, int n_shared, int32_t* ids, float* weights, float* probs, float* partial,
                        int splits, hipStream_t stream) {
  int per = (H + splits - 1) / splits;
  per = (per + kBK - 1) / kBK * kBK;
  dim3 g1((E + kTE - 1) / kTE, (T + kTT - 1) / kTT, splits);
  if (x_fp16)
    route_logits_kernel<1><<<g1, 256, 0, stream>>>((const uint16_t*)x, T, H, w_router, E, per, partial);
  else
    route_logits_kernel<0><<<g1, 256, 0, stream>>>((const uint16_t*)x, T, H, w_router, E, per, partial);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  dim3 g2((T + 3) / 4);
  const int vpl = (E + 63) / 64;
#define MOE_SEL(V) route_select_kernel<V><<<g2, 256, 0, stream>>>(partial, splits, T, E, bias, top_k, n_shared, ids, weights, probs)
  if (vpl <= 1) MOE_SEL(1);
  else if (vpl <= 2) MOE_SEL(2);
  else if (vpl <= 4) MOE_SEL(4);
  else if (vpl <= 8) MOE_SEL(8);
  else MOE_SEL(16);
#undef MOE_SEL
  return hipGetLastError();
}

}  // namespace moe
