// Weighted combine (Cascadia, Sec. 3.1 "weighted reduction"; FP32 output as in Cascadia Fig. 2):
//   y[t, :] = sum_{j ascending} weights[t, j] * y_slots[t*k + j, :]
// One thread owns four consecutive outputs of one token (16-byte loads and stores); no atomics.
// The slots are read in batches of kBatch with all of a batch's loads issued before the first
// multiply-add (a load-then-use loop waits one memory latency per slot); indices past the last
// slot re-read the last one (a cache hit) and their products are dropped.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {
constexpr int kBatch = 8;

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_slots,
                                                      const float* __restrict__ weights, int T, int k_total,
                                                      int H, float* __restrict__ y) {
  const int h4 = H >> 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * h4) return;
  const int t = (int)(i / h4), c = (int)(i % h4) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const float* src = y_slots + (int64_t)t * k_total * H + c;
  const float* wt = weights + (int64_t)t * k_total;
  for (int j0 = 0; j0 < k_total; j0 += kBatch) {
    float w[kBatch];
    f32x4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = min(j0 + u, k_total - 1);
      w[u] = wt[j];
      v[u] = *reinterpret_cast<const f32x4*>(src + (int64_t)j * H);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {  // selects, not a branch: the loads stay ahead of the adds
      const bool ok = j0 + u < k_total;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float s = acc[e] + w[u] * v[u][e];
        acc[e] = ok ? s : acc[e];
      }
    }
  }
  *reinterpret_cast<f32x4*>(y + (int64_t)t * H + c) = acc;
}
// Combination and FP32 restoration of the range-managed path (Cascadia Sec. 3.3, Eq. 1).  Per
// token: F = 2^ceil(log2 max(1, sum_j |w_j|)) (fp32 sum in ascending j; frexp gives the exponent
// exactly), y~ = binary16(sum_j (w_j / F) * y16[j]) (fp32 accumulation in ascending j; w_j / F is
// exact), then y = y~ * (A * F) in fp32 -- exact, being a product of powers of two with a binary16
// value.  One thread per four outputs of a token, as in combine_kernel.
__global__ __launch_bounds__(256) void combine_restore_kernel(const uint16_t* __restrict__ y16,
                                                              const float* __restrict__ weights, int T, int k_total,
                                                              int H, float A, float* __restrict__ y) {
  const int h4 = H >> 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * h4) return;
  const int t = (int)(i / h4), c = (int)(i % h4) * 4;
  const float* wt = weights + (int64_t)t * k_total;
  float sum = 0.0f;
  for (int j = 0; j < k_total; ++j) sum += fabsf(wt[j]);
  int ex;
  const float mant = frexpf(fmaxf(sum, 1.0f), &ex);
  const float F = ldexpf(1.0f, mant == 0.5f ? ex - 1 : ex);
  const float rF = 1.0f / F;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* src = y16 + (int64_t)t * k_total * H + c;
  for (int j = 0; j < k_total; ++j) {
    const float w = wt[j] * rF;
    const u32x2 v = *reinterpret_cast<const u32x2*>(src + (int64_t)j * H);
    const f16x2 a = bitcast<f16x2>(v[0]), b = bitcast<f16x2>(v[1]);
    acc[0] += w * (float)a[0];
    acc[1] += w * (float)a[1];
    acc[2] += w * (float)b[0];
    acc[3] += w * (float)b[1];
  }
  const float AF = A * F;
  f32x4 out;
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = (float)(_Float16)acc[e] * AF;
  *reinterpret_cast<f32x4*>(y + (int64_t)t * H + c) = out;
}
}  // namespace

hipError_t launch_combine_restore(const uint16_t* y16, const float* weights, int T, int k_total, int H, int att_log2,
                                  float* y, hipStream_t stream) {
  const int64_t n = (int64_t)T * (H >> 2);
  combine_restore_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, stream>>>(y16, weights, T, k_total, H,
                                                                               ldexpf(1.0f, att_log2), y);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y_slots, const float* weights, int T, int k_total, int H, float* y,
                          hipStream_t stream) {
  const int64_t n = (int64_t)T * (H >> 2);
  combine_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, stream>>>(y_slots, weights, T, k_total, H, y);
  return hipGetLastError();
}

}  // namespace moe
