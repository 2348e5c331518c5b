// Weighted combine (Cascadia, Sec. 3.1 "weighted reduction"; FP32 output as in Cascadia Fig. 2):
//   y[t, :] = sum_{j ascending} weights[t, j] * y_slots[t*k + j, :]
// One thread owns four consecutive outputs of one token (16-byte loads and stores); no atomics.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y_slots,
                                                      const float* __restrict__ weights, int T, int k_total,
                                                      int H, float* __restrict__ y) {
  const int h4 = H >> 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * h4) return;
  const int t = (int)(i / h4), c = (int)(i % h4) * 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const float* src = y_slots + (int64_t)t * k_total * H + c;
  for (int j = 0; j < k_total; ++j) {
    const float w = weights[(int64_t)t * k_total + j];
    const f32x4 v = *reinterpret_cast<const f32x4*>(src + (int64_t)j * H);
    acc[0] += w * v[0];
    acc[1] += w * v[1];
    acc[2] += w * v[2];
    acc[3] += w * v[3];
  }
  *reinterpret_cast<f32x4*>(y + (int64_t)t * H + c) = acc;
}
}  // namespace

hipError_t launch_combine(const float* y_slots, const float* weights, int T, int k_total, int H, float* y,
                          hipStream_t stream) {
  const int64_t n = (int64_t)T * (H >> 2);
  combine_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, stream>>>(y_slots, weights, T, k_total, H, y);
  return hipGetLastError();
}

}  // namespace moe
