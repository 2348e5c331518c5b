// The expert FFN's MXFP4 decode primitive on its own (FreeToken DeepSeek-V4-Flash post, "MXFP4 is
// not NVFP4": decoded weight v(c) * 2^(e-127) for 32 E2M1 codes sharing one E8M0 scale).
// One thread decodes one 16-byte block (32 codes) into 32 bf16 values with the same device
// function the FFN kernels use.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, int n_rows, int K,
                                                      int64_t code_stride, int64_t scale_stride,
                                                      uint16_t* __restrict__ out) {
  const int bpr = K >> 5;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)n_rows * bpr) return;
  const int n = (int)(i / bpr), b = (int)(i % bpr);
  const u32x4 q = ld16(codes + (int64_t)n * code_stride + 16 * b);
  const float sc = e8m0_to_f32(scales[(int64_t)n * scale_stride + b]);
  uint16_t* dst = out + (int64_t)n * K + 32 * b;
#pragma unroll
  for (int s = 0; s < 4; ++s) st16(dst + 8 * s, bitcast<u32x4>(decode8_bf16(q[s], sc)));
}
}  // namespace

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, int n_rows, int K, int64_t code_stride,
                          int64_t scale_stride, uint16_t* out, hipStream_t stream) {
  const int64_t n = (int64_t)n_rows * (K >> 5);
  dequant_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, stream>>>(codes, scales, n_rows, K, code_stride,
                                                                        scale_stride, out);
  return hipGetLastError();
}

}  // namespace moe
