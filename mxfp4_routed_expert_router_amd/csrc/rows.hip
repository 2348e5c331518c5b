// Fixed row-shape calls (Cascadia Sec. 3.2: the runtime picks one of the row shapes its compiled
// layer supports, pads the extra rows with zero routing weights, and hands back only the real
// rows).  Here the "compiled layer" is a HIP graph captured for one row shape; the real row count
// lives in device memory so that one captured graph serves every count up to its shape.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// Rows t >= n (n = *n_rows clamped to [0, T_shape]) get zero routing weights and the invalid id
// -1, so the bucketing drops their slots and no expert runs on them.  One thread per slot.
__global__ __launch_bounds__(256) void pad_rows_kernel(const int32_t* __restrict__ n_rows, int T_shape, int k_total,
                                                       int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T_shape * k_total) return;
  const int n = min(max(*n_rows, 0), T_shape);
  if (i / k_total >= n) {
    ids[i] = -1;
    weights[i] = 0.0f;
  }
}

}  // namespace

hipError_t launch_pad_rows(const int32_t* n_rows, int T_shape, int k_total, int32_t* ids, float* weights,
                           hipStream_t stream) {
  const int64_t n = (int64_t)T_shape * k_total;
  pad_rows_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, stream>>>(n_rows, T_shape, k_total, ids, weights);
  return hipGetLastError();
}

}  // namespace moe
