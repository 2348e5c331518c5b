// Shared device helpers for the gfx950 kernels of the routed-MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---- 16-byte global loads / stores (the ABI guarantees 16-byte alignment where used) ----
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

template <typename T, typename S>
__device__ __forceinline__ T bitcast(S s) {
  static_assert(sizeof(T) == sizeof(S), "bitcast size");
  T t;
  __builtin_memcpy(&t, &s, sizeof(T));
  return t;
}

// ---- MXFP4 decode [MX]: E8M0 code e -> fp32 2^(e-127).  e >= 1 is the binary32 exponent field;
//      e == 0 is the subnormal 2^-127.  Code 255 is outside the contract. ----
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return __uint_as_float(e == 0 ? 0x00400000u : (e << 23));
}

// Eight E2M1 codes (one dword, element 2i in the low nibble of byte i) times a block scale ->
// eight bf16 values, exact [MX].  v_cvt_scalef32_pk_bf16_fp4 decodes the two codes of one byte.
__device__ __forceinline__ bf16x8 decode8_bf16(uint32_t codes, float scale) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// ---- wave-level reductions (wave64) ----
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  return v;
}

// fp32 -> bf16 round-to-nearest-even (finite inputs) and the residual high/low split.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

}  // namespace moe
