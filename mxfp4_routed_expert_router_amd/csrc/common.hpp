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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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
// Reductions through DPP moves (no LDS round trips): a running max / sum over 16-lane rows
// (row_shr 1, 2, 4, 8), then row 0 -> 1 and row 2 -> 3 (row_bcast15), then rows 0-1 -> 2-3
// (row_bcast31).  Lane 63 then holds the whole wave's result, read back as a uniform value.  A
// lane whose DPP source is out of its row (or in a disabled row) keeps `old`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWS, 0xF, false);
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

__device__ __forceinline__ float wave_max_dpp(float v) {
  uint32_t u = __float_as_uint(v);
#define MOE_DPP_MAX(C, R) u = __float_as_uint(fmaxf(__uint_as_float(u), __uint_as_float(dpp_u32<C, R>(u, u))))
  MOE_DPP_MAX(kDppRowShr1, 0xF);
  MOE_DPP_MAX(kDppRowShr2, 0xF);
  MOE_DPP_MAX(kDppRowShr4, 0xF);
  MOE_DPP_MAX(kDppRowShr8, 0xF);
  MOE_DPP_MAX(kDppRowBcast15, 0xA);
  MOE_DPP_MAX(kDppRowBcast31, 0xC);
#undef MOE_DPP_MAX
  return __uint_as_float(__builtin_amdgcn_readlane(u, 63));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  uint32_t u = __float_as_uint(v);
#define MOE_DPP_ADD(C, R) u = __float_as_uint(__uint_as_float(u) + __uint_as_float(dpp_u32<C, R>(0u, u)))
  MOE_DPP_ADD(kDppRowShr1, 0xF);
  MOE_DPP_ADD(kDppRowShr2, 0xF);
  MOE_DPP_ADD(kDppRowShr4, 0xF);
  MOE_DPP_ADD(kDppRowShr8, 0xF);
  MOE_DPP_ADD(kDppRowBcast15, 0xA);
  MOE_DPP_ADD(kDppRowBcast31, 0xC);
#undef MOE_DPP_ADD
  return __uint_as_float(__builtin_amdgcn_readlane(u, 63));
}
// Inclusive prefix sum over the lanes of a wave in DPP steps (within rows of 16, then across rows).
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t u) {
#define MOE_DPP_SCAN(C, R) u += dpp_u32<C, R>(0u, u)
  MOE_DPP_SCAN(kDppRowShr1, 0xF);
  MOE_DPP_SCAN(kDppRowShr2, 0xF);
  MOE_DPP_SCAN(kDppRowShr4, 0xF);
  MOE_DPP_SCAN(kDppRowShr8, 0xF);
  MOE_DPP_SCAN(kDppRowBcast15, 0xA);
  MOE_DPP_SCAN(kDppRowBcast31, 0xC);
#undef MOE_DPP_SCAN
  return u;
}
// Maximum of an unsigned 32-bit value over the wave, returned uniform.
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t u) {
#define MOE_DPP_MAXU(C, R) u = max(u, dpp_u32<C, R>(u, u))
  MOE_DPP_MAXU(kDppRowShr1, 0xF);
  MOE_DPP_MAXU(kDppRowShr2, 0xF);
  MOE_DPP_MAXU(kDppRowShr4, 0xF);
  MOE_DPP_MAXU(kDppRowShr8, 0xF);
  MOE_DPP_MAXU(kDppRowBcast15, 0xA);
  MOE_DPP_MAXU(kDppRowBcast31, 0xC);
#undef MOE_DPP_MAXU
  return __builtin_amdgcn_readlane(u, 63);
}
// Order-preserving map of a float (finite or infinite) onto uint32, and back.
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
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
