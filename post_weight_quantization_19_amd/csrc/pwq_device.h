// Device-side helpers shared by the libpwq kernels (gfx950 / CDNA4 only).
//
// MFMA operand layouts used below (wave64):
//   v_mfma_f32_32x32x16_bf16 : A lane l holds A[l%32][8*(l/32) + e], e=0..7;
//                              B lane l holds B[8*(l/32) + e][l%32].
//   v_mfma_f32_32x32x2f32    : A lane l holds A[l%32][l/32]; B [l/32][l%32].
//   v_mfma_f64_16x16x4f64    : A lane l holds A[l%16][l/16]; B [l/16][l%16].
//   32x32 results: lane l, register r -> C[8*(r/4) + 4*(l/32) + r%4][l%32].
//   16x16 f32 results: lane l, register r -> C[4*(l/16) + r][l%16].
//   16x16 f64 results: lane l, register r -> C[4*r + l/16][l%16].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pwq {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(double)))) double f64x4_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Element loads from W (bf16 bits or float) widened to the working type.
template <typename T>
__device__ __forceinline__ T load_w(const void* W, int32_t wdtype, int64_t idx) {
  if (wdtype == 1) return (T)bf16_to_f32(((const uint16_t*)W)[idx]);
  return (T)(((const float*)W)[idx]);
}

// Broadcast lane q of every 16-lane row to the whole row (DPP row_newbcast).
template <int Q>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                         0x150 + Q, 0xF, 0xF, false));
}
template <int Q>
__device__ __forceinline__ double row_bcast(double v) {
  long long b = __builtin_bit_cast(long long, v);
  int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffll), 0x150 + Q, 0xF, 0xF, false);
  int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), 0x150 + Q, 0xF, 0xF, false);
  return __builtin_bit_cast(double, (long long)(((unsigned long long)(unsigned)hi << 32) |
                                                (unsigned long long)(unsigned)lo));
}

__device__ __forceinline__ float rint_t(float x) { return __builtin_rintf(x); }
__device__ __forceinline__ double rint_t(double x) { return __builtin_rint(x); }

// Deterministic wave64 sum (butterfly; the same order on every run).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, 64));
  return v;
}

// Kernel status flags kept in the workspace: [0] = first failing column + 1.
struct DevFlags {
  int32_t info;
  int32_t pad[63];
};

}  // namespace pwq
