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

#include <type_traits>

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
// Every lane is written (all rows and banks enabled), so the "old" operand
// is the value itself: no separate register has to be cleared first.
template <int Q>
__device__ __forceinline__ float row_bcast(float v) {
  const int b = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, 0x150 + Q, 0xF, 0xF, false));
}
template <int Q>
__device__ __forceinline__ double row_bcast(double v) {
  long long b = __builtin_bit_cast(long long, v);
  const int l0 = (int)(b & 0xffffffffll), h0 = (int)(b >> 32);
  int lo = __builtin_amdgcn_update_dpp(l0, l0, 0x150 + Q, 0xF, 0xF, false);
  int hi = __builtin_amdgcn_update_dpp(h0, h0, 0x150 + Q, 0xF, 0xF, false);
  return __builtin_bit_cast(double, (long long)(((unsigned long long)(unsigned)hi << 32) |
                                                (unsigned long long)(unsigned)lo));
}

// Straight-line "loop" I = N-1, N-2, ..., 0 with I a compile-time constant in
// the body (register arrays stay registers; DPP controls stay immediates).
template <int I, typename F>
__device__ __forceinline__ void static_for_down(F&& f) {
  if constexpr (I >= 0) {
    f(std::integral_constant<int, I>{});
    static_for_down<I - 1>(f);
  }
}

// Global -> LDS copy of a ROWS x COLS tile by NT threads: every load is issued
// before the first LDS store, so the tile costs one memory latency, not one
// per loop iteration.  get(r, c) returns the (masked) source element.
template <typename T, int ROWS, int COLS, int NT, int LDD, typename Get>
__device__ __forceinline__ void tile_to_lds(T* __restrict__ dst, int tid, Get&& get) {
  constexpr int PER = (ROWS * COLS + NT - 1) / NT;
  T v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + NT * i;
    v[i] = (e < ROWS * COLS) ? get(e / COLS, e % COLS) : (T)0;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + NT * i;
    if (e < ROWS * COLS) dst[(e / COLS) * LDD + e % COLS] = v[i];
  }
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations (lgkmcnt(0)) and meets the other waves, without the release
// fence of __syncthreads(), whose vmcnt(0) would drain global loads that are
// deliberately still in flight.  The signal fences stop the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt(63) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Empty register constraint: the value must exist in a VGPR at this point.
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(double& v) { asm volatile("" : "+v"(v)); }

// Straight-line "loop" I = 0 .. N-1 with I a compile-time constant.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for_up(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_up<N, I + 1>(f);
  }
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
