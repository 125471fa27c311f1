// Processing orders and per-call status flags.
//
// "The Geometry of LLM Quantization: GPTQ as Babai's Nearest Plane
// Algorithm", technical summary 2.2 (standard GPTQ runs first to last
// column, Babai last to first) and 2.3 (the bound depends on the pivot
// order; "act-order" takes columns by descending Hessian diagonal).
// A permutation maps position k -> original column perm[k]; position n-1 is
// processed first.
#include "pwq_device.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

__global__ void init_flags(DevFlags* flags, pwq_result* res, int reset_info) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    flags->info = 0;
    if (reset_info) res->info = 0;
  }
}

__global__ __launch_bounds__(256) void reverse_perm(int32_t* __restrict__ perm, int n) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k < n) perm[k] = n - 1 - k;
}

// rank_i = #{ j : d_j > d_i or (d_j == d_i and j < i) }, d = diag H with
// erased (zero) inputs counted as 1 and NaN as -inf (a total order, so the
// ranks are a permutation); the column of rank 0 is processed first.
__global__ __launch_bounds__(256) void act_order_perm(const float* __restrict__ H, int n,
                                                      int32_t* __restrict__ perm) {
  __shared__ float dj[256];
  const int i = blockIdx.x * 256 + threadIdx.x;
  float di = 0.0f;
  if (i < n) {
    di = H[(int64_t)i * n + i];
    if (di == 0.0f) di = 1.0f;
    if (di != di) di = -INFINITY;
  }
  int rank = 0;
  for (int j0 = 0; j0 < n; j0 += 256) {
    __syncthreads();
    const int j = j0 + threadIdx.x;
    float v = 0.0f;
    if (j < n) {
      v = H[(int64_t)j * n + j];
      if (v == 0.0f) v = 1.0f;
      if (v != v) v = -INFINITY;
    }
    dj[threadIdx.x] = v;
    __syncthreads();
    const int lim = min(256, n - j0);
    for (int t = 0; t < lim; ++t) {
      const float d = dj[t];
      rank += (d > di) || (d == di && j0 + t < i);
    }
  }
  if (i < n) perm[n - 1 - rank] = i;
}

__global__ __launch_bounds__(256) void iota_perm(int32_t* __restrict__ perm, int n) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k < n) perm[k] = k;
}

__global__ __launch_bounds__(256) void clear_i32(int32_t* __restrict__ p, int n) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k < n) p[k] = 0;
}

__global__ __launch_bounds__(256) void count_perm(const int32_t* __restrict__ perm, int n,
                                                  int32_t* __restrict__ seen,
                                                  DevFlags* flags, pwq_result* res) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= n) return;
  const int v = perm[k];
  if (v < 0 || v >= n) {
    flags->info = -1;
    res->info = -1;
    return;
  }
  atomicAdd(&seen[v], 1);
}

__global__ __launch_bounds__(256) void check_seen(const int32_t* __restrict__ seen, int n,
                                                  DevFlags* flags, pwq_result* res) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k < n && seen[k] != 1) {
    flags->info = -1;
    res->info = -1;
  }
}

}  // namespace

hipError_t launch_init_flags(DevFlags* flags, pwq_result* res, int reset_info, hipStream_t st) {
  init_flags<<<1, 64, 0, st>>>(flags, res, reset_info);
  return hipGetLastError();
}

hipError_t launch_identity_perm(int32_t* perm, int64_t n, hipStream_t st) {
  iota_perm<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(perm, (int)n);
  return hipGetLastError();
}

hipError_t launch_order(int32_t order_kind, const float* H, int64_t n, const int32_t* perm_in,
                        int32_t* perm_out, int32_t* seen, pwq_result* res, DevFlags* flags,
                        hipStream_t st) {
  const unsigned g = (unsigned)((n + 255) / 256);
  switch (order_kind) {
    case PWQ_ORDER_FRONT_TO_BACK:
      reverse_perm<<<g, 256, 0, st>>>(perm_out, (int)n);
      break;
    case PWQ_ORDER_ACT:
      act_order_perm<<<g, 256, 0, st>>>(H, (int)n, perm_out);
      break;
    case PWQ_ORDER_PERM:
      clear_i32<<<g, 256, 0, st>>>(seen, (int)n);
      count_perm<<<g, 256, 0, st>>>(perm_in, (int)n, seen, flags, res);
      check_seen<<<g, 256, 0, st>>>(seen, (int)n, flags, res);
      break;
    default:
      break;
  }
  return hipGetLastError();
}

}  // namespace pwq
