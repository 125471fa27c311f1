// Dead features, damping and the Cholesky factor of the damped Hessian.
//
// "WaterSIC: ...", technical summary 2: factor Sigma = L L^T (L lower) and
// erase inputs of (near) zero variance; "Initialisation Determines the
// Basin ...", section 3: the damped Hessian H + lambda I; "The Geometry of
// LLM Quantization ...", technical summary 2.1, Theorem 1: any factor of the
// Hessian gives the same closest-vector instance, so the square Cholesky
// factor replaces the tall input matrix.
//
// Design (gfx950): right-looking blocked Cholesky with 64-column panels, in
// place on an n x n working copy (float or double).  Per panel:
//   chol_panel_step  every workgroup factors the tall panel made of the
//                    64x64 diagonal block and its own 64 panel rows (4 waves,
//                    lane = row, one LDS broadcast + barrier per column), so
//                    L_kk and L_ik = A_ik L_kk^-T come out of one pass
//   chol_trailing    the trailing lower triangle A_ij -= L_ik L_jk^T as 128x128
//                 MFMA tiles (v_mfma_f32_32x32x2f32 / v_mfma_f64_16x16x4f64);
//                 both operands are panel rows, contiguous along K.
// A non-positive or non-finite pivot stops the factorization and records the
// LAPACK-style order of the failing minor; every later kernel sees the flag
// and returns at once.
#include "pwq_device.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

constexpr int NB = 64;   // panel width

// lambda = damp * mean(diag H'), H'_kk = 1 where H_kk == 0.  One workgroup;
// fixed-order fp64 reduction.
__global__ __launch_bounds__(256) void damp_prep(const float* __restrict__ H,
                                                 int n, double damp,
                                                 int32_t* __restrict__ dead,
                                                 pwq_result* __restrict__ res,
                                                 DevFlags* flags,
                                                 double* __restrict__ lam_out) {
  __shared__ double ssum[256];
  __shared__ int scnt[256];
  double s = 0.0;
  int cnt = 0;
  for (int i = threadIdx.x; i < n; i += 256) {
    const float h = H[(int64_t)i * n + i];
    const int d = h == 0.0f;
    if (dead) dead[i] = d;
    cnt += d;
    s += d ? 1.0 : (double)h;
  }
  ssum[threadIdx.x] = s;
  scnt[threadIdx.x] = cnt;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      ssum[threadIdx.x] += ssum[threadIdx.x + o];
      scnt[threadIdx.x] += scnt[threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double lam = damp * (ssum[0] / (double)n);
    *lam_out = lam;
    res->lambda = lam;
    res->ndead = scnt[0];
  }
}

// A[i][j] = H'[p_i][p_j] (+ lambda on the diagonal) for j <= i, 0 above.
template <typename T>
__global__ __launch_bounds__(256) void copy_damped(const float* __restrict__ H,
                                                   int n, const int32_t* __restrict__ perm,
                                                   const double* __restrict__ lam_p,
                                                   T* __restrict__ A, const DevFlags* flags) {
  if (flags->info != 0) return;
  const int i = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  const double lam = *lam_p;
  T v = (T)0;
  if (j <= i) {
    const int pi = perm ? perm[i] : i, pj = perm ? perm[j] : j;
    const int a = pi > pj ? pi : pj, b = pi > pj ? pj : pi;
    const float h = H[(int64_t)a * n + b];
    if (i == j)
      v = (T)((h == 0.0f ? 1.0 : (double)h) + lam);
    else
      v = (T)h;
  }
  A[(int64_t)i * n + j] = v;
}

__device__ __forceinline__ float readlane_t(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_t(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffffll), l);
  const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) |
                                          (unsigned long long)(unsigned)lo));
}

// Pivot square root and reciprocal: hardware ops for float (about 1 ulp; the
// factor's own rounding error is larger), correctly rounded for double.
__device__ __forceinline__ void pivot_ops(float piv, float& d, float& inv) {
  d = __builtin_amdgcn_sqrtf(piv);
  inv = __builtin_amdgcn_rcpf(d);
}
__device__ __forceinline__ void pivot_ops(double piv, double& d, double& inv) {
  d = sqrt(piv);
  inv = 1.0 / d;
}

// One panel step on the tall panel [A_kk; A_bk]: workgroup b factors the
// 64x64 diagonal block (slot 0) together with its own 64 panel rows
// k0 + 64 b .. (slot 1, b >= 1) in a single right-looking pass, so the panel
// solve L_bk = A_bk L_kk^-T needs no separate substitution.  Every
// workgroup repeats the diagonal factorization (bitwise identical results);
// workgroup 0 stores L_kk.  Lane = row; wave w keeps columns 16w..16w+15 of
// both slots in registers.  Columns go in groups of 4: the owner wave
// factors the group in registers (pivot rows broadcast with readlane) and
// publishes it in LDS; after one barrier every wave applies the rank-4
// update to its later columns.  The group buffer is double buffered, so one
// barrier per group suffices.
template <typename T>
__global__ __launch_bounds__(256) void chol_panel_step(T* __restrict__ A, int n, int k0,
                                                      DevFlags* flags,
                                                      pwq_result* __restrict__ res) {
  __shared__ __attribute__((aligned(16))) T gbuf[2][2][4][NB];
  __shared__ int fail_col;
  if (flags->info != 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = min(NB, n - k0);
  const int row1 = k0 + NB * blockIdx.x + lane;     // slot-1 row (blockIdx.x >= 1)
  const bool has1 = blockIdx.x > 0 && row1 < n;
  T d0[16], d1[16];
  {
    const T* src0 = A + (int64_t)(k0 + min(lane, nb - 1)) * n + k0 + 16 * wave;
    const T* src1 = A + (int64_t)(has1 ? row1 : k0) * n + k0 + 16 * wave;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const int col = 16 * wave + c;
      d0[c] = (lane < nb) ? (col <= lane ? src0[c] : (T)0) : (col == lane ? (T)1 : (T)0);
      d1[c] = has1 ? src1[c] : (T)0;
    }
  }
  if (tid == 0) fail_col = -1;
  __syncthreads();
  static_for_up<NB / 4>([&](auto G) {
    constexpr int g = decltype(G)::value;
    constexpr int j0 = 4 * g, wj = j0 / 16, jl0 = j0 % 16;
    if (wave == wj) {
      static_for_up<4>([&](auto U) {
        constexpr int u = decltype(U)::value;
        constexpr int j = j0 + u, jl = jl0 + u;
        const T piv = readlane_t(d0[jl], j);
        const bool bad = !(piv > (T)0) || !(piv < (T)INFINITY);
        if (bad && lane == 0 && fail_col < 0) fail_col = j;
        T d, inv;
        pivot_ops(piv, d, inv);
        d0[jl] = (lane == j) ? d : d0[jl] * inv;
        d1[jl] = d1[jl] * inv;
        static_for_up<3 - u>([&](auto V) {
          constexpr int k = j + 1 + decltype(V)::value;
          const T lkj = readlane_t(d0[jl], k);
          d0[jl0 + (k - j0)] -= d0[jl] * lkj;
          d1[jl0 + (k - j0)] -= d1[jl] * lkj;
        });
        gbuf[g & 1][0][u][lane] = d0[jl];
        gbuf[g & 1][1][u][lane] = d1[jl];
      });
    }
    __syncthreads();
    if (wave >= wj) {
      T li0[4], li1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        li0[u] = gbuf[g & 1][0][u][lane];
        li1[u] = gbuf[g & 1][1][u][lane];
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int k = 16 * wave + c;
        if (k >= j0 + 4) {                      // uniform per wave
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const T lkj = gbuf[g & 1][0][u][k];
            d0[c] -= li0[u] * lkj;
            d1[c] -= li1[u] * lkj;
          }
        }
      }
    }
  });
  __syncthreads();
  const int fc = fail_col;
  if (fc >= 0 && fc < nb) {
    if (blockIdx.x == 0 && tid == 0) {
      flags->info = k0 + fc + 1;
      res->info = k0 + fc + 1;
    }
    return;
  }
  if (blockIdx.x == 0) {
    if (lane < nb) {
      T* dst = A + (int64_t)(k0 + lane) * n + k0 + 16 * wave;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int col = 16 * wave + c;
        if (col <= lane && col < nb) dst[c] = d0[c];
      }
    }
  } else if (has1) {
    T* dst = A + (int64_t)row1 * n + k0 + 16 * wave;
#pragma unroll
    for (int c = 0; c < 16; ++c) dst[c] = d1[c];
  }
}

// Trailing update of the lower triangle: A_ij -= P_i P_j^T, P = the panel
// (columns k0..k0+64 of the rows below the diagonal block), 128x128 tiles.
template <typename T>
__global__ __launch_bounds__(256) void chol_trailing(T* __restrict__ A, int n, int k0,
                                                     const DevFlags* flags) {
  constexpr int TB = 128, LD = NB + 1;
  __shared__ T As[TB * LD];
  __shared__ T Bs[TB * LD];
  if (flags->info != 0) return;
  const int base = k0 + NB;
  int ti, tj;
  {
    const int t = blockIdx.x;
    int r = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    while (r * (r + 1) / 2 > t) --r;
    ti = r;
    tj = t - r * (r + 1) / 2;
  }
  const bool diag = ti == tj;
  const int r0 = base + ti * TB, c0 = base + tj * TB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  tile_to_lds<T, TB, NB, 256, LD>(As, tid, [&](int r, int k) {
    return (r0 + r < n) ? A[(int64_t)(r0 + r) * n + k0 + k] : (T)0;
  });
  if (!diag)
    tile_to_lds<T, TB, NB, 256, LD>(Bs, tid, [&](int r, int k) {
      return (c0 + r < n) ? A[(int64_t)(c0 + r) * n + k0 + k] : (T)0;
    });
  __syncthreads();
  const T* Bp = diag ? As : Bs;
  if constexpr (sizeof(T) == 4) {
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
#pragma unroll 8
    for (int k = 0; k < NB; k += 2) {
      const int ko = k + (lane >> 5);
      const float a0 = As[(wm * 64 + (lane & 31)) * LD + ko];
      const float a1 = As[(wm * 64 + 32 + (lane & 31)) * LD + ko];
      const float b0 = Bp[(wn * 64 + (lane & 31)) * LD + ko];
      const float b1 = Bp[(wn * 64 + 32 + (lane & 31)) * LD + ko];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
    }
    // epilogue: all loads first, then the stores
    float old[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gr = r0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int gc = c0 + wn * 64 + j * 32 + (lane & 31);
          old[i][j][r] = (gr < n && gc <= gr) ? A[(int64_t)gr * n + gc] : 0.0f;
        }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gr = r0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int gc = c0 + wn * 64 + j * 32 + (lane & 31);
          if (gr < n && gc <= gr) A[(int64_t)gr * n + gc] = old[i][j][r] - acc[i][j][r];
        }
  } else {
    f64x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0;
#pragma unroll 4
    for (int k = 0; k < NB; k += 4) {
      const int ko = k + (lane >> 4);
      double av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[(wm * 64 + i * 16 + (lane & 15)) * LD + ko];
        bv[i] = Bp[(wn * 64 + i * 16 + (lane & 15)) * LD + ko];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double old[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gr = r0 + wm * 64 + i * 16 + 4 * r + (lane >> 4);
          const int gc = c0 + wn * 64 + j * 16 + (lane & 15);
          old[j][r] = (gr < n && gc <= gr) ? A[(int64_t)gr * n + gc] : 0.0;
        }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gr = r0 + wm * 64 + i * 16 + 4 * r + (lane >> 4);
          const int gc = c0 + wn * 64 + j * 16 + (lane & 15);
          if (gr < n && gc <= gr) A[(int64_t)gr * n + gc] = old[j][r] - acc[i][j][r];
        }
    }
  }
}

template <typename T>
hipError_t factor_impl(T* A, int n, DevFlags* flags, pwq_result* res, hipStream_t st) {
  for (int k0 = 0; k0 < n; k0 += NB) {
    const int rows = n - k0;
    chol_panel_step<T><<<(rows + NB - 1) / NB, 256, 0, st>>>(A, n, k0, flags, res);
    const int below = n - k0 - NB;
    if (below > 0) {
      const int nt = (below + 127) / 128;
      chol_trailing<T><<<nt * (nt + 1) / 2, 256, 0, st>>>(A, n, k0, flags);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_damp_cholesky(const float* H, int64_t n, double damp, int32_t prec,
                                const int32_t* perm, void* L, int32_t* dead,
                                pwq_result* res, DevFlags* flags, double* lam,
                                hipStream_t st) {
  damp_prep<<<1, 256, 0, st>>>(H, (int)n, damp, dead, res, flags, lam);
  dim3 g((unsigned)((n + 255) / 256), (unsigned)n);
  if (prec == PWQ_F64) {
    copy_damped<double><<<g, 256, 0, st>>>(H, (int)n, perm, lam, (double*)L, flags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return factor_impl<double>((double*)L, (int)n, flags, res, st);
  }
  copy_damped<float><<<g, 256, 0, st>>>(H, (int)n, perm, lam, (float*)L, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return factor_impl<float>((float*)L, (int)n, flags, res, st);
}

}  // namespace pwq
