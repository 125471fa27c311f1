// Dead features, damping and the Cholesky factor of the damped Hessian.
//
// "WaterSIC: ...", technical summary 2: factor Sigma = L L^T (L lower) and
// erase inputs of (near) zero variance; "Initialisation Determines the
// Basin ...", section 3: the damped Hessian H + lambda I; "The Geometry of
// LLM Quantization ...", technical summary 2.1, Theorem 1: any factor of the
// Hessian gives the same closest-vector instance, so the square Cholesky
// factor replaces the tall input matrix.
//
// Design (gfx950): right-looking blocked Cholesky with 64-column panels and
// a one-panel look-ahead, in place on an n x n working copy (float or
// double).  chol_panel_first factors the first tall panel; then one
// chol_step launch per panel both factors the next panel (after applying the
// current panel's update to it) and applies the current panel to the
// trailing triangle beyond it, so the serial panel work overlaps the
// parallel trailing update instead of alternating with it:
//   panel role     every workgroup factors the tall panel made of the 64x64
//                  diagonal block and its own 64 panel rows (4 waves, lane =
//                  row, rank-4 column groups through LDS), so L_kk and
//                  L_ik = A_ik L_kk^-T come out of one pass
//   trailing role  A_ij -= L_ik L_jk^T as 128x128 MFMA tiles, several
//                  pending panels at once (lazy_panels); with 16-byte
//                  aligned rows the operands go straight from memory into
//                  registers (v_mfma_f32_16x16x4f32 / v_mfma_f64_16x16x4f64),
//                  otherwise through LDS; both operands are panel rows,
//                  contiguous along K.
// A non-positive or non-finite pivot stops the factorization and records the
// LAPACK-style order of the failing minor; every later kernel sees the flag
// and returns at once.
#include "pwq_device.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

constexpr int NB = 64;   // panel width
// Panels per trailing update.  Applying several pending panels at once pays
// the trailing tiles' read-modify-write once per pass, but every panel in
// between applies the pending ones to itself, which lengthens the serial
// panel role; the balance moves with n.  Measured (register trailing tiles):
//   fp32  n = 28672: 84.6 / 81.1 ms with 4 / 8;  n = 20480: 34.6 / 34.0;
//         n = 14336: 19.5 / 15.8 / 14.4 / 15.0 ms with 1 / 2 / 4 / 8;
//         n = 8192: 4.92 / 4.56 / 4.62 / 5.22;  n = 4096: 1.51 / 1.50 / 1.64
//   fp64  n = 28672: 195 / 184 / 180 / 179 / 182 ms with 4 / 6 / 8 / 12 / 16;
//         n = 16384: 48.3 / 42.1 / 41.3 / 41.4 with 2 / 4 / 6 / 8;
//         n = 12288: 29.8 / 23.3 / 21.3 with 1 / 2 / 4;
//         n = 8192: 9.98 / 8.78 / 8.86 / 9.94 with 1 / 2 / 4 / 8;
//         n = 4096: 2.45 / 2.57 / 2.90 / 3.54 with 1 / 2 / 4 / 8.
template <typename T> int lazy_panels(int n) {
  if (sizeof(T) == 8) return n <= 4096 ? 1 : (n <= 8192 ? 2 : (n <= 12288 ? 4 : 8));
  return n >= 20480 ? 8 : (n >= 8192 ? 4 : 1);
}
// Panels per trailing update at the step with rem columns still to
// factor.  The count follows rem, so the large early passes gather more
// panels and the chain near the end applies fewer.  Against the size rule,
// same process, alternating: fp32 n = 4096 1.43 vs 1.47 ms, 8192 4.31 vs
// 4.47, 14336 14.08 vs 14.27 (at 20480 it was 1% slower and at 28672 even,
// so larger fp32 factors keep the size rule); fp64 n = 8192 8.50 vs 8.73,
// 16384 39.8 vs 40.3, 28672 176.3 vs 176.6 (n <= 4096 keeps one panel).
template <typename T> int lazy_panels_at(int n, int rem) {
  if (sizeof(T) == 8) {
    if (n <= 4096) return lazy_panels<T>(n);
    return rem >= 12288 ? 8 : (rem >= 6144 ? 4 : (rem >= 2048 ? 2 : 1));
  }
  if (n >= 20480) return lazy_panels<T>(n);
  return rem >= 6144 ? 4 : (rem >= 2048 ? 2 : 1);
}

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

// In place, for a Hessian already in the working copy (natural order):
// A[i][i] = H'_ii + lambda as copy_damped forms it, 0 above the diagonal,
// the lower triangle as it is.  One workgroup per matrix row.
__global__ __launch_bounds__(256) void damp_in_place(float* __restrict__ A, int n,
                                                    const double* __restrict__ lam_p,
                                                    const DevFlags* flags) {
  if (flags->info != 0) return;
  const int i = blockIdx.x;
  float* a = A + (int64_t)i * n;
  if (threadIdx.x == 0) {
    const float h = a[i];
    a[i] = (float)((h == 0.0f ? 1.0 : (double)h) + *lam_p);
  }
  for (int j = i + 1 + (int)threadIdx.x; j < n; j += 256) a[j] = 0.0f;
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

// LDS of one workgroup of the factorization kernels (either role).
template <typename T>
struct CholSmem {
  static constexpr int LD = NB + 1;                                  // padded row
  static constexpr size_t trail = 2 * 128 * LD * sizeof(T);          // two 128-row panels
  static constexpr size_t panel = 4 * 64 * LD * sizeof(T)            // Q, P, U0, U1
                                  + 2 * 2 * 4 * NB * sizeof(T);      // column groups
  static constexpr size_t bytes = trail > panel ? trail : panel;
};

// Factor the tall panel [A_kk; A_bk] held in registers and store it: the
// 64x64 diagonal block (slot 0, d0) together with the workgroup's own 64
// panel rows k0 + 64 b .. (slot 1, d1, b >= 1) in a single right-looking
// pass, so the panel solve L_bk = A_bk L_kk^-T needs no separate
// substitution.  Every workgroup repeats the diagonal factorization
// (bitwise identical results); workgroup b = 0 stores L_kk.  Lane = row;
// wave w keeps columns 16w..16w+15 of both slots in registers.  Columns go
// in groups of 4: the owner wave factors the group in registers (pivot rows
// broadcast with readlane) and publishes it in LDS; after one barrier every
// wave applies the rank-4 update to its later columns.  The group buffer is
// double buffered, so one barrier per group suffices.
template <typename T>
__device__ __forceinline__ void panel_factor_store(T* __restrict__ A, int n, int k0, int b,
                                                   T (&d0)[16], T (&d1)[16],
                                                   T (*gbuf)[2][4][NB], int* fail_col,
                                                   T* __restrict__ dbuf, DevFlags* flags,
                                                   pwq_result* res) {
  // the wave index as a scalar: "wave >= owner" below is then a scalar branch
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = min(NB, n - k0);
  const int row1 = k0 + NB * b + lane;
  const bool has1 = b > 0 && row1 < n;
  if (tid == 0) *fail_col = NB;
  // first bad pivot this wave owns (columns are factored in order, so the
  // smallest over the waves is the first bad one); kept in a register and
  // published once after the loop, off the column chain
  int my_fail = NB;
  // the owner's chain of group g: its 4 columns in registers, published in
  // the group buffer
  auto chain = [&](auto G) {
    constexpr int g = decltype(G)::value;
    constexpr int j0 = 4 * g, jl0 = j0 % 16;
    static_for_up<4>([&](auto U) {
      constexpr int u = decltype(U)::value;
      constexpr int j = j0 + u, jl = jl0 + u;
      const T piv = readlane_t(d0[jl], j);
      const bool bad = !(piv > (T)0) || !(piv < (T)INFINITY);
      if (bad && my_fail == NB) my_fail = j;
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
  };
  // rank-4 update of local column c by group g (li: this lane's row values)
  auto upd = [&](int gb, int c, int k, const T (&li0)[4], const T (&li1)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const T lkj = gbuf[gb][0][u][k];
      d0[c] -= li0[u] * lkj;
      d1[c] -= li1[u] * lkj;
    }
  };
  if (wave == 0) chain(std::integral_constant<int, 0>());
  // After group g is published: the owner of group g + 1 updates that
  // group's 4 columns, runs its chain, and only then updates its other
  // later columns, all in one block, so the scheduler can fill the chain's
  // dependent latencies with those independent updates; every other wave
  // at or after g's owner updates its later columns.
  static_for_up<NB / 4>([&](auto G) {
    constexpr int g = decltype(G)::value;
    constexpr int j0 = 4 * g, wj = j0 / 16;
    constexpr int gn = g + 1, jn0 = 4 * gn, wn = jn0 / 16, jln = jn0 % 16;
    __syncthreads();
    if (wave >= wj) {
      T li0[4], li1[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        li0[u] = gbuf[g & 1][0][u][lane];
        li1[u] = gbuf[g & 1][1][u][lane];
      }
      if (gn < NB / 4 && wave == wn) {
#pragma unroll
        for (int c = jln; c < jln + 4; ++c) upd(g & 1, c, 16 * wn + c, li0, li1);
        if constexpr (gn < NB / 4) chain(std::integral_constant<int, gn>());
#pragma unroll
        for (int c = jln + 4; c < 16; ++c) upd(g & 1, c, 16 * wn + c, li0, li1);
      } else {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
          const int k = 16 * wave + c;
          if (k >= j0 + 4) upd(g & 1, c, k, li0, li1);   // uniform per wave
        }
      }
    }
  });
  if (lane == 0 && my_fail < NB) atomicMin(fail_col, my_fail);
  __syncthreads();
  const int fc = *fail_col;
  if (fc < nb) {
    if (b == 0 && tid == 0) {
      flags->info = k0 + fc + 1;
      res->info = k0 + fc + 1;
    }
    return;
  }
  if (b == 0) {
    // L_kk goes to the side buffer: the diagonal block in A is still being
    // read by workgroups of this launch that started later
    if (lane < nb) {
      T* dst = dbuf + lane * NB + 16 * wave;
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

// Registers of the tall panel at k0 for workgroup b: the lower 64x64
// diagonal block (identity-padded past n) and the workgroup's panel rows.
template <typename T>
__device__ __forceinline__ void panel_load(const T* __restrict__ A, int n, int k0, int b,
                                           T (&d0)[16], T (&d1)[16]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nb = min(NB, n - k0);
  const int row1 = k0 + NB * b + lane;
  const bool has1 = b > 0 && row1 < n;
  const T* src0 = A + (int64_t)(k0 + min(lane, nb - 1)) * n + k0 + 16 * wave;
  const T* src1 = A + (int64_t)(has1 ? row1 : k0) * n + k0 + 16 * wave;
  if constexpr (sizeof(T) == 4) {
    // a whole fp32 panel with 16-byte aligned rows: 16-byte loads, masks after
    if (nb == NB && n % 4 == 0 && ((uintptr_t)A & 15) == 0) {
      float4 a[4], b4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = *(const float4*)(src0 + 4 * i);
        b4[i] = *(const float4*)(src1 + 4 * i);
      }
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const int col = 16 * wave + c;
        d0[c] = col <= lane ? (&a[c >> 2].x)[c & 3] : 0.0f;
        d1[c] = has1 ? (&b4[c >> 2].x)[c & 3] : 0.0f;
      }
      return;
    }
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const int col = 16 * wave + c;
    d0[c] = (lane < nb) ? (col <= lane ? src0[c] : (T)0) : (col == lane ? (T)1 : (T)0);
    d1[c] = has1 ? src1[c] : (T)0;
  }
}

// Diagonal block kq..kq+63 of L from the side buffer into A (lower part).
template <typename T>
__device__ __forceinline__ void diag_copy(T* __restrict__ A, int n, int kq,
                                          const T* __restrict__ dbuf) {
  const int nb = min(NB, n - kq);
  for (int e = threadIdx.x; e < NB * NB; e += 256) {
    const int r = e / NB, c = e % NB;
    if (r < nb && c <= r) A[(int64_t)(kq + r) * n + kq + c] = dbuf[e];
  }
}

// First panel (nothing to apply before it).  L_00 goes to side buffer 0.
template <typename T>
__global__ __launch_bounds__(256) void chol_panel_first(T* __restrict__ A, int n,
                                                       T* __restrict__ dbuf, DevFlags* flags,
                                                       pwq_result* __restrict__ res) {
  __shared__ __attribute__((aligned(16))) T gbuf[2][2][4][NB];
  __shared__ int fail_col;
  if (flags->info != 0) return;
  T d0[16], d1[16];
  panel_load<T>(A, n, 0, blockIdx.x, d0, d1);
  panel_factor_store<T>(A, n, 0, blockIdx.x, d0, d1, gbuf, &fail_col, dbuf, flags, res);
}

// The last diagonal block, after the final step.
template <typename T>
__global__ __launch_bounds__(256) void chol_diag_last(T* __restrict__ A, int n, int kq,
                                                     const T* __restrict__ dbuf,
                                                     const DevFlags* flags) {
  if (flags->info != 0) return;
  diag_copy<T>(A, n, kq, dbuf);
}

// U (+)= S Q^T for 64 x 64 operands in LDS (rows x NB, padded), accumulated
// in registers over K chunks and then written to LDS.  Wave w owns the
// 32x32 block (w>>1, w&1).
template <typename T>
struct Mfma64 {
  static constexpr int LD = NB + 1;
  // fp32: one 32x32 accumulator; fp64: 2x2 16x16 accumulators (lane l,
  // register r -> row 4r + l/16, col l%16)
  typename std::conditional<sizeof(T) == 4, f32x16_t, f64x4_t[2][2]>::type acc;

  __device__ __forceinline__ void zero() {
    if constexpr (sizeof(T) == 4) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0;
    }
  }
  __device__ __forceinline__ void add(const T* __restrict__ S, const T* __restrict__ Q) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    if constexpr (sizeof(T) == 4) {
#pragma unroll 8
      for (int k = 0; k < NB; k += 2) {
        const int ko = k + (lane >> 5);
        const float a = S[(wm * 32 + (lane & 31)) * LD + ko];
        const float bq = Q[(wn * 32 + (lane & 31)) * LD + ko];
        acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bq, acc, 0, 0, 0);
      }
    } else {
#pragma unroll 4
      for (int k = 0; k < NB; k += 4) {
        const int ko = k + (lane >> 4);
        double av[2], bv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          av[i] = S[(wm * 32 + i * 16 + (lane & 15)) * LD + ko];
          bv[i] = Q[(wn * 32 + i * 16 + (lane & 15)) * LD + ko];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(T* __restrict__ U) const {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    if constexpr (sizeof(T) == 4) {
      // 32x32 layout: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, col l%32
#pragma unroll
      for (int r = 0; r < 16; ++r)
        U[(wm * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * LD + wn * 32 + (lane & 31)] =
            acc[r];
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            U[(wm * 32 + i * 16 + 4 * r + (lane >> 4)) * LD + wn * 32 + j * 16 + (lane & 15)] =
                acc[i][j][r];
    }
  }
};

// Trailing update of one 128x128 lower-triangle tile t (row-major triangle
// order) of A[base:, base:] by the panel at columns k0..k0+63:
// A_ij -= P_i P_j^T with P the panel rows, K = 64 on MFMA
// (v_mfma_f32_32x32x2f32 / v_mfma_f64_16x16x4f64); both operands are panel
// rows, contiguous along K.
template <typename T>
__device__ __forceinline__ void trailing_tile(T* __restrict__ A, int n, int kfrom, int npan,
                                              int base, int t, char* smem) {
  constexpr int TB = 128, LD = NB + 1;
  T* As = (T*)smem;
  T* Bs = As + TB * LD;
  int ti, tj;
  {
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
  // The accumulators start from the current tile (loads issued first, so
  // their latency overlaps the panel loads) and the panel enters negated:
  // acc = A_ij + sum (-P_ik) P_jk.
  if constexpr (sizeof(T) == 4) {
    // 32x32 result layout: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, col l%32
    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gr = r0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int gc = c0 + wn * 64 + j * 32 + (lane & 31);
          acc[i][j][r] = (gr < n && gc <= gr) ? A[(int64_t)gr * n + gc] : 0.0f;
        }
    for (int pc = 0; pc < npan; ++pc) {
    const int k0 = kfrom + pc * NB;
    if (pc > 0) __syncthreads();          // the previous chunk's LDS reads are done
    // an opaque copy of n per chunk keeps the compiler from hoisting the 64
    // row addresses out of the loop (they would stay live in registers)
    int nl = n;
    asm volatile("" : "+s"(nl));
    tile_to_lds<T, TB, NB, 256, LD>(As, tid, [&](int r, int k) {
      return (r0 + r < nl) ? A[(int64_t)(r0 + r) * nl + k0 + k] : (T)0;
    });
    if (!diag)
      tile_to_lds<T, TB, NB, 256, LD>(Bs, tid, [&](int r, int k) {
        return (c0 + r < nl) ? A[(int64_t)(c0 + r) * nl + k0 + k] : (T)0;
      });
    __syncthreads();
    const T* Bp = diag ? As : Bs;
#pragma unroll 4
    for (int k = 0; k < NB; k += 2) {
      const int ko = k + (lane >> 5);
      const float a0 = -As[(wm * 64 + (lane & 31)) * LD + ko];
      const float a1 = -As[(wm * 64 + 32 + (lane & 31)) * LD + ko];
      const float b0 = Bp[(wn * 64 + (lane & 31)) * LD + ko];
      const float b1 = Bp[(wn * 64 + 32 + (lane & 31)) * LD + ko];
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
    }
    }
    // the store addresses are recomputed from an opaque copy of n, so the
    // 64 load addresses need not stay live through the K loop
    int ns = n;
    asm volatile("" : "+s"(ns));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gr = r0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int gc = c0 + wn * 64 + j * 32 + (lane & 31);
          if (gr < ns && gc <= gr) A[(int64_t)gr * ns + gc] = acc[i][j][r];
        }
  } else {
    // 16x16 f64 result layout: lane l, register r -> row 4r + l/16, col l%16
    f64x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gr = r0 + wm * 64 + i * 16 + 4 * r + (lane >> 4);
          const int gc = c0 + wn * 64 + j * 16 + (lane & 15);
          acc[i][j][r] = (gr < n && gc <= gr) ? A[(int64_t)gr * n + gc] : 0.0;
        }
    for (int pc = 0; pc < npan; ++pc) {
    const int k0 = kfrom + pc * NB;
    if (pc > 0) __syncthreads();          // the previous chunk's LDS reads are done
    // an opaque copy of n per chunk keeps the compiler from hoisting the 64
    // row addresses out of the loop (they would stay live in registers)
    int nl = n;
    asm volatile("" : "+s"(nl));
    tile_to_lds<T, TB, NB, 256, LD>(As, tid, [&](int r, int k) {
      return (r0 + r < nl) ? A[(int64_t)(r0 + r) * nl + k0 + k] : (T)0;
    });
    if (!diag)
      tile_to_lds<T, TB, NB, 256, LD>(Bs, tid, [&](int r, int k) {
        return (c0 + r < nl) ? A[(int64_t)(c0 + r) * nl + k0 + k] : (T)0;
      });
    __syncthreads();
    const T* Bp = diag ? As : Bs;
#pragma unroll 4
    for (int k = 0; k < NB; k += 4) {
      const int ko = k + (lane >> 4);
      double av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = -As[(wm * 64 + i * 16 + (lane & 15)) * LD + ko];
        bv[i] = Bp[(wn * 64 + i * 16 + (lane & 15)) * LD + ko];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gr = r0 + wm * 64 + i * 16 + 4 * r + (lane >> 4);
          const int gc = c0 + wn * 64 + j * 16 + (lane & 15);
          if (gr < n && gc <= gr) A[(int64_t)gr * n + gc] = acc[i][j][r];
        }
  }
}

// fp32 trailing tile with 16-byte aligned rows (n % 4 == 0): the same update
// as trailing_tile, with both operands loaded straight into registers as
// v_mfma_f32_16x16x4f32 operands.  Wave (wm, wn) takes rows 64 wm ..,
// columns 64 wn .. of the tile as 4 x 4 accumulators of 16 x 16; lane
// (r, q) = (l % 16, l / 16) holds K values 16 g + 4 q .. 16 g + 4 q + 3 of
// its row of each 16-row block (one 16-byte load each, so the 4 lanes of a
// row read 64 contiguous bytes and a load touches 16 rows), and MFMA step
// s of group g sums K = 16 g + 4 q + s over the lane groups q; both
// operands use the same order, so this is the product over all 64 K in a
// different rounding order.  No LDS and no barriers.  Rows and columns
// past n are clamped into the matrix (they only reach outputs that are not
// stored).
// 16x16 result layout: lane l, register r -> row 4 (l / 16) + r, col l % 16.
__device__ __forceinline__ void trailing_tile_f32_reg(float* __restrict__ A, int n, int kfrom,
                                                      int npan, int base, int t) {
  constexpr int TB = 128;
  int ti, tj;
  {
    int r = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    while (r * (r + 1) / 2 > t) --r;
    ti = r;
    tj = t - r * (r + 1) / 2;
  }
  const int r0 = base + ti * TB, c0 = base + tj * TB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, lq = lane >> 4, lr = lane & 15;
  // acc = A_ij - sum_k P_ik P_jk: the accumulators start from the tile.
  // The tile's addresses are formed from opaque copies of n, here and at the
  // stores, so the compiler cannot keep 64 of them live through the K loop.
  f32x4_t acc[4][4];
  {
    int nl = n;
    asm volatile("" : "+s"(nl));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gr = min(r0 + wm * 64 + i * 16 + 4 * lq + r, nl - 1);
          const int gc = min(c0 + wn * 64 + j * 16 + lr, nl - 1);
          acc[i][j][r] = A[(int64_t)gr * nl + gc];
        }
  }
  // Half a panel's operands (K groups g = 2 h, 2 h + 1 of each lane's rows):
  // 16 16-byte loads per lane, their row addresses formed here (eight row
  // pointers kept live would not fit beside the accumulators and operands).
  const int ra = r0 + wm * 64 + lr, rb = c0 + wn * 64 + lr;
  auto load = [&](float4 (&a)[4][2], float4 (&b)[4][2], int kc, int h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* pa = A + (int64_t)min(ra + 16 * i, n - 1) * n + 4 * lq + kc + 32 * h;
      const float* pb = A + (int64_t)min(rb + 16 * i, n - 1) * n + 4 * lq + kc + 32 * h;
#pragma unroll
      for (int gg = 0; gg < 2; ++gg) {
        a[i][gg] = *(const float4*)(pa + 16 * gg);
        b[i][gg] = *(const float4*)(pb + 16 * gg);
      }
    }
  };
  auto mma = [&](const float4 (&a)[4][2], const float4 (&b)[4][2]) {
#pragma unroll
    for (int gg = 0; gg < 2; ++gg)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          av[i] = -(&a[i][gg].x)[e];
          bv[i] = (&b[i][gg].x)[e];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
  };
  // Two half-panel operand sets in turn: the next half's loads are issued
  // before the current half's 128 MFMAs (a scheduling barrier keeps them
  // there; the scheduler would otherwise spread them among the MFMAs), so
  // their latency runs under the MFMAs; the wait before the MFMAs leaves the
  // newer loads in flight (vector memory counts complete in order).  The
  // last panel is peeled off, so that every wait inside the loop sees the
  // same loads in flight.
  float4 a0[4][2], b0[4][2], a1[4][2], b1[4][2];
  load(a0, b0, kfrom, 0);
  int kc = kfrom;
  for (int pc = 0; pc + 1 < npan; ++pc, kc += NB) {
    load(a1, b1, kc, 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0);
    load(a0, b0, kc + NB, 0);
    __builtin_amdgcn_sched_barrier(0);
    mma(a1, b1);
  }
  load(a1, b1, kc, 1);
  __builtin_amdgcn_sched_barrier(0);
  mma(a0, b0);
  __builtin_amdgcn_sched_barrier(0);
  mma(a1, b1);
  int ns = n;
  asm volatile("" : "+s"(ns));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gr = r0 + wm * 64 + i * 16 + 4 * lq + r;
        const int gc = c0 + wn * 64 + j * 16 + lr;
        if (gr < ns && gc <= gr) A[(int64_t)gr * ns + gc] = acc[i][j][r];
      }
}

// fp64 trailing tile with 16-byte aligned rows (n even): the register form
// of trailing_tile for doubles, as trailing_tile_f32_reg with
// v_mfma_f64_16x16x4f64: lane (r, q) = (l % 16, l / 16) holds K values
// 16 g + 4 q .. 16 g + 4 q + 3 of its row of each 16-row block (two 16-byte
// loads), MFMA step s of group g sums K = 16 g + 4 q + s over the lane
// groups q, and the operands of one K group (16 loads per lane) are
// double-buffered.  The fp64 kernel runs one workgroup per CU, so a lane
// has room for the accumulators (128 registers) and both operand sets.
// 16x16 f64 result layout: lane l, register r -> row 4 r + l / 16, col l % 16.
__device__ __forceinline__ void trailing_tile_f64_reg(double* __restrict__ A, int n, int kfrom,
                                                      int npan, int base, int t) {
  constexpr int TB = 128;
  int ti, tj;
  {
    int r = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
    while ((r + 1) * (r + 2) / 2 <= t) ++r;
    while (r * (r + 1) / 2 > t) --r;
    ti = r;
    tj = t - r * (r + 1) / 2;
  }
  const int r0 = base + ti * TB, c0 = base + tj * TB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, lq = lane >> 4, lr = lane & 15;
  f64x4_t acc[4][4];
  {
    int nl = n;
    asm volatile("" : "+s"(nl));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int gr = min(r0 + wm * 64 + i * 16 + 4 * r + lq, nl - 1);
          const int gc = min(c0 + wn * 64 + j * 16 + lr, nl - 1);
          acc[i][j][r] = A[(int64_t)gr * nl + gc];
        }
  }
  const int ra = r0 + wm * 64 + lr, rb = c0 + wn * 64 + lr;
  // one K group (16 K values; four doubles per lane and row block): step st
  // is group st % 4 of panel st / 4
  auto load = [&](double2 (&a)[4][2], double2 (&b)[4][2], int st) {
    const int kc = kfrom + NB * (st >> 2) + 16 * (st & 3) + 4 * lq;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const double* pa = A + (int64_t)min(ra + 16 * i, n - 1) * n + kc;
      const double* pb = A + (int64_t)min(rb + 16 * i, n - 1) * n + kc;
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        a[i][v] = *(const double2*)(pa + 2 * v);
        b[i][v] = *(const double2*)(pb + 2 * v);
      }
    }
  };
  auto mma = [&](const double2 (&a)[4][2], const double2 (&b)[4][2]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      double av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = -(e & 1 ? a[i][e >> 1].y : a[i][e >> 1].x);
        bv[i] = (e & 1 ? b[i][e >> 1].y : b[i][e >> 1].x);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
  };
  // two operand sets in turn, one K group ahead (4 npan steps, an even
  // count; the last two are peeled so every wait in the loop sees the same
  // loads in flight)
  double2 a0[4][2], b0[4][2], a1[4][2], b1[4][2];
  const int nst = 4 * npan;
  load(a0, b0, 0);
  for (int st = 0; st + 2 < nst; st += 2) {
    load(a1, b1, st + 1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0);
    load(a0, b0, st + 2);
    __builtin_amdgcn_sched_barrier(0);
    mma(a1, b1);
  }
  load(a1, b1, nst - 1);
  __builtin_amdgcn_sched_barrier(0);
  mma(a0, b0);
  __builtin_amdgcn_sched_barrier(0);
  mma(a1, b1);
  int ns = n;
  asm volatile("" : "+s"(ns));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gr = r0 + wm * 64 + i * 16 + 4 * r + lq;
        const int gc = c0 + wn * 64 + j * 16 + lr;
        if (gr < ns && gc <= gr) A[(int64_t)gr * ns + gc] = acc[i][j][r];
      }
}

// 64 rows r0 .. r0+63, columns kc .. kc+63 of fp32 A into LDS (row pitch
// NB + 1), for 16-byte aligned rows: four 16-byte loads per thread from rows
// clamped into the matrix, rows past n stored as zeros.
// One step with look-ahead, given the finished panel at k0 (columns
// k0..k0+63 of every row >= k0 hold L).  The trailing update is applied
// lazily, several panels at a time: panels kfrom/64 .. k0/64 (npan of them)
// have not yet been applied to the columns beyond the current panel.  Two
// roles in one launch, reading only finished panels, so they run
// concurrently:
//  * workgroups 0 .. np-1 take the NEXT panel p1 = k0 + 64: each applies the
//    pending panels to the rows it factors (the diagonal block and its own
//    64 rows; A -= P Q^T with K = 64 npan on MFMA through LDS) and factors
//    them as above -- the serial part of the factorization;
//  * if ntrail > 0, the next workgroups apply the same pending panels to the
//    trailing triangle beyond the next panel, A[k0+128:, k0+128:] (a
//    K = 64 npan update: the read-modify-write of the trailing triangle is
//    paid once per npan panels).
// The next panel's columns are written by the first role only, the columns
// beyond it by the second only.
template <typename T>
__global__ __launch_bounds__(256, sizeof(T) == 4 ? 2 : 1) void chol_step(T* __restrict__ A, int n, int k0, int kfrom,
                                                 int np, int ntrail, T* __restrict__ dbuf,
                                                 DevFlags* flags, pwq_result* __restrict__ res) {
  constexpr int LD = NB + 1;
  __shared__ __attribute__((aligned(16))) char smem[CholSmem<T>::bytes];
  __shared__ int fail_col;
  if (flags->info != 0) return;
  const int q = k0 / NB;
  const int npan = (k0 - kfrom) / NB + 1;
  if ((int)blockIdx.x >= np + ntrail) {
    // the finished diagonal block of panel k0 (no workgroup of this launch
    // reads rows k0..k0+63)
    diag_copy<T>(A, n, k0, dbuf + (q & 1) * NB * NB);
    return;
  }
  if ((int)blockIdx.x >= np) {
    if constexpr (sizeof(T) == 4) {
      if (n % 4 == 0 && ((uintptr_t)A & 15) == 0) {
        trailing_tile_f32_reg(A, n, kfrom, npan, k0 + 2 * NB, blockIdx.x - np);
        return;
      }
    } else {
      if (n % 2 == 0 && ((uintptr_t)A & 15) == 0) {
        trailing_tile_f64_reg(A, n, kfrom, npan, k0 + 2 * NB, blockIdx.x - np);
        return;
      }
    }
    trailing_tile<T>(A, n, kfrom, npan, k0 + 2 * NB, blockIdx.x - np, smem);
    return;
  }
  const int b = blockIdx.x, p1 = k0 + NB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  T* Q = (T*)smem;                 // pending-panel columns of rows p1 .. p1+63
  T* S = Q + 64 * LD;              // pending-panel columns of rows p1+64b .. (b >= 1)
  T* U0 = S + 64 * LD;
  T* U1 = U0 + 64 * LD;
  T(*gbuf)[2][4][NB] = (T(*)[2][4][NB])(U1 + 64 * LD);
  Mfma64<T> u0, u1;
  u0.zero();
  u1.zero();
  bool npan_done = false;   // the pending panels were applied by a vector path below
  if constexpr (sizeof(T) == 8) {
    if (n % 2 == 0 && ((uintptr_t)A & 15) == 0) {
      // fp64 rows of 16-byte multiples: the pending-panel rows come in as
      // 16-byte pairs from rows clamped into the matrix (rows past n are
      // zeroed on the way into LDS), and the next chunk's loads are in
      // flight while the current chunk's MFMAs run
      double2 qv[8], sv[8];
      auto vload = [&](int kc) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = tid + 256 * i, r = e >> 5, c2 = (e & 31) * 2;
          qv[i] = *(const double2*)(A + (int64_t)min(p1 + r, n - 1) * n + kc + c2);
          if (b > 0)
            sv[i] = *(const double2*)(A + (int64_t)min(p1 + NB * b + r, n - 1) * n + kc + c2);
        }
      };
      auto vstore = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int e = tid + 256 * i, r = e >> 5, c2 = (e & 31) * 2;
          const bool okq = p1 + r < n;
          Q[r * LD + c2] = okq ? qv[i].x : 0.0;
          Q[r * LD + c2 + 1] = okq ? qv[i].y : 0.0;
          if (b > 0) {
            const bool oks = p1 + NB * b + r < n;
            S[r * LD + c2] = oks ? sv[i].x : 0.0;
            S[r * LD + c2 + 1] = oks ? sv[i].y : 0.0;
          }
        }
      };
      vload(kfrom);
      for (int pc = 0; pc < npan; ++pc) {
        if (pc > 0) __syncthreads();   // the previous chunk's LDS reads are done
        vstore();
        __syncthreads();
        if (pc + 1 < npan) vload(kfrom + (pc + 1) * NB);
        u0.add(Q, Q);
        if (b > 0) u1.add(S, Q);
      }
      npan_done = true;
    }
  } else {
    if (n % 4 == 0 && ((uintptr_t)A & 15) == 0) {
      // fp32 rows of 16-byte multiples: the same with 16-byte loads, the
      // next chunk's loads in flight under the current chunk's MFMAs
      float4 qv[4], sv[4];
      auto vload = [&](int kc) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = tid + 256 * i, r = e >> 4, c4 = (e & 15) * 4;
          qv[i] = *(const float4*)(A + (int64_t)min(p1 + r, n - 1) * n + kc + c4);
          if (b > 0)
            sv[i] = *(const float4*)(A + (int64_t)min(p1 + NB * b + r, n - 1) * n + kc + c4);
        }
      };
      auto vstore = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = tid + 256 * i, r = e >> 4, c4 = (e & 15) * 4;
          const bool okq = p1 + r < n;
          Q[r * LD + c4 + 0] = okq ? qv[i].x : 0.0f;
          Q[r * LD + c4 + 1] = okq ? qv[i].y : 0.0f;
          Q[r * LD + c4 + 2] = okq ? qv[i].z : 0.0f;
          Q[r * LD + c4 + 3] = okq ? qv[i].w : 0.0f;
          if (b > 0) {
            const bool oks = p1 + NB * b + r < n;
            S[r * LD + c4 + 0] = oks ? sv[i].x : 0.0f;
            S[r * LD + c4 + 1] = oks ? sv[i].y : 0.0f;
            S[r * LD + c4 + 2] = oks ? sv[i].z : 0.0f;
            S[r * LD + c4 + 3] = oks ? sv[i].w : 0.0f;
          }
        }
      };
      vload(kfrom);
      for (int pc = 0; pc < npan; ++pc) {
        if (pc > 0) __syncthreads();   // the previous chunk's LDS reads are done
        vstore();
        __syncthreads();
        if (pc + 1 < npan) vload(kfrom + (pc + 1) * NB);
        u0.add(Q, Q);
        if (b > 0) u1.add(S, Q);
      }
      npan_done = true;
    }
  }
  // rows that are not 16-byte aligned: element loads, chunk by chunk
  for (int pc = 0; pc < npan && !npan_done; ++pc) {
    const int kc = kfrom + pc * NB;
    if (pc > 0) __syncthreads();   // the previous chunk's LDS reads are done
    tile_to_lds<T, 64, NB, 256, LD>(Q, tid, [&](int r, int k) {
      return (p1 + r < n) ? A[(int64_t)(p1 + r) * n + kc + k] : (T)0;
    });
    if (b > 0)
      tile_to_lds<T, 64, NB, 256, LD>(S, tid, [&](int r, int k) {
        const int row = p1 + NB * b + r;
        return (row < n) ? A[(int64_t)row * n + kc + k] : (T)0;
      });
    __syncthreads();
    u0.add(Q, Q);
    if (b > 0) u1.add(S, Q);
  }
  // the panel itself is loaded only now: holding it in registers through the
  // accumulation would cost the trailing role its second workgroup per CU
  T d0[16], d1[16];
  panel_load<T>(A, n, p1, b, d0, d1);
  u0.store(U0);
  if (b > 0) u1.store(U1);
  __syncthreads();
  const int nb = min(NB, n - p1);
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const int col = 16 * wave + c;
    if (lane < nb && col <= lane) d0[c] -= U0[lane * LD + col];
    if (b > 0) d1[c] -= U1[lane * LD + col];
  }
  panel_factor_store<T>(A, n, p1, b, d0, d1, gbuf, &fail_col, dbuf + ((q + 1) & 1) * NB * NB,
                        flags, res);
}

// dbuf: two 64x64 side buffers (T) for the diagonal blocks in flight.
template <typename T>
hipError_t factor_impl(T* A, int n, T* dbuf, DevFlags* flags, pwq_result* res,
                       hipStream_t st) {
  chol_panel_first<T><<<(n + NB - 1) / NB, 256, 0, st>>>(A, n, dbuf, flags, res);
  int k0 = 0;
  int kfrom = 0;   // first panel not yet applied to the columns beyond the next panel
  for (; k0 + NB < n; k0 += NB) {
    const int p1 = k0 + NB;
    const int np = (n - p1 + NB - 1) / NB;
    const int base2 = k0 + 2 * NB;
    const int nt = base2 < n ? (n - base2 + 127) / 128 : 0;
    // the trailing triangle takes the pending panels lazy_panels_at<T> at a time
    const bool trail = nt > 0 && (k0 - kfrom) / NB + 1 >= lazy_panels_at<T>(n, n - k0);
    const int ntrail = trail ? nt * (nt + 1) / 2 : 0;
    chol_step<T><<<np + ntrail + 1, 256, 0, st>>>(A, n, k0, kfrom, np, ntrail, dbuf, flags,
                                                  res);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (trail) kfrom = k0 + NB;
  }
  chol_diag_last<T><<<1, 256, 0, st>>>(A, n, k0, dbuf + ((k0 / NB) & 1) * NB * NB, flags);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_damp_cholesky_in_place(float* A, int64_t n, double damp, int32_t* dead,
                                         pwq_result* res, DevFlags* flags, double* lam,
                                         void* dscratch, hipStream_t st) {
  damp_prep<<<1, 256, 0, st>>>(A, (int)n, damp, dead, res, flags, lam);
  damp_in_place<<<(unsigned)n, 256, 0, st>>>(A, (int)n, lam, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return factor_impl<float>(A, (int)n, (float*)dscratch, flags, res, st);
}

hipError_t launch_damp_lambda(const float* H, int64_t n, double damp, int32_t* dead,
                              pwq_result* res, DevFlags* flags, double* lam, hipStream_t st) {
  damp_prep<<<1, 256, 0, st>>>(H, (int)n, damp, dead, res, flags, lam);
  return hipGetLastError();
}

hipError_t launch_damp_cholesky(const float* H, int64_t n, double damp, int32_t prec,
                                const int32_t* perm, void* L, int32_t* dead,
                                pwq_result* res, DevFlags* flags, double* lam, void* dscratch,
                                hipStream_t st) {
  damp_prep<<<1, 256, 0, st>>>(H, (int)n, damp, dead, res, flags, lam);
  dim3 g((unsigned)((n + 255) / 256), (unsigned)n);
  if (prec == PWQ_F64) {
    copy_damped<double><<<g, 256, 0, st>>>(H, (int)n, perm, lam, (double*)L, flags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return factor_impl<double>((double*)L, (int)n, (double*)dscratch, flags, res, st);
  }
  copy_damped<float><<<g, 256, 0, st>>>(H, (int)n, perm, lam, (float*)L, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return factor_impl<float>((float*)L, (int)n, (float*)dscratch, flags, res, st);
}

}  // namespace pwq
