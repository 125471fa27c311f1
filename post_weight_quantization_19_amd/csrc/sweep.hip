// Grid steps, the back-to-front nearest-plane sweep and the lazy block
// update.
//
// "The Geometry of LLM Quantization: GPTQ as Babai's Nearest Plane
// Algorithm", technical summary 2.1 (lattice basis X diag(s), fixed before
// the sweep), 2.2 (GPTQ's error propagation is the projection onto the
// nearest hyperplane followed by rounding; run from the last column to the
// first it is Babai's algorithm, Theorem 4), 2.3 (no clipping; Theorem 5
// bound (1/4) sum s^2 D); "WaterSIC: ...", technical summary 2 (L lower from
// Sigma = L L^T, decide the last column first and cancel the interference of
// decided columns; spacing alpha_i = c / |l_ii|).
//
// With R = L^T, a row's error d = w - w^ costs ||R d||^2 = sum_k (l_kk d_k +
// sum_{j>k} l_jk d_j)^2, so column k is rounded at the running target
//     w~_k = w_k + acc_k / l_kk,   acc_k = sum_{j>k} l_jk e_j,
// with e_j = w_j - s_j z_j the ORIGINAL weight minus the dequantized one.
//
// Design (gfx950):
//  * rows are independent closest-vector instances: 16 lanes work on one row
//    (4 rows per wave, 16 per 256-thread workgroup), each lane owning every
//    16th column of the current block in registers (acc, target terms,
//    step).  Per column the owning lane rounds, and its error is broadcast
//    to the other 15 lanes of the row with one DPP row_newbcast; every lane
//    then folds e * l_kj into its own open columns.  Rows of L for the block
//    are staged in LDS (the diagonal and the upper triangle stored as zero,
//    so updates of already-decided columns add exactly 0).
//  * after a block, its errors E [m x B] reach every earlier column in one
//    MFMA GEMM, acc[:, :j0] += E L[blk, :j0] (v_mfma_f32_32x32x2f32 or
//    v_mfma_f64_16x16x4f64), written (not read) on the first block.
//  * losses are accumulated per workgroup in fp64 and summed in a fixed
//    order by a final one-workgroup kernel.
#include "pwq_device.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

// ---------------------------------------------------------------- steps

__global__ __launch_bounds__(256) void grid_steps_kernel(
    const void* __restrict__ W, int32_t wdtype, int m, int n, int64_t ldw,
    const int32_t* __restrict__ dead, int kind, int bits, int G,
    float* __restrict__ scales, int32_t* __restrict__ zeros,
    const DevFlags* flags) {
  if (flags && flags->info != 0) return;
  const int ng = n / G;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wid >= m * ng) return;
  const int r = wid / ng, g = wid % ng;
  float mx = -INFINITY, mn = INFINITY, amax = 0.0f;
  for (int c = g * G + lane; c < (g + 1) * G; c += 64) {
    float w = load_w<float>(W, wdtype, (int64_t)r * ldw + c);
    if (dead && dead[c]) w = 0.0f;
    mx = fmaxf(mx, w);
    mn = fminf(mn, w);
    amax = fmaxf(amax, fabsf(w));
  }
  mx = wave_max(mx);
  mn = wave_min(mn);
  amax = wave_max(amax);
  if (lane != 0) return;
  if (kind == PWQ_GRID_SYM) {
    float s = amax / (float)((1 << (bits - 1)) - 1);
    if (s == 0.0f) s = 1.0f;
    scales[(int64_t)r * ng + g] = s;
  } else {
    const float lo = fminf(mn, 0.0f), hi = fmaxf(mx, 0.0f);
    float s = (hi - lo) / (float)((1 << bits) - 1);
    if (s == 0.0f) s = 1.0f;
    scales[(int64_t)r * ng + g] = s;
    zeros[(int64_t)r * ng + g] = (int32_t)rintf(-lo / s);
  }
}

// 1/l_kk, l_kk and (column spacing) alpha_k = c / l_kk.
template <typename T>
__global__ __launch_bounds__(256) void diag_prep(const T* __restrict__ L, int n, int colspacing,
                                                 double c, const int32_t* __restrict__ colmap,
                                                 T* __restrict__ invd, T* __restrict__ dg,
                                                 T* __restrict__ alpha,
                                                 float* __restrict__ scales_out,
                                                 const DevFlags* flags) {
  if (flags->info != 0) return;
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= n) return;
  const T d = L[(int64_t)k * n + k];
  dg[k] = d;
  invd[k] = (T)1 / d;
  if (colspacing) {
    const T a = (T)c / d;
    alpha[k] = a;
    scales_out[colmap ? colmap[k] : k] = (float)a;
  }
}

// ---------------------------------------------------------------- sweep

template <typename T>
struct SweepArgs {
  const void* W;
  int32_t wdtype;
  int64_t ldw;
  int m, n;
  const T* L;
  const T* invd;
  const T* dg;
  const T* alpha;        // column spacing (or nullptr)
  const float* scales;   // [m, ng] (SYM/ASYM)
  const int32_t* zeros;  // [m, ng] (ASYM) or nullptr
  int ng, G;
  const int32_t* colmap; // position -> original column, or nullptr
  const int32_t* dead;   // per ORIGINAL column, or nullptr
  T* acc;                // [m, n] running corrections (position frame)
  T* E;                  // [m, B] errors of the current block
  int32_t* codes;        // [m, n] original column order
  double* partials;      // [nblk, nwg, 4]
  const DevFlags* flags;
};

template <int Q, typename T>
__device__ __forceinline__ T bcast_q(T v) { return row_bcast<Q>(v); }

template <typename T>
__device__ __forceinline__ T bcast(T v, int q) {
  switch (q) {
    case 0: return bcast_q<0>(v);   case 1: return bcast_q<1>(v);
    case 2: return bcast_q<2>(v);   case 3: return bcast_q<3>(v);
    case 4: return bcast_q<4>(v);   case 5: return bcast_q<5>(v);
    case 6: return bcast_q<6>(v);   case 7: return bcast_q<7>(v);
    case 8: return bcast_q<8>(v);   case 9: return bcast_q<9>(v);
    case 10: return bcast_q<10>(v); case 11: return bcast_q<11>(v);
    case 12: return bcast_q<12>(v); case 13: return bcast_q<13>(v);
    case 14: return bcast_q<14>(v); default: return bcast_q<15>(v);
  }
}

template <typename T, int B>
__global__ __launch_bounds__(256) void sweep_block(SweepArgs<T> a, int blk, int first) {
  constexpr int P = 16, S = B / P;
  constexpr int CH0 = 16384 / (B * (int)sizeof(T));
  constexpr int CH = CH0 < 8 ? 8 : (CH0 > 32 ? 32 : CH0);
  static_assert(B % CH == 0, "chunk must divide block");
  __shared__ T Ls[CH * B];
  __shared__ double red[4][4];
  if (a.flags->info != 0) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane & 15;
  const int row = blockIdx.x * 16 + wave * 4 + (lane >> 4);
  const bool rok = row < a.m;
  const int n = a.n;
  const int j0 = blk * B;

  T acc[S], av[S], bv[S], sv[S], wv[S];
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const int col = j0 + q + P * t;
    const bool ok = rok && col < n;
    T w = (T)0, s = (T)1, il = (T)0, ac = (T)0;
    if (ok) {
      const int oc = a.colmap ? a.colmap[col] : col;
      w = load_w<T>(a.W, a.wdtype, (int64_t)row * a.ldw + oc);
      if (a.dead && a.dead[oc]) w = (T)0;
      s = a.alpha ? a.alpha[col] : (T)a.scales[(int64_t)row * a.ng + oc / a.G];
      il = a.invd[col];
      if (!first) ac = a.acc[(int64_t)row * n + col];
    }
    // true (correctly rounded) quotients: with no feedback yet the coordinate
    // is exactly w / s, so an exact tie is rounded to even as on paper
    acc[t] = ac;
    av[t] = il / s;
    bv[t] = w / s;
    sv[t] = s;
    wv[t] = w;
  }

  double loss_d = 0.0, bound = 0.0, dsq = 0.0;

#pragma unroll
  for (int kk = B - 1; kk >= 0; --kk) {
    if (kk % CH == CH - 1) {
      // stage rows j0+kk-CH+1 .. j0+kk of L (strictly-lower part of the block)
      const int cb = kk - CH + 1;
      __syncthreads();
      for (int e = tid; e < CH * B; e += 256) {
        const int rr = e / B, i = e % B;
        const int kr = cb + rr;
        T v = (T)0;
        if (i < kr && j0 + kr < n) v = a.L[(int64_t)(j0 + kr) * n + j0 + i];
        Ls[e] = v;
      }
      __syncthreads();
    }
    const int t = kk / P, qk = kk % P;
    const T c = acc[t] * av[t] + bv[t];
    const T z = rint_t(c);
    const T e = wv[t] - sv[t] * z;
    const T eb = bcast(e, qk);
    const T* lrow = &Ls[(kk % CH) * B + q];
#pragma unroll
    for (int t2 = 0; t2 <= t; ++t2) acc[t2] += eb * lrow[P * t2];
    if (qk == 0) {
      // every lane's slot t is final now: record its decision
      const int col = j0 + q + P * t;
      const T cc = acc[t] * av[t] + bv[t];
      const T zz = rint_t(cc);
      const T rho = cc - zz;
      const T ee = wv[t] - sv[t] * zz;
      if (rok && col < n) {
        const int oc = a.colmap ? a.colmap[col] : col;
        int32_t code = (int32_t)zz;
        if (a.zeros) code += a.zeros[(int64_t)row * a.ng + oc / a.G];
        a.codes[(int64_t)row * n + oc] = code;
        a.E[(int64_t)row * B + q + P * t] = ee;
        const double sl = (double)sv[t] * (double)a.dg[col];
        loss_d += (double)rho * (double)rho * sl * sl;
        bound += sl * sl;
        dsq += (double)ee * (double)ee;
      } else if (rok) {
        a.E[(int64_t)row * B + q + P * t] = (T)0;
      }
    }
  }

  loss_d = wave_sum(loss_d);
  bound = wave_sum(bound);
  dsq = wave_sum(dsq);
  if (lane == 0) {
    red[wave][0] = loss_d;
    red[wave][1] = bound;
    red[wave][2] = dsq;
  }
  __syncthreads();
  if (tid == 0) {
    double* p = a.partials + ((int64_t)blk * gridDim.x + blockIdx.x) * 4;
    p[0] = (red[0][0] + red[1][0]) + (red[2][0] + red[3][0]);
    p[1] = (red[0][1] + red[1][1]) + (red[2][1] + red[3][1]);
    p[2] = (red[0][2] + red[1][2]) + (red[2][2] + red[3][2]);
    p[3] = 0.0;
  }
}

// ------------------------------------------------------------ lazy update
// acc[r, c] (+)= sum_{k < kb} E[r, k] * L[j0 + k, c]   for r < m, c < j0.
template <typename T>
__global__ __launch_bounds__(256) void lazy_update(const T* __restrict__ E, int B, int kb,
                                                   const T* __restrict__ L, int n, int j0,
                                                   int m, T* __restrict__ acc, int first,
                                                   const DevFlags* flags) {
  constexpr int TM = 128, KC = 32, LDA = KC + 1, LDB = TM + 1;
  __shared__ T Es[TM * LDA];
  __shared__ T Lt[KC * LDB];
  if (flags->info != 0) return;
  const int c0 = blockIdx.x * TM, r0 = blockIdx.y * TM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  if constexpr (sizeof(T) == 4) {
    f32x16_t cc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) cc[i][j][r] = 0.0f;
    for (int kc = 0; kc < kb; kc += KC) {
      __syncthreads();
      for (int e = tid; e < TM * KC; e += 256) {
        const int r = e / KC, k = e % KC;
        Es[r * LDA + k] = (r0 + r < m && kc + k < kb) ? E[(int64_t)(r0 + r) * B + kc + k] : 0.0f;
        const int kr = e / TM, cc_ = e % TM;
        Lt[kr * LDB + cc_] = (kc + kr < kb && c0 + cc_ < j0)
                                 ? L[(int64_t)(j0 + kc + kr) * n + c0 + cc_] : 0.0f;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < KC; k += 2) {
        const int ko = k + (lane >> 5);
        const float a0 = Es[(wm * 64 + (lane & 31)) * LDA + ko];
        const float a1 = Es[(wm * 64 + 32 + (lane & 31)) * LDA + ko];
        const float b0 = Lt[ko * LDB + wn * 64 + (lane & 31)];
        const float b1 = Lt[ko * LDB + wn * 64 + 32 + (lane & 31)];
        cc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, cc[0][0], 0, 0, 0);
        cc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, cc[0][1], 0, 0, 0);
        cc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, cc[1][0], 0, 0, 0);
        cc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, cc[1][1], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int gr = r0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int gc = c0 + wn * 64 + j * 32 + (lane & 31);
          if (gr < m && gc < j0) {
            T* p = acc + (int64_t)gr * n + gc;
            *p = first ? cc[i][j][r] : *p + cc[i][j][r];
          }
        }
  } else {
    f64x4_t cc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) cc[i][j][r] = 0.0;
    for (int kc = 0; kc < kb; kc += KC) {
      __syncthreads();
      for (int e = tid; e < TM * KC; e += 256) {
        const int r = e / KC, k = e % KC;
        Es[r * LDA + k] = (r0 + r < m && kc + k < kb) ? E[(int64_t)(r0 + r) * B + kc + k] : 0.0;
        const int kr = e / TM, cc_ = e % TM;
        Lt[kr * LDB + cc_] = (kc + kr < kb && c0 + cc_ < j0)
                                 ? L[(int64_t)(j0 + kc + kr) * n + c0 + cc_] : 0.0;
      }
      __syncthreads();
#pragma unroll 2
      for (int k = 0; k < KC; k += 4) {
        const int ko = k + (lane >> 4);
        double av[4], bv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          av[i] = Es[(wm * 64 + i * 16 + (lane & 15)) * LDA + ko];
          bv[i] = Lt[ko * LDB + wn * 64 + i * 16 + (lane & 15)];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            cc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[i], bv[j], cc[i][j], 0, 0, 0);
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
          if (gr < m && gc < j0) {
            T* p = acc + (int64_t)gr * n + gc;
            *p = first ? cc[i][j][r] : *p + cc[i][j][r];
          }
        }
  }
}

// ---------------------------------------------------------------- finalize

__global__ __launch_bounds__(256) void finalize(const double* __restrict__ partials, int count,
                                                pwq_result* __restrict__ res,
                                                const DevFlags* flags) {
  __shared__ double s[3][256];
  if (flags->info != 0) return;
  double a = 0.0, b = 0.0, c = 0.0;
  for (int i = threadIdx.x; i < count; i += 256) {
    a += partials[(int64_t)i * 4 + 0];
    b += partials[(int64_t)i * 4 + 1];
    c += partials[(int64_t)i * 4 + 2];
  }
  s[0][threadIdx.x] = a;
  s[1][threadIdx.x] = b;
  s[2][threadIdx.x] = c;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) {
      s[0][threadIdx.x] += s[0][threadIdx.x + o];
      s[1][threadIdx.x] += s[1][threadIdx.x + o];
      s[2][threadIdx.x] += s[2][threadIdx.x + o];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    res->loss_damped = s[0][0];
    res->bound = 0.25 * s[1][0];
    res->delta_sq = s[2][0];
    res->loss = s[0][0] - res->lambda * s[2][0];
  }
}

template <typename T, int B>
hipError_t run_sweep(const SweepLaunch& sl, hipStream_t st) {
  SweepArgs<T> a;
  a.W = sl.W; a.wdtype = sl.wdtype; a.ldw = sl.ldw; a.m = (int)sl.m; a.n = (int)sl.n;
  a.L = (const T*)sl.L; a.invd = (const T*)sl.invd; a.dg = (const T*)sl.dg;
  a.alpha = sl.colspacing ? (const T*)sl.alpha : nullptr;
  a.scales = sl.scales; a.zeros = sl.zeros; a.ng = sl.ng; a.G = sl.G;
  a.colmap = sl.colmap; a.dead = sl.dead; a.acc = (T*)sl.acc; a.E = (T*)sl.E;
  a.codes = sl.codes; a.partials = sl.partials; a.flags = sl.flags;
  diag_prep<T><<<(unsigned)((sl.n + 255) / 256), 256, 0, st>>>(
      (const T*)sl.L, (int)sl.n, sl.colspacing, sl.c, sl.colmap, (T*)sl.invd, (T*)sl.dg,
      (T*)sl.alpha, sl.scales_out, sl.flags);
  const int nblk = (int)((sl.n + B - 1) / B);
  const unsigned nwg = (unsigned)((sl.m + 15) / 16);
  for (int b = nblk - 1; b >= 0 && nwg > 0; --b) {
    const int first = b == nblk - 1;
    sweep_block<T, B><<<nwg, 256, 0, st>>>(a, b, first);
    const int j0 = b * B;
    if (j0 > 0) {
      const int kb = (int)(sl.n - j0 < B ? sl.n - j0 : B);
      dim3 g((unsigned)((j0 + 127) / 128), (unsigned)((sl.m + 127) / 128));
      lazy_update<T><<<g, 256, 0, st>>>((const T*)sl.E, B, kb, (const T*)sl.L, (int)sl.n, j0,
                                        (int)sl.m, (T*)sl.acc, first, sl.flags);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  finalize<<<1, 256, 0, st>>>(sl.partials, nblk * (int)nwg, sl.result, sl.flags);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grid_steps(const void* W, int32_t wdtype, int64_t m, int64_t n, int64_t ldw,
                             const int32_t* dead, int kind, int bits, int G, float* scales,
                             int32_t* zeros, const DevFlags* flags, hipStream_t st) {
  const int64_t waves = m * (n / G);
  grid_steps_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, st>>>(
      W, wdtype, (int)m, (int)n, ldw, dead, kind, bits, G, scales, zeros, flags);
  return hipGetLastError();
}

size_t sweep_partials_bytes(int64_t m, int64_t n, int32_t block) {
  const int64_t nblk = (n + block - 1) / block;
  const int64_t nwg = (m + 15) / 16;
  return (size_t)(nblk * nwg * 4) * sizeof(double);
}

hipError_t launch_sweep(const SweepLaunch& sl, hipStream_t st) {
  if (sl.prec == PWQ_F64) {
    switch (sl.block) {
      case 32: return run_sweep<double, 32>(sl, st);
      case 64: return run_sweep<double, 64>(sl, st);
      case 128: return run_sweep<double, 128>(sl, st);
      case 256: return run_sweep<double, 256>(sl, st);
    }
  } else {
    switch (sl.block) {
      case 32: return run_sweep<float, 32>(sl, st);
      case 64: return run_sweep<float, 64>(sl, st);
      case 128: return run_sweep<float, 128>(sl, st);
      case 256: return run_sweep<float, 256>(sl, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace pwq
