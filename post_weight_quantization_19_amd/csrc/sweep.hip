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
//  * the errors E reach the earlier columns through MFMA GEMMs,
//    acc[:, cols] += E L[blk, cols], in groups of blocks (256 columns in
//    fp32, 512 in fp64): after each block, its errors reach the open columns
//    of its own group; after a group's last block, the whole group's errors
//    reach every column before the group in one pass, so acc is read and
//    written once per group.  acc is written (not read) where a column is
//    first touched.
//  * losses are accumulated per workgroup in fp64 and summed in a fixed
//    order by a final one-workgroup kernel.
#include "pwq_device.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

// ---------------------------------------------------------------- steps

// One 16-lane quarter of a wave per (row, group): 16 groups per workgroup.
__global__ __launch_bounds__(256) void grid_steps_kernel(
    const void* __restrict__ W, int32_t wdtype, int m, int n, int64_t ldw,
    const int32_t* __restrict__ dead, int kind, int bits, int G, float kappa,
    float* __restrict__ scales, int32_t* __restrict__ zeros,
    const DevFlags* flags) {
  if (flags && flags->info != 0) return;
  const int ng = n / G;
  const int64_t gid = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  const bool live = gid < (int64_t)m * ng;
  const int r = live ? (int)(gid / ng) : 0, g = live ? (int)(gid % ng) : 0;
  float mx = -INFINITY, mn = INFINITY, amax = 0.0f;
  if (live) {
    for (int c = g * G + sub; c < (g + 1) * G; c += 16) {
      float w = load_w<float>(W, wdtype, (int64_t)r * ldw + c);
      if (dead && dead[c]) w = 0.0f;
      mx = fmaxf(mx, w);
      mn = fminf(mn, w);
      amax = fmaxf(amax, fabsf(w));
    }
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o, 16));
    mn = fminf(mn, __shfl_xor(mn, o, 16));
    amax = fmaxf(amax, __shfl_xor(amax, o, 16));
  }
  if (!live || sub != 0) return;
  // kappa: one multiplier on every step (1 by default), applied after the
  // zero-step rule; the asymmetric zero point follows the scaled step
  if (kind == PWQ_GRID_SYM) {
    float s = amax / (float)((1 << (bits - 1)) - 1);
    if (s == 0.0f) s = 1.0f;
    s *= kappa;
    scales[(int64_t)r * ng + g] = s;
  } else {
    const float lo = fminf(mn, 0.0f), hi = fmaxf(mx, 0.0f);
    float s = (hi - lo) / (float)((1 << bits) - 1);
    if (s == 0.0f) s = 1.0f;
    s *= kappa;
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

// 16-byte vector of T (4 floats or 2 doubles).
template <typename T> struct Vec16;
template <> struct Vec16<float> { typedef float4 type; };
template <> struct Vec16<double> { typedef double2 type; };

// Rows cb .. cb + CH - 1 of the block's strictly-lower part of L, stored
// transposed: Lt[i * LP + r] = L[j0 + cb + r][j0 + i] for i < cb + r (zero
// elsewhere and for rows past n), so the coefficients of one column i for
// consecutive rows are contiguous.  Thread t takes row r = t % CH and the
// column range (t / CH) of the block; consecutive lanes write consecutive
// LDS words.  `vec`: 16-byte loads (whole block inside the matrix, rows
// 16-byte aligned).
template <typename T, int B, int CH, int LP>
__device__ __forceinline__ void stage_lt(T* __restrict__ Lt, const T* __restrict__ L, int n,
                                         int j0, int cb, bool vec) {
  constexpr int VW = 16 / (int)sizeof(T);
  constexpr int PARTS = 256 / CH, CW = B / PARTS;
  static_assert(256 % CH == 0 && B % PARTS == 0 && CW % VW == 0, "staging shape");
  typedef typename Vec16<T>::type V;
  const int r = threadIdx.x % CH, part = threadIdx.x / CH;
  const int kr = cb + r;
  const bool rowok = j0 + kr < n;
  const T* src = L + (int64_t)(rowok ? j0 + kr : 0) * n + j0 + part * CW;
  // all of the thread's loads first, then the LDS writes (one wait)
  T v[CW];
  if (vec) {
    // uniform: the whole block lies inside the matrix, every row is valid
#pragma unroll
    for (int c = 0; c < CW; c += VW) {
      const V x = *(const V*)(src + c);
      __builtin_memcpy(&v[c], &x, sizeof(x));
    }
  } else {
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      const int i = part * CW + c;
      v[c] = (rowok && i < kr) ? src[c] : (T)0;
    }
  }
#pragma unroll
  for (int c = 0; c < CW; ++c) {
    const int i = part * CW + c;
    Lt[i * LP + r] = (rowok && i < kr) ? v[c] : (T)0;
  }
}

// One sub-block of Bi columns [j0, j0 + Bi) of every row.  E (leading
// dimension ldE) receives the sub-block's errors at column offset e_off.
template <typename T, int B>
__global__ __launch_bounds__(256) void sweep_block(SweepArgs<T> a, int j0, int ldE, int e_off,
                                                  int first, int part) {
  constexpr int P = 16, S = B / P;
  // rows of L staged per LDS pass (about 64 KB of the CU's 160 KB)
  constexpr int CH0 = 65536 / (B * (int)sizeof(T));
  constexpr int CH = CH0 < 8 ? 8 : (CH0 > B ? B : CH0);
  static_assert(B % CH == 0, "chunk must divide block");
  // L is read VW rows (columns of the sweep) at a time: one 16-byte LDS read
  // per slot covers the next VW columns
  constexpr int VW = 16 / (int)sizeof(T);
  constexpr int LP = CH + VW;           // padded: 16 lanes hit distinct banks
  static_assert(CH % VW == 0, "groups inside a chunk");
  typedef typename Vec16<T>::type V;
  __shared__ __attribute__((aligned(16))) T Lt[B * LP];
  __shared__ double red[4][4];
  // After a failed factorization or an invalid permutation (info != 0) the
  // column map may hold anything: no index is formed from it.  The flag is
  // the same for the whole launch, so every workgroup leaves before its
  // first barrier.
  if (a.flags->info != 0) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane & 15;
  const int row = blockIdx.x * 16 + wave * 4 + (lane >> 4);
  const bool rok = row < a.m;
  const int n = a.n;

  T acc[S], av[S], bv[S], sv[S], wv[S], dv[S];
  int ocv[S], zpv[S];
  // Every slot's loads are issued together, from indices clamped into the
  // arrays (row 0 / column 0 for slots outside the matrix), and the values
  // selected afterwards: no per-slot branch serializes their latencies.
  const int rowc = rok ? row : 0;
  int colc[S];
  bool okv[S];
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const int col = j0 + q + P * t;
    okv[t] = rok && col < n;
    colc[t] = okv[t] ? col : 0;
    ocv[t] = colc[t];
  }
  if (a.colmap) {
#pragma unroll
    for (int t = 0; t < S; ++t) ocv[t] = a.colmap[colc[t]];
  }
  // (uniform branches outside the slot loops, raw bits kept until every
  // load is in flight, so that no conversion forces an early wait)
  uint32_t wraw[S];
  int dd[S], zl[S];
  float sraw[S];
  T al0[S], il0[S], dl0[S], acl[S];
  int64_t gi[S];
#pragma unroll
  for (int t = 0; t < S; ++t) {
    gi[t] = (int64_t)rowc * a.ng + ocv[t] / a.G;
    dd[t] = 0;
    zl[t] = 0;
    sraw[t] = 1.0f;
    al0[t] = (T)1;
    acl[t] = (T)0;
  }
  if (a.wdtype == 1) {
    const uint16_t* W16 = (const uint16_t*)a.W + (int64_t)rowc * a.ldw;
#pragma unroll
    for (int t = 0; t < S; ++t) wraw[t] = W16[ocv[t]];
  } else {
    const uint32_t* W32 = (const uint32_t*)a.W + (int64_t)rowc * a.ldw;
#pragma unroll
    for (int t = 0; t < S; ++t) wraw[t] = W32[ocv[t]];
  }
  if (a.dead) {
#pragma unroll
    for (int t = 0; t < S; ++t) dd[t] = a.dead[ocv[t]];
  }
  if (a.alpha) {
#pragma unroll
    for (int t = 0; t < S; ++t) al0[t] = a.alpha[colc[t]];
  } else {
#pragma unroll
    for (int t = 0; t < S; ++t) sraw[t] = a.scales[gi[t]];
  }
  if (a.zeros) {
#pragma unroll
    for (int t = 0; t < S; ++t) zl[t] = a.zeros[gi[t]];
  }
#pragma unroll
  for (int t = 0; t < S; ++t) {
    il0[t] = a.invd[colc[t]];
    dl0[t] = a.dg[colc[t]];
  }
  if (!first) {
    const T* accr = a.acc + (int64_t)rowc * n;
#pragma unroll
    for (int t = 0; t < S; ++t) acl[t] = accr[colc[t]];
  }
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const bool ok = okv[t];
    const T wl = a.wdtype == 1 ? (T)bf16_to_f32((uint16_t)wraw[t]) : (T)__uint_as_float(wraw[t]);
    const T sl = a.alpha ? al0[t] : (T)sraw[t];
    const T w = (ok && !dd[t]) ? wl : (T)0;
    const T s = ok ? sl : (T)1;
    const T il = ok ? il0[t] : (T)0;
    const T d = ok ? dl0[t] : (T)0;
    const T ac = ok ? acl[t] : (T)0;
    const int zp = ok ? zl[t] : 0;
    ocv[t] = ok ? ocv[t] : -1;
    // true (correctly rounded) quotients: with no feedback yet the coordinate
    // is exactly w / s, so an exact tie is rounded to even as on paper
    acc[t] = ac;
    av[t] = il / s;
    bv[t] = w / s;
    // computed here, off the column chain (the compiler would otherwise
    // sink each division to the first column that uses it)
    pin(av[t]);
    pin(bv[t]);
    sv[t] = s;
    wv[t] = w;
    dv[t] = d;
    zpv[t] = zp;
  }
  int32_t* codes_row = a.codes + (int64_t)(rok ? row : 0) * n;
  T* e_row = a.E + (int64_t)(rok ? row : 0) * ldE + e_off;

  double loss_d = 0.0, bound = 0.0, dsq = 0.0;
  // coefficients l_kj of the current and the next group of VW columns (k),
  // for the lane's columns j = q + 16 t (one 16-byte LDS read per slot)
  V cur[S], nxt[S];
#pragma unroll
  for (int t = 0; t < S; ++t) {
    __builtin_memset(&cur[t], 0, sizeof(V));
    __builtin_memset(&nxt[t], 0, sizeof(V));
  }
  const bool vec = j0 + B <= n && n % VW == 0 && ((uintptr_t)a.L % 16) == 0;

  static_for_down<B - 1>([&](auto KK) {
    constexpr int kk = decltype(KK)::value;
    constexpr int t = kk / P, qk = kk % P;
    constexpr int pos = kk % VW;          // position in its group (VW-1 first)
    if constexpr (kk % CH == CH - 1) {
      // stage rows j0+kk-CH+1 .. j0+kk of L (strictly-lower part of the block)
      constexpr int cb = kk - CH + 1;
      __syncthreads();
      stage_lt<T, B, CH, LP>(Lt, a.L, n, j0, cb, vec);
      __syncthreads();
#pragma unroll
      for (int t2 = 0; t2 <= t; ++t2)
        cur[t2] = *(const V*)&Lt[(q + P * t2) * LP + (kk % CH) - (VW - 1)];
    }
    // the next group's coefficients, one group ahead, when already staged
    if constexpr (pos == VW - 1 && kk >= VW && (kk - VW) % CH != CH - 1) {
      constexpr int kn = kk - VW, tn = kn / P;
#pragma unroll
      for (int t2 = 0; t2 <= tn; ++t2)
        nxt[t2] = *(const V*)&Lt[(q + P * t2) * LP + (kn % CH) - (VW - 1)];
    }
    const T c = acc[t] * av[t] + bv[t];
    const T z = rint_t(c);
    const T e = wv[t] - sv[t] * z;
    const T eb = row_bcast<qk>(e);
#pragma unroll
    for (int t2 = 0; t2 <= t; ++t2) {
      acc[t2] += eb * (&cur[t2].x)[pos];
      // materialise the update here: without this the compiler sinks the
      // updates toward their distant use and keeps every broadcast alive
      pin(acc[t2]);
    }
    if constexpr (pos == 0) {
#pragma unroll
      for (int t2 = 0; t2 < S; ++t2) cur[t2] = nxt[t2];
    }
    // one column per scheduling region: bounded live ranges
    __builtin_amdgcn_sched_barrier(0);
  });

  // Record the decisions.  Slot t of every lane is final once column 16 t
  // has been swept (later columns add only the zero upper-triangle
  // coefficients to it), so the running target here is the one each column
  // was rounded at; done after the column chain to keep it short.
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const T cc = acc[t] * av[t] + bv[t];
    const T zz = rint_t(cc);
    const T rho = cc - zz;
    const T ee = wv[t] - sv[t] * zz;
    if (ocv[t] >= 0) {
      codes_row[ocv[t]] = (int32_t)zz + zpv[t];
      e_row[q + P * t] = ee;
      const double sl = (double)sv[t] * (double)dv[t];
      loss_d += (double)rho * (double)rho * sl * sl;
      bound += sl * sl;
      dsq += (double)ee * (double)ee;
    } else if (rok) {
      e_row[q + P * t] = (T)0;
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
    double* p = a.partials + ((int64_t)part * gridDim.x + blockIdx.x) * 4;
    p[0] = (red[0][0] + red[1][0]) + (red[2][0] + red[3][0]);
    p[1] = (red[0][1] + red[1][1]) + (red[2][1] + red[3][1]);
    p[2] = (red[0][2] + red[1][2]) + (red[2][2] + red[3][2]);
    p[3] = 0.0;
  }
}

// ------------------------------------------------------------ lazy update
// acc[r, c] (+)= sum_{k < kb} E[r, e_off + k] * L[k_lo + k, c]
//   for r < m and c in [c_lo, j0); "first" stores instead of adding.
// 128 x 128 output tiles.  The accumulators start from the current acc
// values (their loads are issued first, so their latency overlaps the
// operand loads and the MFMAs), K runs in chunks of 32 staged through LDS
// with the next chunk's global loads in flight while the current chunk's
// MFMAs run, and the tile is stored once.  fp32 rows that are not 16-byte
// aligned (the aligned ones take the kernels below); fp64 has its own form,
// lazy_update_f64.
template <typename T>
__global__ __launch_bounds__(256, 2) void lazy_update(
    const T* __restrict__ E, int B, int e_off, int kb, const T* __restrict__ L, int n,
    int k_lo, int c_lo, int j0, int m, T* __restrict__ acc, int first,
    const DevFlags* flags) {
  static_assert(sizeof(T) == 4, "fp32 only");
  constexpr int TM = 128, KC = 32, LDA = KC + 1, LDB = TM + 1;
  constexpr int PE = TM * KC / 256;   // elements per thread per operand
  __shared__ T Es[TM * LDA];
  __shared__ T Lt[KC * LDB];
  (void)flags;
  E += e_off;
  const int c0 = c_lo + blockIdx.x * TM, r0 = blockIdx.y * TM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  T re[PE], rl[PE];
  auto gload = [&](int kc) {
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const int e = tid + 256 * i;
      const int r = e / KC, k = e % KC;          // E tile [TM][KC]
      re[i] = (r0 + r < m && kc + k < kb) ? E[(int64_t)(r0 + r) * B + kc + k] : (T)0;
      const int kr = e / TM, cc = e % TM;        // L tile [KC][TM]
      rl[i] = (kc + kr < kb && c0 + cc < j0) ? L[(int64_t)(k_lo + kc + kr) * n + c0 + cc]
                                             : (T)0;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const int e = tid + 256 * i;
      Es[(e / KC) * LDA + e % KC] = re[i];
      Lt[(e / TM) * LDB + e % TM] = rl[i];
    }
  };

  // 32x32 result layout: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, col l%32
  f32x16_t cc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gr = r0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int gc = c0 + wn * 64 + j * 32 + (lane & 31);
        cc[i][j][r] = (!first && gr < m && gc < j0) ? acc[(int64_t)gr * n + gc] : 0.0f;
      }
  gload(0);
  for (int kc = 0; kc < kb; kc += KC) {
    __syncthreads();
    lstore();
    __syncthreads();
    if (kc + KC < kb) gload(kc + KC);
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
        if (gr < m && gc < j0) acc[(int64_t)gr * n + gc] = cc[i][j][r];
      }
}

// fp32 form of the same update for 16-byte aligned rows of L (n % 4 == 0),
// K <= 128.  Persistent, one 512-thread workgroup per CU: workgroup w owns
// row strip w % nstrip (128 rows) and visits the column tiles w / nstrip,
// w / nstrip + ngrp, ...  Each of the 8 waves keeps its 32 rows of E in
// registers for the whole launch as the MFMA A operand; the tile's panel of
// L (K x 128 columns, 64 KB) is copied into an LDS double buffer with
// global_load_lds_dwordx4 while the previous tile computes, and the next
// tile's acc values are loaded into registers at the same time, so HBM
// traffic and MFMAs overlap.  K is visited in a permuted order so that a
// lane's A values are four consecutive k of its row (one 16-byte load): in
// group g, MFMA t pairs k = 8g + t (lanes 0..31) with k = 8g + 4 + t
// (lanes 32..63).
// s_waitcnt immediate (gfx9 encoding): vmcnt <= v, expcnt and lgkmcnt not waited for.
constexpr int waitcnt_vm(int v) { return (v & 15) | (((v >> 4) & 3) << 14) | 0x70 | 0xF00; }

constexpr int UPD_NT = 512;
__global__ __launch_bounds__(UPD_NT, 1) void lazy_update_f32(
    const float* __restrict__ E, int B, int e_off, int kb, const float* __restrict__ L, int n,
    int k_lo, int c_lo, int j0, int m, float* __restrict__ acc, int first, int nstrip,
    int ngrp) {
  constexpr int TM = 128, KMAX = 128;
  __shared__ __attribute__((aligned(16))) float Ls[2][KMAX * TM];   // [k][col]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, h = lane >> 5;   // rows 32 wm, cols 64 wn
  const int ncol = (j0 - c_lo + TM - 1) / TM;
  const int r0 = (blockIdx.x % nstrip) * TM;
  const int tile0 = blockIdx.x / nstrip;
  if (tile0 >= ncol) return;

  // this wave's 32 rows of E: lane (row, h) holds k = 8g + 4h .. 8g + 4h + 3
  f32x4_t ea[16];
  {
    const int gr = r0 + wm * 32 + (lane & 31);
    const float* er = E + (int64_t)(gr < m ? gr : 0) * B + e_off + 4 * h;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
      const int k = 8 * g + 4 * h;
      if (gr < m && k + 3 < kb) {
        v = *(const f32x4_t*)(er + 8 * g);
      } else if (gr < m && k < kb) {   // ragged end of K: element by element
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (k + t < kb) v[t] = er[8 * g + t];
      }
      ea[g] = v;
    }
  }
  // L panel rows k_lo .. k_lo + kb - 1, columns c0 .. c0 + 127 -> LDS
  // buffer.  Rows past kb repeat row k_lo (their E values are zero); column
  // chunks past n read the last chunk of the row (those outputs are not
  // stored).
  auto fetch_l = [&](int c0, int buf) {
#pragma unroll
    for (int i = 0; i < KMAX * TM / 4 / UPD_NT; ++i) {
      const int ci = tid + UPD_NT * i;         // 16-byte chunk of the [k][col] panel
      const int k = ci / (TM / 4), q = ci % (TM / 4);
      const int row = k_lo + (k < kb ? k : 0);
      const int col = min(c0 + 4 * q, n - 4);
      __builtin_amdgcn_global_load_lds(
          (const void*)(L + (int64_t)row * n + col),
          (__attribute__((address_space(3))) void*)&Ls[buf][(wave * 64 + UPD_NT * i) * 4], 16,
          0, 0);
    }
  };
  // acc goes through a buffer resource: an element outside the tile's valid
  // range gets an out-of-range offset, so its load returns 0 and its store
  // is dropped, and every lane issues the same 32 loads / 32 stores per tile
  // (the in-order vmcnt wait below relies on that count).
  const __amdgpu_buffer_rsrc_t racc =
      __builtin_amdgcn_make_buffer_rsrc(acc, 0, m * n * 4, 0x00020000);
  // 32x32 result layout: lane l, register r -> row 8(r/4) + 4(l/32) + r%4, col l%32
  const int rbase = r0 + wm * 32 + 4 * (lane >> 5);
  auto c_off = [&](int c0, int j, int r) -> int {
    const int gr = rbase + 8 * (r >> 2) + (r & 3);
    const int gc = c0 + wn * 64 + j * 32 + (lane & 31);
    return (gr < m && gc < j0) ? (gr * n + gc) * 4 : -1;
  };
  // on the first block acc is written, not read: every load is out of range
  const int lmask = first ? -1 : 0;
  auto fetch_c = [&](int c0, f32x16_t (&cn)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        cn[j][r] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(racc, c_off(c0, j, r) | lmask, 0, 0));
  };

  // One tile: its acc values (already in `cur`) += E L; the next tile's L
  // panel and acc values go to the other buffer and `nxt` meanwhile.
  // Returns false after the last tile.  Two register sets alternate, so the
  // loop below is unrolled by two.
  int t = tile0;
  auto step = [&](f32x16_t (&cur)[2], f32x16_t (&nxt)[2], int buf) -> bool {
    const int c0 = c_lo + t * TM;
    // This tile's L panel and acc values were issued before the previous
    // tile's 32 stores; vector memory counts complete in order, so waiting
    // until at most 32 remain leaves only those stores in flight.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(32));
    lds_barrier();
    const int tn = t + ngrp;
    if (tn < ncol) {
      fetch_l(c_lo + tn * TM, buf ^ 1);
      // all LDS copies before the acc loads: a copy placed after them makes
      // the compiler wait for every outstanding load first
      __builtin_amdgcn_sched_barrier(0);
      fetch_c(c_lo + tn * TM, nxt);
    }
    // Every group runs: past kb the E values are zero (and the L rows
    // finite), so the extra products add exactly 0.  Each group's 4 LDS
    // reads are issued together ahead of its 8 MFMAs.
    const float* Lb = Ls[buf] + 4 * h * TM + wn * 64 + (lane & 31);
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      float bv[4][2];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        bv[tt][0] = Lb[(8 * g + tt) * TM];
        bv[tt][1] = Lb[(8 * g + tt) * TM + 32];
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        cur[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(ea[g][tt], bv[tt][0], cur[0], 0, 0, 0);
        cur[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(ea[g][tt], bv[tt][1], cur[1], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(cur[j][r]), racc,
                                              c_off(c0, j, r), 0, 0);
    t = tn;
    return tn < ncol;
  };

  f32x16_t ca[2], cb[2];
  fetch_l(c_lo + t * TM, 0);
  __builtin_amdgcn_sched_barrier(0);
  fetch_c(c_lo + t * TM, ca);
  __builtin_amdgcn_s_waitcnt(0);     // E, the first L panel and acc values
  while (step(ca, cb, 0) && step(cb, ca, 1)) {
  }
}

// The update of a whole group of blocks (K up to 128 NCH), for fp32 with
// 16-byte aligned rows: acc[:, c_lo:j0] += E L over the errors of every
// block of the group at once, so acc is read and written once per group
// instead of once per block.  Persistent, one 512-thread workgroup per CU
// owning row strip w % nstrip (128 rows) and the column tiles w / nstrip,
// w / nstrip + ngrp, ...  Wave v takes rows 16 v .. 16 v + 15 of the strip
// and all 128 columns of a tile as eight v_mfma_f32_16x16x4f32
// accumulators, so every row of E is held by one wave only and the whole
// strip's E stays in registers for the launch: lane (r, q) = (l % 16,
// l / 16) holds E[r][16 g + 4 q .. 16 g + 4 q + 3] for every 16-row group g
// of K (one 16-byte load each).  MFMA step s of group g sums
// k = 16 g + 4 q + s over the lane groups q; the B operand of lane (c, q)
// is L[k_lo + 16 g + 4 q + s][c0 + 16 j + c], read from LDS.  K runs in
// chunks of 128 rows of L (64 KB), double-buffered in LDS and copied with
// global_load_lds_dwordx4 one chunk ahead; a tile's acc values are loaded
// during its predecessor's last chunk and stored once after its own last
// chunk.  The four rows one MFMA step reads are 512 B apart, so the 16-byte
// column chunks of row k are stored XOR-swizzled by 4 ((k / 4) mod 4): the
// lane groups then read distinct banks.
// 16x16 result layout: lane l, register r -> row 4 (l / 16) + r, col l % 16.
template <int NCH>
__global__ __launch_bounds__(UPD_NT, 1) void lazy_update_f32_group(
    const float* __restrict__ E, int ldE, int e_off, int kb, const float* __restrict__ L,
    int n, int k_lo, int c_lo, int j0, int m, float* __restrict__ acc, int first, int nstrip,
    int ngrp) {
  constexpr int TM = 128, KC = 128;
  __shared__ __attribute__((aligned(16))) float Ls[2][KC * TM];   // [k][col]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int ncol = (j0 - c_lo + TM - 1) / TM;
  const int r0 = (blockIdx.x % nstrip) * TM;
  const int tile0 = blockIdx.x / nstrip;
  if (tile0 >= ncol) return;
  const int nch = (kb + KC - 1) / KC;   // 1 .. NCH

  // the strip's E: ea[8 ch + g] = E[row][e_off + 128 ch + 16 g + 4 lq + 0..3]
  // (zero past kb)
  f32x4_t ea[NCH * 8];
  {
    const int gr = r0 + 16 * wave + lr;
    const float* er = E + (int64_t)(gr < m ? gr : 0) * ldE + e_off + 4 * lq;
#pragma unroll
    for (int i = 0; i < NCH * 8; ++i) {
      f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
      const int k = 16 * i + 4 * lq;
      if (gr < m && k + 3 < kb) {
        v = *(const f32x4_t*)(er + 16 * i);
      } else if (gr < m && k < kb) {   // ragged end of K: element by element
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (k + t < kb) v[t] = er[16 * i + t];
      }
      ea[i] = v;
    }
  }
  // chunk ch of the L panel (rows k_lo + 128 ch .., columns c0 .. c0 + 127)
  // -> LDS buffer (physical 16-byte chunk q of row r holds logical chunk
  // q ^ 4 ((r / 4) mod 4)).  Rows past kb repeat row k_lo (their E values are
  // zero); column chunks past n read the last chunk of the row (those
  // outputs are not stored).
  auto fetch_l = [&](int c0, int ch, int buf) {
#pragma unroll
    for (int i = 0; i < KC * TM / 4 / UPD_NT; ++i) {
      const int ci = tid + UPD_NT * i;         // 16-byte chunk of the [k][col] panel
      const int r = ci / (TM / 4), k = KC * ch + r;
      const int q = (ci % (TM / 4)) ^ (4 * ((r >> 2) & 3));
      const int row = k_lo + (k < kb ? k : 0);
      const int col = min(c0 + 4 * q, n - 4);
      __builtin_amdgcn_global_load_lds(
          (const void*)(L + (int64_t)row * n + col),
          (__attribute__((address_space(3))) void*)&Ls[buf][(wave * 64 + UPD_NT * i) * 4], 16,
          0, 0);
    }
  };
  // acc through a buffer resource: an element outside the tile's valid range
  // gets an out-of-range offset (its load returns 0, its store is dropped),
  // so every lane issues the same 32 loads / 32 stores per tile (the
  // in-order vmcnt waits below rely on that count)
  const __amdgpu_buffer_rsrc_t racc =
      __builtin_amdgcn_make_buffer_rsrc(acc, 0, m * n * 4, 0x00020000);
  const int rbase = r0 + 16 * wave + 4 * lq;
  auto c_off = [&](int c0, int j, int r) -> int {
    const int gr = rbase + r, gc = c0 + 16 * j + lr;
    return (gr < m && gc < j0) ? (gr * n + gc) * 4 : -1;
  };
  const int lmask = first ? -1 : 0;   // first update: acc is written, not read
  auto fetch_c = [&](int c0, f32x4_t (&cn)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        cn[j][r] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(racc, c_off(c0, j, r) | lmask, 0, 0));
  };

  int t = tile0, buf = 0;
  // One tile: every chunk of K into `cur` (its acc values already there),
  // then one store.  The next chunk (or the next tile's first chunk and its
  // acc values, into `nxt`) is copied while this chunk's MFMAs run.
  auto tile = [&](f32x4_t (&cur)[8], f32x4_t (&nxt)[8]) -> bool {
    const int c0 = c_lo + t * TM;
    const int tn = t + ngrp;
    static_for_up<NCH>([&](auto CH) {
      constexpr int ch = decltype(CH)::value;
      if (ch < nch) {
        // This chunk's copy (and on the first chunk the tile's acc values)
        // was issued before the previous tile's 32 stores; vector memory
        // counts complete in order, so on the first chunk waiting until at
        // most 32 remain leaves only those stores in flight.
        if (ch == 0)
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(32));
        else
          __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        lds_barrier();
        if (ch + 1 < nch) {
          fetch_l(c0, ch + 1, buf ^ 1);
        } else if (tn < ncol) {
          fetch_l(c_lo + tn * TM, 0, buf ^ 1);
          // the LDS copies before the acc loads (as in lazy_update_f32)
          __builtin_amdgcn_sched_barrier(0);
          fetch_c(c_lo + tn * TM, nxt);
        }
        // step i = 4 g + sk reads row 16 g + 4 lq + sk, logical columns
        // 16 j + lr (physical 16 (j ^ lq) + lr); the reads of step i + 1 are
        // issued before the MFMAs of step i (two operand sets in turn)
        const float* Lb = Ls[buf] + 4 * lq * TM + lr;
        float bv[2][8];
        auto rd = [&](int i, float (&v)[8]) {
#pragma unroll
          for (int j = 0; j < 8; ++j) v[j] = Lb[(16 * (i >> 2) + (i & 3)) * TM + 16 * (j ^ lq)];
        };
        rd(0, bv[0]);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (i + 1 < 32) rd(i + 1, bv[(i + 1) & 1]);
#pragma unroll
          for (int j = 0; j < 8; ++j)
            cur[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[8 * ch + (i >> 2)][i & 3],
                                                          bv[i & 1][j], cur[j], 0, 0, 0);
          if (i + 1 < 32) __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
        buf ^= 1;
      }
    });
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(cur[j][r]), racc, c_off(c0, j, r),
                                              0, 0);
    t = tn;
    return tn < ncol;
  };

  f32x4_t ca[8], cb[8];
  fetch_l(c_lo + t * TM, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
  fetch_c(c_lo + t * TM, ca);
  __builtin_amdgcn_s_waitcnt(0);     // E, the first chunk and the acc values
  while (tile(ca, cb) && tile(cb, ca)) {
  }
}

// A lazy update over a narrow column range (K <= 128), for fp32 with
// 16-byte aligned rows: a block's errors reaching the open columns of its
// own group, which the persistent kernels would give to only a few
// workgroups.  One 256-thread workgroup per 16 rows and 128 columns; wave w
// takes columns 32 w .. 32 w + 31 as two v_mfma_f32_16x16x4f32
// accumulators, with E and L loaded straight into registers (both are small
// and shared through L2): lane (r, q) = (l % 16, l / 16) holds
// E[r][16 g + 4 q .. 16 g + 4 q + 3] and L[k_lo + 16 g + 4 q + s][c + r]
// for its columns c, so MFMA step s of group g sums k = 16 g + 4 q + s over
// the lane groups q.
// 16x16 result layout: lane l, register r -> row 4 (l / 16) + r, col l % 16.
__global__ __launch_bounds__(256) void near_update_f32(
    const float* __restrict__ E, int ldE, int e_off, int kb, const float* __restrict__ L,
    int n, int k_lo, int c_lo, int j0, int m, float* __restrict__ acc, int first) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int r0 = blockIdx.x * 16;
  const int c0 = c_lo + blockIdx.y * 128 + 32 * wave;
  if (c0 >= j0) return;   // the wave's columns are all past the range
  // E rows past m read row m - 1 and K past kb reads zeros (outputs of rows
  // past m are not stored)
  const float* er = E + (int64_t)min(r0 + lr, m - 1) * ldE + e_off + 4 * lq;
  f32x4_t ea[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    const int k = 16 * g + 4 * lq;
    f32x4_t v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (k + 3 < kb) {
      v = *(const f32x4_t*)(er + 16 * g);
    } else if (k < kb) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (k + t < kb) v[t] = er[16 * g + t];
    }
    ea[g] = v;
  }
  // L rows past kb repeat row k_lo (their E values are zero); columns past
  // n - 1 read column n - 1 (those outputs are not stored)
  float bv[8][4][2];
#pragma unroll
  for (int g = 0; g < 8; ++g)
#pragma unroll
    for (int sk = 0; sk < 4; ++sk) {
      const int k = 16 * g + 4 * lq + sk;
      const float* lrow = L + (int64_t)(k < kb ? k_lo + k : k_lo) * n;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) bv[g][sk][jj] = lrow[min(c0 + 16 * jj + lr, n - 1)];
    }
  f32x4_t c[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gr = r0 + 4 * lq + r, gc = c0 + 16 * jj + lr;
      c[jj][r] = (!first && gr < m && gc < j0) ? acc[(int64_t)gr * n + gc] : 0.0f;
    }
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    if (16 * g >= kb) break;   // uniform
#pragma unroll
    for (int sk = 0; sk < 4; ++sk)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
        c[jj] = __builtin_amdgcn_mfma_f32_16x16x4f32(ea[g][sk], bv[g][sk][jj], c[jj], 0, 0, 0);
  }
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int gr = r0 + 4 * lq + r, gc = c0 + 16 * jj + lr;
      if (gr < m && gc < j0) acc[(int64_t)gr * n + gc] = c[jj][r];
    }
}

// fp64 form of the generic update: the same tiles and K order (chunks of
// 32 through LDS, v_mfma_f64_16x16x4f64), with eight waves of 32 x 64 per
// 128 x 128 tile, so that each SIMD has two waves to cover the other's LDS
// and barrier waits, and a double-buffered LDS stage: the next chunk's
// global loads are in flight under the current chunk's MFMAs and are
// written to the other buffer afterwards, one barrier per chunk.
constexpr int F64U_NT = 512;
__global__ __launch_bounds__(F64U_NT, 1) void lazy_update_f64(
    const double* __restrict__ E, int B, int e_off, int kb, const double* __restrict__ L, int n,
    int k_lo, int c_lo, int j0, int m, double* __restrict__ acc, int first) {
  constexpr int TM = 128, KC = 32, LDA = KC + 1, LDB = TM + 1;
  constexpr int PE = TM * KC / F64U_NT;   // elements per thread per operand
  __shared__ double Es[2][TM * LDA];
  __shared__ double Lt[2][KC * LDB];
  E += e_off;
  const int c0 = c_lo + blockIdx.x * TM, r0 = blockIdx.y * TM;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;   // rows 32 wm, columns 64 wn of the tile
  double re[PE], rl[PE];
  auto gload = [&](int kc) {
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const int e = tid + F64U_NT * i;
      const int r = e / KC, k = e % KC;          // E tile [TM][KC]
      re[i] = (r0 + r < m && kc + k < kb) ? E[(int64_t)(r0 + r) * B + kc + k] : 0.0;
      const int kr = e / TM, cc = e % TM;        // L tile [KC][TM]
      rl[i] = (kc + kr < kb && c0 + cc < j0) ? L[(int64_t)(k_lo + kc + kr) * n + c0 + cc] : 0.0;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const int e = tid + F64U_NT * i;
      Es[buf][(e / KC) * LDA + e % KC] = re[i];
      Lt[buf][(e / TM) * LDB + e % TM] = rl[i];
    }
  };
  // 16x16 f64 result layout: lane l, register r -> row 4r + l/16, col l%16
  f64x4_t cc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gr = r0 + wm * 32 + i * 16 + 4 * r + (lane >> 4);
        const int gc = c0 + wn * 64 + j * 16 + (lane & 15);
        cc[i][j][r] = (!first && gr < m && gc < j0) ? acc[(int64_t)gr * n + gc] : 0.0;
      }
  gload(0);
  lstore(0);
  __syncthreads();
  const int nch = (kb + KC - 1) / KC;
  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    if (c + 1 < nch) gload((c + 1) * KC);
    const double* Eb = Es[buf];
    const double* Lb = Lt[buf];
#pragma unroll 2
    for (int k = 0; k < KC; k += 4) {
      const int ko = k + (lane >> 4);
      double av[2], bv[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = Eb[(wm * 32 + i * 16 + (lane & 15)) * LDA + ko];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Lb[ko * LDB + wn * 64 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          cc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[i], bv[j], cc[i][j], 0, 0, 0);
    }
    // the other buffer's readers (chunk c - 1) passed the previous barrier
    if (c + 1 < nch) lstore(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gr = r0 + wm * 32 + i * 16 + 4 * r + (lane >> 4);
        const int gc = c0 + wn * 64 + j * 16 + (lane & 15);
        if (gr < m && gc < j0) acc[(int64_t)gr * n + gc] = cc[i][j][r];
      }
}

// One lazy update launch: acc[:, c_lo:j0] (+)= E[:, e_off:e_off+kb] L[k_lo:k_lo+kb, c_lo:j0]
// (E with leading dimension ldE).
template <typename T>
void update_launch(const T* E, int ldE, int e_off, int kb, const T* L, int n, int k_lo, int c_lo,
                   int j0, int m, T* acc, int first, const DevFlags* flags, hipStream_t st) {
  dim3 g((unsigned)((j0 - c_lo + 127) / 128), (unsigned)((m + 127) / 128));
  if constexpr (sizeof(T) == 4) {
    if (n % 4 == 0 && ((uintptr_t)L % 16) == 0 && ((uintptr_t)E % 16) == 0 && ldE % 4 == 0 &&
        e_off % 4 == 0 && (int64_t)m * n * 4 < ((int64_t)1 << 31)) {
      if (kb <= 128 && j0 - c_lo <= 256) {
        // a narrow range: one workgroup per 16 rows and 128 columns
        near_update_f32<<<dim3((unsigned)((m + 15) / 16), (unsigned)((j0 - c_lo + 127) / 128)),
                          256, 0, st>>>(E, ldE, e_off, kb, L, n, k_lo, c_lo, j0, m, acc, first);
        return;
      }
      // one workgroup per CU: every row strip, as many column groups as fit
      const int nstrip = (m + 127) / 128;
      const int ncol = (j0 - c_lo + 127) / 128;
      int ngrp = 256 / nstrip;
      if (ngrp < 1) ngrp = 1;
      if (ngrp > ncol) ngrp = ncol;
      if (kb <= 128)
        lazy_update_f32<<<(unsigned)(nstrip * ngrp), UPD_NT, 0, st>>>(
            E, ldE, e_off, kb, L, n, k_lo, c_lo, j0, m, acc, first, nstrip, ngrp);
      else if (kb <= 256)
        lazy_update_f32_group<2><<<(unsigned)(nstrip * ngrp), UPD_NT, 0, st>>>(
            E, ldE, e_off, kb, L, n, k_lo, c_lo, j0, m, acc, first, nstrip, ngrp);
      // (K = 512 would need 128 registers of E per lane: more than fit)
      if (kb <= 256) return;
      // wider K: the generic kernel below
    }
  }
  if constexpr (sizeof(T) == 8)
    lazy_update_f64<<<g, F64U_NT, 0, st>>>(E, ldE, e_off, kb, L, n, k_lo, c_lo, j0, m, acc,
                                           first);
  else
    lazy_update<T><<<g, 256, 0, st>>>(E, ldE, e_off, kb, L, n, k_lo, c_lo, j0, m, acc, first,
                                      flags);
}

// ---------------------------------------------------------------- finalize

__global__ __launch_bounds__(256) void finalize(const double* __restrict__ partials, int count,
                                                pwq_result* __restrict__ res,
                                                const DevFlags* flags) {
  __shared__ double s[3][256];
  if (flags->info != 0) return;
  double a = 0.0, b = 0.0, c = 0.0;
#pragma unroll 8
  for (int i = threadIdx.x; i < count; i += 256) {
    const double4 v = *(const double4*)(partials + (int64_t)i * 4);
    a += v.x;
    b += v.y;
    c += v.z;
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

// Columns swept per kernel launch: a lazy block of B columns is swept in
// sub-blocks of Bi, with a small MFMA update inside the block between them
// (the same arithmetic regrouped; keeps the per-lane state in registers).
int inner_block(int32_t prec, int32_t block) {
  const int cap = 128;
  return block < cap ? block : cap;
}

int64_t sweep_parts(int64_t n, int32_t block, int32_t prec) {
  const int bi = inner_block(prec, block);
  int64_t parts = 0;
  for (int64_t jb0 = 0; jb0 < n; jb0 += block) {
    const int64_t w = (n - jb0 < block) ? n - jb0 : block;
    parts += (w + bi - 1) / bi;
  }
  return parts;
}

template <typename T, int Bi>
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
  const int n = (int)sl.n, m = (int)sl.m, B = sl.block;
  const int nblk = (n + B - 1) / B;
  const unsigned nwg = (unsigned)((m + 15) / 16);
  // Blocks go in groups of grp (update_group_cols columns).  A block's errors
  // reach the open columns of its own group at once (K = the block); the
  // columns before the group receive the errors of the whole group in one
  // pass once its last block is swept (K = the group), so acc is read and
  // written once per group rather than once per block.  E holds the group's
  // errors (leading dimension ldE), block b at column (b - first block) B.
  const int grp = update_group_cols(sl.prec) / B, ldE = grp * B;
  const int top = (nblk - 1) / grp;
  int part = 0;
  KernelTimer& tsweep = g_timers[PWQ_TIMER_SWEEP_BLOCK];
  KernelTimer& tupd = g_timers[PWQ_TIMER_LAZY_UPDATE];
  auto timed_update = [&](int e_off, int kb, int k_lo, int c_lo, int j0, int first) {
    hipError_t te = hipSuccess;
    const int64_t ti = tupd.begin(st, &te);
    if (te != hipSuccess) return te;
    update_launch<T>((const T*)sl.E, ldE, e_off, kb, (const T*)sl.L, n, k_lo, c_lo, j0, m,
                     (T*)sl.acc, first, sl.flags, st);
    return tupd.end(ti, st);
  };
  for (int b = nblk - 1; b >= 0 && nwg > 0; --b) {
    const int jb0 = b * B, jb1 = (n < jb0 + B) ? n : jb0 + B;
    const int gb0 = (b / grp) * grp, cg0 = gb0 * B, e_base = (b - gb0) * B;
    const int nsub = (jb1 - jb0 + Bi - 1) / Bi;
    for (int s = nsub - 1; s >= 0; --s) {
      const int js0 = jb0 + s * Bi;
      const int first_sub = (b == nblk - 1) && (s == nsub - 1);
      hipError_t te = hipSuccess;
      int64_t ti = tsweep.begin(st, &te);
      if (te != hipSuccess) return te;
      sweep_block<T, Bi><<<nwg, 256, 0, st>>>(a, js0, ldE, e_base + js0 - jb0, first_sub,
                                               part++);
      te = tsweep.end(ti, st);
      if (te != hipSuccess) return te;
      if (s > 0) {
        // the sub-block's errors reach the open columns of its own block
        const int kb = (jb1 - js0 < Bi) ? jb1 - js0 : Bi;
        te = timed_update(e_base + js0 - jb0, kb, js0, jb0, js0, first_sub);
        if (te != hipSuccess) return te;
      }
    }
    if (jb0 > cg0) {   // the block's errors reach the open columns of its group
      const hipError_t te = timed_update(e_base, jb1 - jb0, jb0, cg0, jb0, b == nblk - 1);
      if (te != hipSuccess) return te;
    }
    if (b == gb0 && cg0 > 0) {   // the group's errors reach every earlier column
      const int kg = ((n < cg0 + ldE) ? n : cg0 + ldE) - cg0;
      const hipError_t te = timed_update(0, kg, cg0, 0, cg0, b / grp == top);
      if (te != hipSuccess) return te;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  finalize<<<1, 256, 0, st>>>(sl.partials, part * (int)nwg, sl.result, sl.flags);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grid_steps(const void* W, int32_t wdtype, int64_t m, int64_t n, int64_t ldw,
                             const int32_t* dead, int kind, int bits, int G, float* scales,
                             int32_t* zeros, const DevFlags* flags, hipStream_t st, float kappa) {
  const int64_t groups = m * (n / G);
  grid_steps_kernel<<<(unsigned)((groups + 15) / 16), 256, 0, st>>>(
      W, wdtype, (int)m, (int)n, ldw, dead, kind, bits, G, kappa, scales, zeros, flags);
  return hipGetLastError();
}

size_t sweep_partials_bytes(int64_t m, int64_t n, int32_t block, int32_t prec) {
  const int64_t nwg = (m + 15) / 16;
  return (size_t)(sweep_parts(n, block, prec) * nwg * 4) * sizeof(double);
}

hipError_t launch_sweep(const SweepLaunch& sl, hipStream_t st) {
  const int bi = inner_block(sl.prec, sl.block);
  if (sl.prec == PWQ_F64) {
    switch (bi) {
      case 32: return run_sweep<double, 32>(sl, st);
      case 64: return run_sweep<double, 64>(sl, st);
      case 128: return run_sweep<double, 128>(sl, st);
    }
  } else {
    switch (bi) {
      case 32: return run_sweep<float, 32>(sl, st);
      case 64: return run_sweep<float, 64>(sl, st);
      case 128: return run_sweep<float, 128>(sl, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace pwq
