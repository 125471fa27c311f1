// Rate of a quantized layer: the empirical Shannon entropy of each column's
// codes, in bits, and their mean over the columns.
//
// "WaterSIC: information-theoretically (near) optimal linear layer
// quantization", technical summary 2, items 1 and 3: columns get unequal
// rates, and the unclipped integer codes are entropy coded, so the rate of a
// column is the entropy of its code distribution.
//
// Design: codes are m x n row-major, so a wave reading one row of 64
// consecutive columns is coalesced.  colrange: per-column min / max.
// colhist: 64 columns per workgroup, a 512-bin LDS histogram per column
// (integer LDS atomics: exact counts), then per column
//     H = -sum_b p_b log2 p_b,  p_b = c_b / m,
// summed in bin order per lane and reduced in a fixed order (deterministic).
// Columns whose code range exceeds 512 values are done by colhist_wide, one
// workgroup per column with a 32768-bin histogram; wider ranges give NaN.
#include "pwq_device.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

constexpr int RC = 64;          // columns per workgroup
constexpr int NBIN = 512;       // bins per column in colhist
constexpr int NBIN_WIDE = 32768;

__global__ __launch_bounds__(256) void colrange(const int32_t* __restrict__ codes, int m, int n,
                                                int64_t ldc, int32_t* __restrict__ cmin,
                                                int32_t* __restrict__ cmax) {
  __shared__ int32_t smin[4][RC], smax[4][RC];
  const int col = blockIdx.x * RC + (threadIdx.x & 63), rg = threadIdx.x >> 6;
  int32_t lo = INT32_MAX, hi = INT32_MIN;
  if (col < n)
    for (int r = rg; r < m; r += 4) {
      const int32_t v = codes[(int64_t)r * ldc + col];
      lo = min(lo, v);
      hi = max(hi, v);
    }
  smin[rg][threadIdx.x & 63] = lo;
  smax[rg][threadIdx.x & 63] = hi;
  __syncthreads();
  if (rg == 0 && col < n) {
    const int c = threadIdx.x;
    cmin[col] = min(min(smin[0][c], smin[1][c]), min(smin[2][c], smin[3][c]));
    cmax[col] = max(max(smax[0][c], smax[1][c]), max(smax[2][c], smax[3][c]));
  }
}

// Entropy (bits) of one column from its histogram: every lane of the wave
// sums -p log2 p (p = c / m) over bins lane, lane + 64, ... in order; a
// fixed butterfly reduction follows.  A constant column gives exactly 0.
__device__ __forceinline__ double entropy_from_hist(const int32_t* h, int nbin, int m) {
  const int lane = threadIdx.x & 63;
  const double inv_m = 1.0 / (double)m;
  double s = 0.0;
  for (int b = lane; b < nbin; b += 64) {
    const int c = h[b];
    if (c > 0) {
      const double p = (double)c * inv_m;
      s -= p * log2(p);
    }
  }
  return wave_sum(s);
}

__global__ __launch_bounds__(256) void colhist(const int32_t* __restrict__ codes, int m, int n,
                                               int64_t ldc, const int32_t* __restrict__ cmin,
                                               const int32_t* __restrict__ cmax,
                                               double* __restrict__ bits) {
  __shared__ int32_t hist[RC][NBIN];    // 128 KB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * RC;
  for (int i = tid; i < RC * NBIN; i += 256) (&hist[0][0])[i] = 0;
  const int col = c0 + lane;
  const bool narrow = col < n && (int64_t)cmax[col] - cmin[col] < NBIN;
  const int32_t base = col < n ? cmin[col] : 0;
  __syncthreads();
  if (narrow)
    for (int r = wave; r < m; r += 4)
      atomicAdd(&hist[lane][codes[(int64_t)r * ldc + col] - base], 1);
  __syncthreads();
  // wave w: columns w, w + 4, ... of the workgroup
  for (int j = wave; j < RC; j += 4) {
    const int cj = c0 + j;
    if (cj >= n) break;
    if ((int64_t)cmax[cj] - cmin[cj] >= NBIN) continue;     // colhist_wide
    const double h = m > 0 ? entropy_from_hist(hist[j], NBIN, m) : 0.0;
    if (lane == 0) bits[cj] = h;
  }
}

__global__ __launch_bounds__(256) void colhist_wide(const int32_t* __restrict__ codes, int m,
                                                    int64_t ldc,
                                                    const int32_t* __restrict__ cmin,
                                                    const int32_t* __restrict__ cmax,
                                                    double* __restrict__ bits) {
  __shared__ int32_t hist[NBIN_WIDE];   // 128 KB
  const int col = blockIdx.x;
  const int64_t range = (int64_t)cmax[col] - cmin[col] + 1;
  if (range <= NBIN) return;            // done by colhist
  if (range > NBIN_WIDE) {
    if (threadIdx.x == 0) bits[col] = __builtin_nan("");
    return;
  }
  for (int i = threadIdx.x; i < NBIN_WIDE; i += 256) hist[i] = 0;
  __syncthreads();
  const int32_t base = cmin[col];
  for (int r = threadIdx.x; r < m; r += 256)
    atomicAdd(&hist[codes[(int64_t)r * ldc + col] - base], 1);
  __syncthreads();
  if (threadIdx.x < 64) {
    const double h = entropy_from_hist(hist, (int)range, m);
    if (threadIdx.x == 0) bits[col] = h;
  }
}

// Mean over the columns in a fixed order (fp64).
__global__ __launch_bounds__(256) void colmean(const double* __restrict__ bits, int n,
                                               double* __restrict__ mean) {
  __shared__ double s[256];
  double a = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) a += bits[i];
  s[threadIdx.x] = a;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *mean = n > 0 ? s[0] / (double)n : 0.0;
}

}  // namespace

hipError_t launch_column_entropy(const int32_t* codes, int64_t m, int64_t n, int64_t ldc,
                                 double* bits, double* mean, int32_t* cmin, int32_t* cmax,
                                 hipStream_t st) {
  if (n > 0) {
    const unsigned g = (unsigned)((n + RC - 1) / RC);
    colrange<<<g, 256, 0, st>>>(codes, (int)m, (int)n, ldc, cmin, cmax);
    colhist<<<g, 256, 0, st>>>(codes, (int)m, (int)n, ldc, cmin, cmax, bits);
    colhist_wide<<<(unsigned)n, 256, 0, st>>>(codes, (int)m, ldc, cmin, cmax, bits);
  }
  if (mean) colmean<<<1, 256, 0, st>>>(bits, (int)n, mean);
  return hipGetLastError();
}

}  // namespace pwq
