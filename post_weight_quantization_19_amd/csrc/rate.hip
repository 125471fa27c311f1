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
// workgroup per column with a 32768-bin histogram; columns wider still (with
// m <= 16384) are sorted there instead, and the length of every run of equal
// codes is put at the run's first position, which makes a histogram of
// their distinct values (zeros elsewhere) for the same entropy and Huffman
// steps.
//
// Huffman-coded length ("The Geometry of LLM Quantization ...", technical
// summary 3, HPTQ: the unconstrained integer codes are Huffman coded): the
// column's counts are sorted (bitonic network in LDS) and merged with the
// two-queue method -- leaves in ascending order in one queue, merged nodes
// (non-decreasing) in the other, each step joins the two smallest fronts --
// and the total length is the sum of the merged weights, an integer that
// every optimal prefix code of those counts shares.
#include "pwq_device.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

constexpr int RC = 64;          // columns per workgroup
constexpr int NBIN = 512;       // bins per column in colhist
constexpr int NBIN_WIDE = 32768;
constexpr int NSORT = NBIN_WIDE / 2;   // rows a column may have for the sorted path

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

// Sort h[0..len) ascending in place (len a power of two); the calling
// threads tid = 0 .. nthr-1 of a wave or workgroup take the compare-exchange
// pairs in turn; `sync` orders the stages.
template <typename Sync>
__device__ __forceinline__ void bitonic_sort(int32_t* h, int len, int tid, int nthr, Sync&& sync) {
  for (int size = 2; size <= len; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < len / 2; t += nthr) {
        const int i = (t / stride) * 2 * stride + (t % stride), j = i + stride;
        const int32_t a = h[i], b = h[j];
        const bool asc = (i & size) == 0;
        if ((a > b) == asc) {
          h[i] = b;
          h[j] = a;
        }
      }
      sync();
    }
}

// Two-queue Huffman total over the ascending counts leaf[lo..hi) (zeros
// already skipped); merged weights go to node[] (capacity hi - lo).  One
// thread.
__device__ __forceinline__ int64_t huffman_merge(const int32_t* leaf, int lo, int hi,
                                                 int32_t* node) {
  int li = lo, nh = 0, nt = 0;
  int64_t total = 0;
  auto pop = [&]() -> int32_t {
    if (nh < nt && (li >= hi || node[nh] < leaf[li])) return node[nh++];
    return leaf[li++];
  };
  for (int left = hi - lo; left > 1; --left) {
    const int32_t a = pop();
    const int32_t b = pop();
    const int32_t w = a + b;
    total += w;
    node[nt++] = w;
  }
  return total;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS accesses done
  __builtin_amdgcn_wave_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__global__ __launch_bounds__(256) void colhist(const int32_t* __restrict__ codes, int m, int n,
                                               int64_t ldc, const int32_t* __restrict__ cmin,
                                               const int32_t* __restrict__ cmax,
                                               double* __restrict__ bits,
                                               int64_t* __restrict__ huff) {
  __shared__ int32_t hist[RC][NBIN];    // 128 KB
  __shared__ int32_t nodes[4][NBIN];    // Huffman node queue per wave
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
    if (huff) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      bitonic_sort(hist[j], NBIN, lane, 64, wave_lds_sync);
      int nz = 0;                                  // zero counts come first
      for (int b = lane; b < NBIN; b += 64) nz += hist[j][b] == 0;
      for (int o = 32; o >= 1; o >>= 1) nz += __shfl_xor(nz, o, 64);
      if (lane == 0) huff[cj] = huffman_merge(hist[j], nz, NBIN, nodes[wave]);
      wave_lds_sync();
    }
  }
}

__global__ __launch_bounds__(256) void colhist_wide(const int32_t* __restrict__ codes, int m,
                                                    int64_t ldc,
                                                    const int32_t* __restrict__ cmin,
                                                    const int32_t* __restrict__ cmax,
                                                    double* __restrict__ bits,
                                                    int64_t* __restrict__ huff) {
  __shared__ int32_t hist[NBIN_WIDE];   // 128 KB
  __shared__ int32_t nzs[4];
  const int col = blockIdx.x;
  const int64_t range = (int64_t)cmax[col] - cmin[col] + 1;
  if (range <= NBIN) return;            // done by colhist
  const auto sync = [] { __syncthreads(); };
  if (range <= NBIN_WIDE) {
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
    if (!huff) return;
    __syncthreads();
    bitonic_sort(hist, NBIN_WIDE, threadIdx.x, 256, sync);
    int nz = 0;
    for (int b = threadIdx.x; b < NBIN_WIDE; b += 256) nz += hist[b] == 0;
    for (int o = 32; o >= 1; o >>= 1) nz += __shfl_xor(nz, o, 64);
    if ((threadIdx.x & 63) == 0) nzs[threadIdx.x >> 6] = nz;
    __syncthreads();
    if (threadIdx.x == 0) {
      const int z = nzs[0] + nzs[1] + nzs[2] + nzs[3];
      // the merged nodes go into the zero prefix; too many symbols: -1
      huff[col] = (NBIN_WIDE - z <= z + 1) ? huffman_merge(hist, z, NBIN_WIDE, hist) : -1;
    }
    return;
  }
  // Wider: sort the column's codes (padded with INT32_MAX to a power of
  // two), put each run's length at its first position, and take the entropy
  // and the Huffman total over those counts.  sv: the sorted codes, later
  // the Huffman node queue; cv: the counts.
  if (m > NSORT) {
    if (threadIdx.x == 0) {
      bits[col] = __builtin_nan("");
      if (huff) huff[col] = -1;
    }
    return;
  }
  int32_t* sv = hist;
  int32_t* cv = hist + NSORT;
  int len = 2;                          // m >= 2: the range spans two values
  while (len < m) len <<= 1;
  for (int i = threadIdx.x; i < len; i += 256)
    sv[i] = i < m ? codes[(int64_t)i * ldc + col] : INT32_MAX;
  __syncthreads();
  bitonic_sort(sv, len, threadIdx.x, 256, sync);
  for (int i = threadIdx.x; i < len; i += 256) {
    int cnt = 0;
    if (i < m && (i == 0 || sv[i] != sv[i - 1])) {
      int j = i + 1;
      while (j < m && sv[j] == sv[i]) ++j;
      cnt = j - i;
    }
    cv[i] = cnt;
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const double h = entropy_from_hist(cv, len, m);
    if (threadIdx.x == 0) bits[col] = h;
  }
  if (!huff) return;
  __syncthreads();
  bitonic_sort(cv, len, threadIdx.x, 256, sync);
  int nz = 0;
  for (int b = threadIdx.x; b < len; b += 256) nz += cv[b] == 0;
  for (int o = 32; o >= 1; o >>= 1) nz += __shfl_xor(nz, o, 64);
  if ((threadIdx.x & 63) == 0) nzs[threadIdx.x >> 6] = nz;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int z = nzs[0] + nzs[1] + nzs[2] + nzs[3];
    huff[col] = huffman_merge(cv, z, len, sv);   // at most len - 1 merged nodes
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
                                 double* bits, double* mean, int64_t* huff, int32_t* cmin,
                                 int32_t* cmax, hipStream_t st) {
  if (n > 0) {
    const unsigned g = (unsigned)((n + RC - 1) / RC);
    colrange<<<g, 256, 0, st>>>(codes, (int)m, (int)n, ldc, cmin, cmax);
    colhist<<<g, 256, 0, st>>>(codes, (int)m, (int)n, ldc, cmin, cmax, bits, huff);
    colhist_wide<<<(unsigned)n, 256, 0, st>>>(codes, (int)m, ldc, cmin, cmax, bits, huff);
  }
  if (mean) colmean<<<1, 256, 0, st>>>(bits, (int)n, mean);
  return hipGetLastError();
}

}  // namespace pwq
