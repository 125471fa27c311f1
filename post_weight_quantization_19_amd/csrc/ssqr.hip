// Overflow entries of quantized codes, for overflow-tolerant steps (SSQR).
//
// "The Geometry of LLM Quantization ...", technical summary 3 (SSQR): a few
// outlier weights are kept at full precision as sparse floating-point
// values, the others quantized at low bit width, and the scale is adjusted
// by a binary search to meet a target outlier density.  The nearest-plane
// sweep never clips (technical summary 2.3), so a stored code can fall
// outside the b-bit range [lo, hi]; those entries are the outliers.  They
// are listed as (row, column, value) sorted by row then column, value =
// float32(step * (code - zero point)), the weight the dequantizer would have
// produced.
//
// Design: codes are m x n row-major.  overflow_rows: one wave per row walks
// it in coalesced 64-column chunks and counts the overflows (exact integer
// counts).  overflow_scan: one workgroup turns the row counts into row
// offsets (exclusive prefix sums, fixed order) and the total.  overflow_write:
// one wave per row again; in each chunk a ballot of the overflowing lanes
// and a popcount of the lower lanes give every entry its position, so the
// list comes out in (row, column) order without sorting.
#include "pwq_device.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

__device__ __forceinline__ bool outside(int32_t c, int lo, int hi) { return c < lo || c > hi; }

__global__ __launch_bounds__(256) void overflow_rows(const int32_t* __restrict__ codes, int m,
                                                     int n, int64_t ldc, int lo, int hi,
                                                     int32_t* __restrict__ row_count) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= m) return;
  const int32_t* row = codes + (int64_t)r * ldc;
  int cnt = 0;
  for (int c = lane; c < n; c += 64) cnt += outside(row[c], lo, hi);
  for (int o = 32; o >= 1; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane == 0) row_count[r] = cnt;
}

// row_off[r] = sum of row_count[0 .. r-1]; *total = sum of all.  One
// workgroup, 256 rows per pass, a fixed-order scan inside the pass.
__global__ __launch_bounds__(256) void overflow_scan(const int32_t* __restrict__ row_count, int m,
                                                     int64_t* __restrict__ row_off,
                                                     int64_t* __restrict__ total) {
  __shared__ int64_t s[256];
  int64_t carry = 0;
  for (int base = 0; base < m; base += 256) {
    const int r = base + (int)threadIdx.x;
    const int64_t v = r < m ? row_count[r] : 0;
    s[threadIdx.x] = v;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {       // inclusive Hillis-Steele scan
      const int64_t add = threadIdx.x >= (unsigned)o ? s[threadIdx.x - o] : 0;
      __syncthreads();
      s[threadIdx.x] += add;
      __syncthreads();
    }
    if (r < m) row_off[r] = carry + s[threadIdx.x] - v;
    carry += s[255];
    __syncthreads();
  }
  if (threadIdx.x == 0) *total = carry;
}

__global__ __launch_bounds__(256) void overflow_write(
    const int32_t* __restrict__ codes, int m, int n, int64_t ldc, int lo, int hi,
    const float* __restrict__ scales, const int32_t* __restrict__ zeros, int ng, int G,
    const int64_t* __restrict__ row_off, int64_t max_out, int32_t* __restrict__ out_rows,
    int32_t* __restrict__ out_cols, float* __restrict__ out_vals) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= m) return;
  const int32_t* row = codes + (int64_t)r * ldc;
  int64_t pos = row_off[r];
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < n && pos < max_out; c0 += 64) {
    const int c = c0 + lane;
    const int32_t code = c < n ? row[c] : lo;
    const bool out = c < n && outside(code, lo, hi);
    const uint64_t mask = __ballot(out);
    const int64_t p = pos + __popcll(mask & below);
    if (out && p < max_out) {
      const int g = c / G;
      const float s = scales[(int64_t)r * ng + g];
      const int32_t z = code - (zeros ? zeros[(int64_t)r * ng + g] : 0);
      out_rows[p] = r;
      out_cols[p] = c;
      out_vals[p] = s * (float)z;
    }
    pos += __popcll(mask);
  }
}

}  // namespace

void code_range(int kind, int bits, int* lo, int* hi) {
  if (kind == PWQ_GRID_SYM) {
    *lo = -(1 << (bits - 1));
    *hi = (1 << (bits - 1)) - 1;
  } else {
    *lo = 0;
    *hi = (int)((1ll << bits) - 1);
  }
}

hipError_t launch_overflow_count(const int32_t* codes, int64_t m, int64_t n, int64_t ldc,
                                 int kind, int bits, int32_t* row_count, int64_t* row_off,
                                 int64_t* total, hipStream_t st) {
  int lo, hi;
  code_range(kind, bits, &lo, &hi);
  if (m > 0)
    overflow_rows<<<(unsigned)((m + 3) / 4), 256, 0, st>>>(codes, (int)m, (int)n, ldc, lo, hi,
                                                           row_count);
  overflow_scan<<<1, 256, 0, st>>>(row_count, (int)m, row_off, total);
  return hipGetLastError();
}

hipError_t launch_overflow_write(const int32_t* codes, int64_t m, int64_t n, int64_t ldc,
                                 int kind, int bits, const float* scales, const int32_t* zeros,
                                 int G, const int64_t* row_off, int64_t max_out,
                                 int32_t* rows, int32_t* cols, float* vals, hipStream_t st) {
  int lo, hi;
  code_range(kind, bits, &lo, &hi);
  if (m > 0 && max_out > 0)
    overflow_write<<<(unsigned)((m + 3) / 4), 256, 0, st>>>(
        codes, (int)m, (int)n, ldc, lo, hi, scales, zeros, (int)(n / G), G, row_off, max_out,
        rows, cols, vals);
  return hipGetLastError();
}

}  // namespace pwq
