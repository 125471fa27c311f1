// Min-pivot processing order: a diagonally pivoted LDL^T of the damped
// Hessian that takes, at every step, the open column whose Schur-complement
// diagonal is smallest.
//
// "The Geometry of LLM Quantization: GPTQ as Babai's Nearest Plane
// Algorithm", technical summary 2.3: the Theorem 5 bound is (1/4) s^T D s
// with D the LDL pivots of the permuted Hessian, so it depends on the pivot
// order; choosing the smallest diagonal entry at each LDL step lowers
// trace D.  Ties go to the lower original index; a NaN diagonal counts as
// smaller than any number (and then fails as not positive).  Step k fills
// position k, so the first pivot is processed last by the back-to-front
// sweep.
//
// Design (fp64 throughout; only the permutation leaves this file, the
// factor of the permuted matrix is then taken by the blocked Cholesky):
//   A    n x n, original index order, lower triangle (i > l) = the Schur
//        complement at the start of the current panel;
//   d    n    current Schur diagonal, updated at every step (d_i -= L_ik^2);
//   P    n x 32: row i holds L_ik for the steps k of the current panel;
//   rem  the columns still open at the start of the panel, in increasing
//        index order (so position order and index order agree);
//   pos  the position of a chosen column, -1 while open.
// One launch per step: every workgroup reduces the previous launch's
// per-workgroup minima to the pivot q (the same, deterministic result in
// every workgroup), then each thread computes L_iq for one open row,
//   L_iq = (A_iq - sum_{p in panel, p < k} L_ip L_qp) / sqrt(d_q),
// subtracts its square from d_i and takes part in this launch's minima.
// After 32 steps the open list is compacted and the lower triangle of the
// open block takes the panel's rank-32 update in 64 x 64 tiles.
#include "pwq_device.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

constexpr int kNB = kMinPivotPanel;  // steps per panel
constexpr int kTile = 64;  // trailing-update tile edge

__device__ __forceinline__ bool better(double v, int i, double bv, int bi) {
  return v < bv || (v == bv && i < bi);
}

__device__ __forceinline__ double order_key(double v) { return v != v ? -INFINITY : v; }

// Block-wide argmin of (v, i) pairs; every thread of the block gets the
// result.  256 threads.
__device__ void block_argmin(double& v, int& i, double* sv, int* si) {
  for (int o = 32; o >= 1; o >>= 1) {
    const double ov = __shfl_xor(v, o, 64);
    const int oi = __shfl_xor(i, o, 64);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sv[w] = v;
    si[w] = i;
  }
  __syncthreads();
  v = sv[0];
  i = si[0];
  for (int t = 1; t < 4; ++t)
    if (better(sv[t], si[t], v, i)) {
      v = sv[t];
      i = si[t];
    }
}

// A[i][l] = H[i][l] for l < i (the lower triangle of H is read).
__global__ __launch_bounds__(256) void mp_copy(const float* __restrict__ H, int n,
                                               double* __restrict__ A,
                                               const DevFlags* flags) {
  if (flags->info != 0) return;
  const int i = blockIdx.y;
  const int l = blockIdx.x * 256 + threadIdx.x;
  if (l < i) A[(int64_t)i * n + l] = (double)H[(int64_t)i * n + l];
}

// d_i = (H_ii, or 1 for an erased input) + lambda; every column open; the
// block minima of d for the first step.
__global__ __launch_bounds__(256) void mp_seed(const float* __restrict__ H, int n,
                                               const double* __restrict__ lam_p,
                                               double* __restrict__ d, int32_t* __restrict__ pos,
                                               int32_t* __restrict__ rem,
                                               double* __restrict__ part_v,
                                               int32_t* __restrict__ part_i,
                                               const DevFlags* flags) {
  __shared__ double sv[4];
  __shared__ int si[4];
  if (flags->info != 0) return;
  const int i = blockIdx.x * 256 + threadIdx.x;
  double v = INFINITY;
  int vi = INT32_MAX;
  if (i < n) {
    const float h = H[(int64_t)i * n + i];
    const double di = (h == 0.0f ? 1.0 : (double)h) + *lam_p;
    d[i] = di;
    pos[i] = -1;
    rem[i] = i;
    v = order_key(di);
    vi = i;
  }
  block_argmin(v, vi, sv, si);
  if (threadIdx.x == 0) {
    part_v[blockIdx.x] = v;
    part_i[blockIdx.x] = vi;
  }
}

// Step k (= panel start + j): choose the pivot, compute its column.
__global__ __launch_bounds__(256) void mp_step(
    const double* __restrict__ A, int n, double* __restrict__ P, double* __restrict__ d,
    int32_t* __restrict__ pos, const int32_t* __restrict__ rem, int nrem, int j, int k,
    const double* __restrict__ in_v, const int32_t* __restrict__ in_i, int nin,
    double* __restrict__ out_v, int32_t* __restrict__ out_i, int32_t* __restrict__ perm,
    double* __restrict__ piv, DevFlags* flags, pwq_result* res) {
  __shared__ double sv[4];
  __shared__ int si[4];
  __shared__ double pq[kNB];
  if (flags->info != 0) return;
  double bv = INFINITY;
  int bi = INT32_MAX;
  for (int t = threadIdx.x; t < nin; t += 256) {
    const double v = in_v[t];
    const int vi = in_i[t];
    if (better(v, vi, bv, bi)) {
      bv = v;
      bi = vi;
    }
  }
  block_argmin(bv, bi, sv, si);
  const int q = bi;
  const double dq = bv;
  if (!(dq > 0.0) || q < 0 || q >= n) {
    // not positive definite: the leading minor of order k + 1 of the
    // permuted matrix (every workgroup of this launch takes this branch)
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      flags->info = k + 1;
      res->info = k + 1;
    }
    return;
  }
  const double lq = sqrt(dq);
  if (threadIdx.x < j) pq[threadIdx.x] = P[(int64_t)q * kNB + threadIdx.x];
  __syncthreads();
  const int a = blockIdx.x * 256 + threadIdx.x;
  double mv = INFINITY;
  int mi = INT32_MAX;
  if (a < nrem) {
    const int i = rem[a];
    if (i == q) {
      P[(int64_t)q * kNB + j] = lq;
      pos[q] = k;
      perm[k] = q;
      if (piv) piv[k] = dq;
    } else if (pos[i] < 0) {
      double s = i > q ? A[(int64_t)i * n + q] : A[(int64_t)q * n + i];
      double* Pi = P + (int64_t)i * kNB;
      for (int p = 0; p < j; ++p) s -= Pi[p] * pq[p];
      const double l = s / lq;
      Pi[j] = l;
      const double di = d[i] - l * l;
      d[i] = di;
      mv = order_key(di);
      mi = i;
    }
  }
  block_argmin(mv, mi, sv, si);
  if (threadIdx.x == 0) {
    out_v[blockIdx.x] = mv;
    out_i[blockIdx.x] = mi;
  }
}

// Drop the panel's pivots from the open list, keeping increasing order.
// One workgroup; each chunk is read whole before any of it is rewritten,
// and the write cursor never passes the chunk's end.
__global__ __launch_bounds__(256) void mp_compact(int32_t* __restrict__ rem, int nrem,
                                                  const int32_t* __restrict__ pos,
                                                  const DevFlags* flags) {
  __shared__ int wcount[4];
  if (flags->info != 0) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  int out = 0;
  for (int base = 0; base < nrem; base += 256) {
    const int a = base + (int)threadIdx.x;
    const int v = a < nrem ? rem[a] : -1;
    const bool keep = a < nrem && pos[v] < 0;
    const uint64_t mask = __ballot(keep);
    if (lane == 0) wcount[w] = __popcll(mask);
    __syncthreads();
    int off = out;
    for (int t = 0; t < w; ++t) off += wcount[t];
    const int total = wcount[0] + wcount[1] + wcount[2] + wcount[3];
    if (keep) rem[off + __popcll(mask & below)] = v;
    out += total;
    __syncthreads();
  }
}

// A[i][l] -= sum_{p < nb} P[i][p] P[l][p] for open i > l, in 64 x 64 tiles
// of open positions (lower-triangle tiles only).
__global__ __launch_bounds__(256) void mp_trailing(double* __restrict__ A, int n,
                                                   const double* __restrict__ P,
                                                   const int32_t* __restrict__ rem, int nr,
                                                   int nb, const DevFlags* flags) {
  __shared__ double pa[kTile][kNB + 1];
  __shared__ double pb[kTile][kNB + 1];
  __shared__ int ia[kTile], ib[kTile];
  if (flags->info != 0) return;
  const int x = blockIdx.x;
  int ta = (int)((sqrt(8.0 * x + 1.0) - 1.0) * 0.5);
  while (ta * (ta + 1) / 2 > x) --ta;
  while ((ta + 1) * (ta + 2) / 2 <= x) ++ta;
  const int tb = x - ta * (ta + 1) / 2;
  const int a0 = ta * kTile, b0 = tb * kTile;
  if (threadIdx.x < kTile) {
    const int a = a0 + (int)threadIdx.x, b = b0 + (int)threadIdx.x;
    ia[threadIdx.x] = a < nr ? rem[a] : -1;
    ib[threadIdx.x] = b < nr ? rem[b] : -1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kTile * kNB; e += 256) {
    const int r = e / kNB, p = e % kNB;
    const int i = ia[r], l = ib[r];
    pa[r][p] = (i >= 0 && p < nb) ? P[(int64_t)i * kNB + p] : 0.0;
    pb[r][p] = (l >= 0 && p < nb) ? P[(int64_t)l * kNB + p] : 0.0;
  }
  __syncthreads();
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  double acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
  for (int p = 0; p < nb; ++p) {
    double av[4], bv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) av[r] = pa[ty + 16 * r][p];
#pragma unroll
    for (int c = 0; c < 4; ++c) bv[c] = pb[tx + 16 * c][p];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] += av[r] * bv[c];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int ra = ty + 16 * r;
    const int i = ia[ra];
    if (i < 0) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int cb = tx + 16 * c;
      const int l = ib[cb];
      if (l >= 0 && (ta > tb || ra > cb)) A[(int64_t)i * n + l] -= acc[r][c];
    }
  }
}

}  // namespace

hipError_t launch_min_pivot(const float* H, int64_t n64, const double* lam, const MinPivotWs& w,
                            int32_t* perm, double* piv, DevFlags* flags, pwq_result* res,
                            hipStream_t st) {
  const int n = (int)n64;
  if (n <= 0) return hipSuccess;
  const int g = (n + 255) / 256;
  mp_copy<<<dim3((unsigned)g, (unsigned)n), 256, 0, st>>>(H, n, w.A, flags);
  mp_seed<<<g, 256, 0, st>>>(H, n, lam, w.d, w.pos, w.rem, w.part_v, w.part_i, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int nin = g;
  for (int k0 = 0; k0 < n; k0 += kNB) {
    const int nb = n - k0 < kNB ? n - k0 : kNB;
    const int nrem = n - k0;
    const int gs = (nrem + 255) / 256;
    for (int j = 0; j < nb; ++j) {
      const int k = k0 + j;
      const int64_t src = (int64_t)(k & 1) * g, dst = (int64_t)((k + 1) & 1) * g;
      mp_step<<<gs, 256, 0, st>>>(w.A, n, w.P, w.d, w.pos, w.rem, nrem, j, k, w.part_v + src,
                                  w.part_i + src, nin, w.part_v + dst, w.part_i + dst, perm,
                                  piv, flags, res);
      nin = gs;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (k0 + nb < n) {
      const int nr = nrem - nb;
      const int T = (nr + kTile - 1) / kTile;
      mp_compact<<<1, 256, 0, st>>>(w.rem, nrem, w.pos, flags);
      mp_trailing<<<(unsigned)((int64_t)T * (T + 1) / 2), 256, 0, st>>>(w.A, n, w.P, w.rem, nr,
                                                                         nb, flags);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace pwq
