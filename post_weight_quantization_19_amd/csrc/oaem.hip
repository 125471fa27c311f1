// OA-EM: output-aware EM initialisation of additive codebooks.
//
// "Initialisation Determines the Basin: Efficient Codebook Optimisation for
// Extreme LLM Quantization", section 3: inside AQLM's residual framework,
// each codebook is initialised by EM.  The M-step moves each centroid to
// minimise the output reconstruction error of its weight groups, weighted
// by H_i = X_i^T X_i + lambda I; the E-step reassigns every group to the
// nearest centroid in that Mahalanobis distance.
//
// Reading: a group is g consecutive inputs of one output row; H_i is the
// g x g diagonal block of the damped Hessian (dead inputs and lambda as for
// the layer); a stage's centroids start at the residual groups the caller
// names; a stage runs `iters` E/M rounds and a final E-step, then the
// residual loses the chosen centroids.  Ties go to the lower centroid; a
// centroid without groups keeps its value.  Everything is float64.
//
// Kernels, per stage and round:
//   oaem_qtable  Q[i][k] = c_k^T H_i c_k                     (ng x K)
//   oaem_estep   one thread per row (four for groups of 8) of a group
//                column: h = H_i w, then argmin_k Q[i][k] - 2 h . c_k with
//                the codebook in LDS (the same argmin as the distance,
//                which differs from it by w^T H_i w)
//   oaem_msums   per (group column, centroid): the sum of the assigned
//                residual groups and their count, four quarter sums (rows
//                in increasing order within each) added in a fixed order
//                (chunks of assignments and rows staged in LDS)
//   oaem_msolve  one workgroup per centroid: A = sum_i cnt_ik H_i,
//                b = sum_i H_i S_ik over fixed slices of i added in order,
//                then A c = b by Cholesky (g <= 16)
//   oaem_apply / oaem_objective after the final E-step.
#include "pwq_device.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

constexpr int kMaxG = kOaemMaxG;

__global__ __launch_bounds__(256) void oaem_blocks(const float* __restrict__ H, int n, int g,
                                                   const double* __restrict__ lam_p,
                                                   double* __restrict__ Hb) {
  const int i = blockIdx.x;
  const int t = threadIdx.x;
  if (t >= g * g) return;
  const int u = t / g, v = t % g;
  const int a = i * g + (u > v ? u : v), b = i * g + (u > v ? v : u);
  const float h = H[(int64_t)a * n + b];
  double x = (double)h;
  if (u == v) x = (h == 0.0f ? 1.0 : (double)h) + *lam_p;
  Hb[(int64_t)i * g * g + t] = x;
}

__global__ __launch_bounds__(256) void oaem_load(const void* __restrict__ W, int wdtype,
                                                 int n, int64_t ldw, double* __restrict__ R) {
  const int r = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  double v;
  if (wdtype == PWQ_BF16) {
    const uint16_t b = ((const uint16_t*)W)[(int64_t)r * ldw + c];
    v = (double)__uint_as_float((uint32_t)b << 16);
  } else {
    v = (double)((const float*)W)[(int64_t)r * ldw + c];
  }
  R[(int64_t)r * n + c] = v;
}

__global__ __launch_bounds__(256) void oaem_seed(const double* __restrict__ R, int m, int n,
                                                 int g, const int64_t* __restrict__ seeds,
                                                 int K, double* __restrict__ C,
                                                 pwq_result* res) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  const int ng = n / g;
  int64_t s = seeds[k];
  if (s < 0 || s >= (int64_t)m * ng) {
    res->info = -1;
    s = 0;
  }
  const int r = (int)(s / ng), i = (int)(s % ng);
  for (int e = 0; e < g; ++e) C[(int64_t)k * g + e] = R[(int64_t)r * n + i * g + e];
}

__global__ __launch_bounds__(256) void oaem_qtable(const double* __restrict__ Hb,
                                                   const double* __restrict__ C, int K, int g,
                                                   double* __restrict__ Q) {
  __shared__ double h[kMaxG * kMaxG];
  const int i = blockIdx.x;
  for (int t = threadIdx.x; t < g * g; t += 256) h[t] = Hb[(int64_t)i * g * g + t];
  __syncthreads();
  for (int k = blockIdx.y * 256 + threadIdx.x; k < K; k += 256 * gridDim.y) {
    double c[kMaxG];
    for (int e = 0; e < g; ++e) c[e] = C[(int64_t)k * g + e];
    double q = 0.0;
    for (int u = 0; u < g; ++u) {
      double hu = 0.0;
      for (int v = 0; v < g; ++v) hu += h[u * g + v] * c[v];
      q += c[u] * hu;
    }
    Q[(int64_t)i * K + k] = q;
  }
}

// grid (ng, ceil(m / (256 RPT))); dynamic LDS: K g + K doubles.  GS is the
// group size when known at compile time (0: the runtime g); each thread
// takes RPT rows, so each centroid read from LDS serves RPT rows.
template <int GS, int RPT>
__global__ __launch_bounds__(256) void oaem_estep(const double* __restrict__ R, int m, int n,
                                                  int g_rt, const double* __restrict__ Hb,
                                                  const double* __restrict__ C,
                                                  const double* __restrict__ Q, int K,
                                                  int32_t* __restrict__ a) {
  constexpr int GM = GS > 0 ? GS : kMaxG;
  const int g = GS > 0 ? GS : g_rt;
  extern __shared__ double lds[];
  __shared__ double h[kMaxG * kMaxG];
  double* cs = lds;             // K x g
  double* qs = lds + K * g;     // K
  const int i = blockIdx.x, ng = n / g;
  for (int t = threadIdx.x; t < K * g; t += 256) cs[t] = C[t];
  for (int t = threadIdx.x; t < K; t += 256) qs[t] = Q[(int64_t)i * K + t];
  for (int t = threadIdx.x; t < g * g; t += 256) h[t] = Hb[(int64_t)i * g * g + t];
  __syncthreads();
  const int r0 = blockIdx.y * 256 * RPT + threadIdx.x;
  if (r0 >= m) return;
  double hw[RPT][GM];
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    const int r = r0 + q * 256 < m ? r0 + q * 256 : r0;   // a clamped row is computed twice
    double w[GM];
#pragma unroll
    for (int e = 0; e < GM; ++e) {
      const double x = R[(int64_t)r * n + i * g + (e < g ? e : 0)];   // index kept in the row
      w[e] = e < g ? x : 0.0;
    }
#pragma unroll
    for (int u = 0; u < GM; ++u) {
      double acc = 0.0;
#pragma unroll
      for (int v = 0; v < GM; ++v)
        if (u < g && v < g) acc += h[u * g + v] * w[v];
      hw[q][u] = 2.0 * acc;
    }
  }
  double best[RPT];
  int bk[RPT];
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    best[q] = INFINITY;
    bk[q] = 0;
  }
  for (int k = 0; k < K; ++k) {
    const double* ck = cs + k * g;
    double c[GM];
#pragma unroll
    for (int e = 0; e < GM; ++e) {
      const double x = ck[e < g ? e : 0];
      c[e] = e < g ? x : 0.0;
    }
    const double qk = qs[k];
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
      double dot = 0.0;
#pragma unroll
      for (int e = 0; e < GM; ++e)
        if (e < g) dot += hw[q][e] * c[e];
      const double sc = qk - dot;
      if (sc < best[q]) {
        best[q] = sc;
        bk[q] = k;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    const int r = r0 + q * 256;
    if (r < m) a[(int64_t)r * ng + i] = bk[q];
  }
}

// grid (ng, ceil(K / 256)), 1024 threads: the groups of column i assigned
// to centroid k are summed by four threads, quarter q of every chunk of
// 1024 rows each (rows in increasing order within a quarter), and the four
// partial sums are added in quarter order.  GS as for the E-step (loops
// over the group unrolled to a compile-time bound so that the sums stay in
// registers).
template <int GS>
__global__ __launch_bounds__(1024) void oaem_msums(const double* __restrict__ R, int m, int n,
                                                   int g_rt, const int32_t* __restrict__ a,
                                                   int K, double* __restrict__ S,
                                                   int32_t* __restrict__ cnt) {
  constexpr int GM = GS > 0 ? GS : kMaxG;
  constexpr int CH = 1024;
  const int g = GS > 0 ? GS : g_rt;
  __shared__ int32_t ac[CH];
  __shared__ double rc[CH * GM];          // row groups; afterwards the quarter partials
  __shared__ int32_t pc[CH];
  const int ng = n / g;
  // workgroup b runs on XCD b % 8: give each XCD a contiguous range of
  // columns, so the lines of assignments (32 columns each) and of R (two
  // columns of 8) are shared in that XCD's L2
  const int per = (ng + 7) / 8;
  const int i = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (i >= ng) return;
  const int lane_k = threadIdx.x & 255, qtr = threadIdx.x >> 8;
  const int k = blockIdx.y * 256 + lane_k;
  double s[GM];
#pragma unroll
  for (int e = 0; e < GM; ++e) s[e] = 0.0;
  int c = 0;
  for (int r0 = 0; r0 < m; r0 += CH) {
    const int rr = r0 + threadIdx.x;
    ac[threadIdx.x] = rr < m ? a[(int64_t)rr * ng + i] : -1;
#pragma unroll
    for (int e = 0; e < GM; ++e) {
      const double x = rr < m && e < g ? R[(int64_t)rr * n + i * g + e] : 0.0;
      rc[threadIdx.x * GM + e] = x;
    }
    __syncthreads();
    // rows past m hold -1 and never match; eight assignments per pass
    const int t_lo = qtr * 256;
    for (int t0 = t_lo; t0 < t_lo + 256; t0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = ac[t0 + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (v[u] == k) {
          ++c;
#pragma unroll
          for (int e = 0; e < GM; ++e) s[e] += rc[(t0 + u) * GM + e];
        }
      }
    }
    __syncthreads();
  }
  // quarter partials through LDS, added in quarter order
#pragma unroll
  for (int e = 0; e < GM; ++e) rc[(qtr * 256 + lane_k) * GM + e] = s[e];
  pc[qtr * 256 + lane_k] = c;
  __syncthreads();
  if (qtr == 0 && k < K) {
    double tot[GM];
    int ct = 0;
#pragma unroll
    for (int e = 0; e < GM; ++e) tot[e] = 0.0;
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 0; e < GM; ++e) tot[e] += rc[(q * 256 + lane_k) * GM + e];
      ct += pc[q * 256 + lane_k];
    }
    const int64_t o = (int64_t)i * K + k;
    cnt[o] = ct;
#pragma unroll
    for (int e = 0; e < GM; ++e)
      if (e < g) S[o * g + e] = tot[e];
  }
}

// grid K: centroid k <- solve (sum_i cnt_ik H_i) c = sum_i H_i S_ik, or
// unchanged when no group is assigned to it.  The sums over the group
// columns i are split into fixed slices (i = s, s + nslices, ...) over all
// 256 threads, each slice with four interleaved accumulators, and
// everything is combined in a fixed order, so the result does not depend
// on timing.
__global__ __launch_bounds__(256) void oaem_msolve(const double* __restrict__ Hb, int ng, int g,
                                                   const double* __restrict__ S,
                                                   const int32_t* __restrict__ cnt, int K,
                                                   double* __restrict__ C) {
  __shared__ double part[256];
  __shared__ double A[kMaxG * kMaxG];
  __shared__ double bsh[kMaxG];
  __shared__ int64_t total;
  const int k = blockIdx.x;
  const int t = threadIdx.x;
  const int gg = g * g;
  // A: entry e = t % gg, slice t / gg
  {
    const int ns = 256 / gg;
    const int e = t % gg, sl = t / gg;
    // four interleaved accumulators (i, i + ns, i + 2 ns, i + 3 ns) keep four
    // iterations' loads in flight; they are combined in a fixed order
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    if (sl < ns) {
      int i = sl;
      for (; i + 3 * ns < ng; i += 4 * ns) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ii = i + q * ns;
          acc[q] += (double)cnt[(int64_t)ii * K + k] * Hb[(int64_t)ii * gg + e];
        }
      }
      for (; i < ng; i += ns) acc[0] += (double)cnt[(int64_t)i * K + k] * Hb[(int64_t)i * gg + e];
    }
    part[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    __syncthreads();
    if (t < gg) {
      double sum = 0.0;
      for (int q = 0; q < ns; ++q) sum += part[q * gg + t];
      A[t] = sum;
    }
    __syncthreads();
  }
  // b: entry u = t % g, slice t / g
  {
    const int ns = 256 / g;
    const int u = t % g, sl = t / g;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    if (sl < ns) {
      int i = sl;
      for (; i + 3 * ns < ng; i += 4 * ns) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ii = i + q * ns;
          const double* hr = Hb + (int64_t)ii * gg + u * g;
          const double* sv = S + ((int64_t)ii * K + k) * g;
          double d = 0.0;
          for (int v = 0; v < g; ++v) d += hr[v] * sv[v];
          acc[q] += d;
        }
      }
      for (; i < ng; i += ns) {
        const double* hr = Hb + (int64_t)i * gg + u * g;
        const double* sv = S + ((int64_t)i * K + k) * g;
        double d = 0.0;
        for (int v = 0; v < g; ++v) d += hr[v] * sv[v];
        acc[0] += d;
      }
    }
    part[t] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    if (t == 0) {
      int64_t c = 0;
      for (int i = 0; i < ng; ++i) c += cnt[(int64_t)i * K + k];
      total = c;
    }
    __syncthreads();
    if (t < g) {
      double sum = 0.0;
      for (int q = 0; q < ns; ++q) sum += part[q * g + t];
      bsh[t] = sum;
    }
    __syncthreads();
  }
  if (t != 0 || total == 0) return;
  // Cholesky A = L L^T in place (lower), then forward / back substitution
  for (int j = 0; j < g; ++j) {
    double d = A[j * g + j];
    for (int p = 0; p < j; ++p) d -= A[j * g + p] * A[j * g + p];
    if (!(d > 0.0)) return;               // keep the centroid
    const double ljj = sqrt(d);
    A[j * g + j] = ljj;
    for (int u = j + 1; u < g; ++u) {
      double x = A[u * g + j];
      for (int p = 0; p < j; ++p) x -= A[u * g + p] * A[j * g + p];
      A[u * g + j] = x / ljj;
    }
  }
  double y[kMaxG];
  for (int u = 0; u < g; ++u) {
    double x = bsh[u];
    for (int p = 0; p < u; ++p) x -= A[u * g + p] * y[p];
    y[u] = x / A[u * g + u];
  }
  for (int u = g - 1; u >= 0; --u) {
    double x = y[u];
    for (int p = u + 1; p < g; ++p) x -= A[p * g + u] * y[p];
    y[u] = x / A[u * g + u];
  }
  for (int u = 0; u < g; ++u) C[(int64_t)k * g + u] = y[u];
}

__global__ __launch_bounds__(256) void oaem_apply(double* __restrict__ R, int n, int g,
                                                  const int32_t* __restrict__ a,
                                                  const double* __restrict__ C) {
  const int r = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= n) return;
  const int ng = n / g, i = c / g, e = c % g;
  const int k = a[(int64_t)r * ng + i];
  R[(int64_t)r * n + c] -= C[(int64_t)k * g + e];
}

// Per-workgroup sums of e^T H_i e over 256 groups (index r ng + i), fixed
// tree; the last launch of a stage sums the partials in order.
template <int GS>
__global__ __launch_bounds__(256) void oaem_objective(const double* __restrict__ R, int m,
                                                      int n, int g_rt,
                                                      const double* __restrict__ Hb,
                                                      double* __restrict__ part) {
  constexpr int GM = GS > 0 ? GS : kMaxG;
  const int g = GS > 0 ? GS : g_rt;
  __shared__ double red[256];
  const int ng = n / g;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  double val = 0.0;
  if (q < (int64_t)m * ng) {
    const int r = (int)(q / ng), i = (int)(q % ng);
    double e[GM];
#pragma unroll
    for (int u = 0; u < GM; ++u) {
      const double x = R[(int64_t)r * n + i * g + (u < g ? u : 0)];
      e[u] = u < g ? x : 0.0;
    }
    const double* h = Hb + (int64_t)i * g * g;
#pragma unroll
    for (int u = 0; u < GM; ++u) {
      double s = 0.0;
#pragma unroll
      for (int v = 0; v < GM; ++v)
        if (u < g && v < g) s += h[u * g + v] * e[v];
      val += e[u] * s;
    }
  }
  red[threadIdx.x] = val;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) part[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void oaem_objective_sum(const double* __restrict__ part,
                                                          int np, double* __restrict__ out) {
  __shared__ double red[256];
  double v = 0.0;
  for (int t = threadIdx.x; t < np; t += 256) v += part[t];
  red[threadIdx.x] = v;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

}  // namespace

int64_t oaem_objective_parts(int64_t m, int64_t n, int32_t g) {
  return (m * (n / g) + 255) / 256;
}

hipError_t launch_oaem(const void* W, int32_t wdtype, int64_t m64, int64_t n64, int64_t ldw,
                       const float* H, const double* lam, int32_t g, int32_t K, int32_t M,
                       int32_t iters, const int64_t* seeds, double* books, int32_t* codes,
                       double* obj, pwq_result* res, const OaemWs& w, hipStream_t st) {
  const int m = (int)m64, n = (int)n64, ng = n / g;
  oaem_blocks<<<ng, 256, 0, st>>>(H, n, g, lam, w.Hb);
  oaem_load<<<dim3((unsigned)((n + 255) / 256), (unsigned)m), 256, 0, st>>>(W, wdtype, n, ldw,
                                                                             w.R);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned kb = (unsigned)((K + 255) / 256);
  const size_t lds = (size_t)(K * g + K) * sizeof(double);
  const int64_t nparts = oaem_objective_parts(m, n, g);
  for (int t = 0; t < M; ++t) {
    double* C = books + (int64_t)t * K * g;
    int32_t* a = codes + (int64_t)t * m * ng;
    oaem_seed<<<kb, 256, 0, st>>>(w.R, m, n, g, seeds + (int64_t)t * K, K, C, res);
    for (int it = 0; it <= iters; ++it) {
      oaem_qtable<<<dim3((unsigned)ng, kb), 256, 0, st>>>(w.Hb, C, K, g, w.Q);
      if (g == 8)
        oaem_estep<8, 4><<<dim3((unsigned)ng, (unsigned)((m + 1023) / 1024)), 256, lds, st>>>(
            w.R, m, n, g, w.Hb, C, w.Q, K, a);
      else
        oaem_estep<0, 1><<<dim3((unsigned)ng, (unsigned)((m + 255) / 256)), 256, lds, st>>>(
            w.R, m, n, g, w.Hb, C, w.Q, K, a);
      if (it < iters) {
        const unsigned gx = (unsigned)(8 * ((ng + 7) / 8));   // whole XCD ranges
        if (g == 8)
          oaem_msums<8><<<dim3(gx, kb), 1024, 0, st>>>(w.R, m, n, g, a, K, w.S, w.cnt);
        else
          oaem_msums<0><<<dim3(gx, kb), 1024, 0, st>>>(w.R, m, n, g, a, K, w.S, w.cnt);
        oaem_msolve<<<(unsigned)K, 256, 0, st>>>(w.Hb, ng, g, w.S, w.cnt, K, C);
      }
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    oaem_apply<<<dim3((unsigned)((n + 255) / 256), (unsigned)m), 256, 0, st>>>(w.R, n, g, a, C);
    if (obj) {
      if (g == 8)
        oaem_objective<8><<<(unsigned)nparts, 256, 0, st>>>(w.R, m, n, g, w.Hb, w.part);
      else
        oaem_objective<0><<<(unsigned)nparts, 256, 0, st>>>(w.R, m, n, g, w.Hb, w.part);
      oaem_objective_sum<<<1, 256, 0, st>>>(w.part, (int)nparts, obj + t);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pwq
