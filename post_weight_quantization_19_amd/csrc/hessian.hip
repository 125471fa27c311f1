// H (+)= 2 X X^T for calibration activations X [n, ntok] (tokens contiguous).
//
// "The Geometry of LLM Quantization: GPTQ as Babai's Nearest Plane
// Algorithm", technical summary 2.1: the closest-vector lattice is generated
// by the calibration inputs, its Gram matrix is the layer Hessian;
// "WaterSIC: ...", technical summary 1: the objective is the output error
// of Y = W X, whose Hessian for X = channels x tokens is 2 X X^T.
//
// Design (gfx950): the product is a symmetric rank-N update, so only the
// lower-triangular 128x128 output tiles are computed.  Both operands are
// rows of X with the token axis contiguous, which is exactly the K-major
// operand layout of the MFMA units, so X is streamed from HBM with 16-byte
// coalesced loads into double-buffered LDS tiles and fed to
// v_mfma_f32_32x32x16_bf16 (bf16 inputs; the products are exact in fp32) or
// v_mfma_f32_32x32x2f32 (fp32 inputs).  Long token axes are split (split-K)
// to fill the 256 CUs; partial tiles are summed in a fixed order by a second
// kernel (no float atomics, so results are bitwise reproducible), which also
// applies the factor 2, the optional accumulation into the previous H and
// the mirror into the upper triangle.
#include "pwq_device.h"
#include "pwq_internal.h"

namespace pwq {

namespace {

constexpr int BM = 128;        // output tile edge
constexpr int NT = 256;        // threads per workgroup (4 waves, 2x2 of 64x64)

template <typename XT> struct SyrkCfg;
template <> struct SyrkCfg<uint16_t> {
  static constexpr int BK = 64;     // tokens per LDS stage
  static constexpr int PAD = 8;     // elements of row padding in LDS
  static constexpr int VEC = 8;     // elements per 16-byte load
};
template <> struct SyrkCfg<float> {
  static constexpr int BK = 32;
  static constexpr int PAD = 4;
  static constexpr int VEC = 4;
};

__device__ __forceinline__ void tile_coords(int t, int& ti, int& tj) {
  // t enumerates the lower-triangular tiles row by row: (0,0),(1,0),(1,1),...
  int r = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  while (r * (r + 1) / 2 > t) --r;
  ti = r;
  tj = t - r * (r + 1) / 2;
}

// One 16-byte vector of X (or fewer elements at a ragged token tail).
template <typename XT>
__device__ __forceinline__ uint4 load_vec(const XT* X, int64_t ldx, int row,
                                          int n, int64_t k, int64_t kend,
                                          bool aligned) {
  constexpr int VEC = SyrkCfg<XT>::VEC;
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row >= n || k >= kend) return v;
  const XT* p = X + (int64_t)row * ldx + k;
  if (aligned && k + VEC <= kend) return *(const uint4*)p;
  XT tmp[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) tmp[e] = (k + e < kend) ? p[e] : (XT)0;
  __builtin_memcpy(&v, tmp, sizeof(v));
  return v;
}

template <typename XT>
__global__ __launch_bounds__(NT) void syrk_tiles(
    const XT* __restrict__ X, int n, int64_t ntok, int64_t ldx, int64_t kps,
    int aligned, float* __restrict__ partial, float* __restrict__ H,
    int direct, int accumulate) {
  constexpr int BK = SyrkCfg<XT>::BK, PAD = SyrkCfg<XT>::PAD,
                VEC = SyrkCfg<XT>::VEC, LD = BK + PAD;
  constexpr int VPR = BK / VEC;                 // vectors per tile row
  constexpr int NV = BM * VPR / NT;             // vectors per thread per panel
  __shared__ __attribute__((aligned(16))) XT As[2][BM * LD];
  __shared__ __attribute__((aligned(16))) XT Bs[2][BM * LD];

  const int tile = blockIdx.x, split = blockIdx.y;
  int ti, tj;
  tile_coords(tile, ti, tj);
  const bool diag = ti == tj;
  const int r0 = ti * BM, c0 = tj * BM;
  const int64_t kbeg = (int64_t)split * kps;
  const int64_t kend = min(ntok, kbeg + kps);
  const int nstage = (int)((kend - kbeg + BK - 1) / BK);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  uint4 ra[NV], rb[NV];
  auto gload = [&](int stage) {
    const int64_t k0 = kbeg + (int64_t)stage * BK;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + NT * i, row = v / VPR, cv = v % VPR;
      ra[i] = load_vec<XT>(X, ldx, r0 + row, n, k0 + cv * VEC, kend, aligned);
      if (!diag) rb[i] = load_vec<XT>(X, ldx, c0 + row, n, k0 + cv * VEC, kend, aligned);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + NT * i, row = v / VPR, cv = v % VPR;
      *(uint4*)&As[buf][row * LD + cv * VEC] = ra[i];
      if (!diag) *(uint4*)&Bs[buf][row * LD + cv * VEC] = rb[i];
    }
  };

  if (nstage > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int s = 0; s < nstage; ++s) {
    const int buf = s & 1;
    if (s + 1 < nstage) gload(s + 1);
    const XT* A = As[buf];
    const XT* B = diag ? As[buf] : Bs[buf];
    if constexpr (sizeof(XT) == 2) {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 16) {
        const int ko = ks + 8 * (lane >> 5);
        bf16x8_t a0 = *(const bf16x8_t*)&A[(wm * 64 + (lane & 31)) * LD + ko];
        bf16x8_t a1 = *(const bf16x8_t*)&A[(wm * 64 + 32 + (lane & 31)) * LD + ko];
        bf16x8_t b0 = *(const bf16x8_t*)&B[(wn * 64 + (lane & 31)) * LD + ko];
        bf16x8_t b1 = *(const bf16x8_t*)&B[(wn * 64 + 32 + (lane & 31)) * LD + ko];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < BK; ks += 2) {
        const int ko = ks + (lane >> 5);
        float a0 = A[(wm * 64 + (lane & 31)) * LD + ko];
        float a1 = A[(wm * 64 + 32 + (lane & 31)) * LD + ko];
        float b0 = B[(wn * 64 + (lane & 31)) * LD + ko];
        float b1 = B[(wn * 64 + 32 + (lane & 31)) * LD + ko];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
      }
    }
    __syncthreads();
    if (s + 1 < nstage) lstore(buf ^ 1);
    __syncthreads();
  }

  if (!direct) {
    float* P = partial + ((int64_t)split * gridDim.x + tile) * (BM * BM);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = wn * 64 + j * 32 + (lane & 31);
          P[row * BM + col] = acc[i][j][r];
        }
    return;
  }
  // Single split: finish here (x2, accumulate, lower + mirrored upper).
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gr = r0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int gc = c0 + wn * 64 + j * 32 + (lane & 31);
        if (gr < n && gc <= gr) {
          float v = 2.0f * acc[i][j][r];
          if (accumulate) v += H[(int64_t)gr * n + gc];
          H[(int64_t)gr * n + gc] = v;
          if (gc != gr) H[(int64_t)gc * n + gr] = v;
        }
      }
}

// Sum split partials in split order, x2, (+H), write lower and mirror.
// One workgroup per 64x64 quarter of an output tile.
__global__ __launch_bounds__(256) void syrk_reduce(
    const float* __restrict__ partial, int ntiles, int nsplit, int n,
    float* __restrict__ H, int accumulate) {
  __shared__ float T[64][65];
  const int tile = blockIdx.x >> 2, quarter = blockIdx.x & 3;
  int ti, tj;
  tile_coords(tile, ti, tj);
  const int qr = (quarter >> 1) * 64, qc = (quarter & 1) * 64;
  const int r0 = ti * BM + qr, c0 = tj * BM + qc;
  if (ti == tj && qr < qc) return;  // strictly-upper quarter of a diagonal tile
  const int tid = threadIdx.x;
  for (int e = tid; e < 64 * 64; e += 256) {
    const int lr = e >> 6, lc = e & 63;
    const int64_t off = (int64_t)(qr + lr) * BM + qc + lc;
    float s = 0.0f;
#pragma unroll 8
    for (int sp = 0; sp < nsplit; ++sp) s += partial[((int64_t)sp * ntiles + tile) * (BM * BM) + off];
    const int gr = r0 + lr, gc = c0 + lc;
    float v = 2.0f * s;
    if (gr < n && gc < n && gc <= gr) {
      if (accumulate) v += H[(int64_t)gr * n + gc];
      H[(int64_t)gr * n + gc] = v;
    }
    T[lr][lc] = v;
  }
  __syncthreads();
  // mirrored writes, coalesced along the destination row
  for (int e = tid; e < 64 * 64; e += 256) {
    const int lr = e >> 6, lc = e & 63;   // destination row gc0+lr, col gr0+lc
    const int gr = r0 + lc, gc = c0 + lr; // source lower element (gr, gc)
    if (gr < n && gc < n && gc < gr) H[(int64_t)gc * n + gr] = T[lc][lr];
  }
}

}  // namespace

void syrk_plan(int64_t n, int64_t ntok, int32_t xdtype, SyrkPlan* p) {
  const int bk = xdtype == 1 ? SyrkCfg<uint16_t>::BK : SyrkCfg<float>::BK;
  const int64_t nt = (n + BM - 1) / BM;
  p->ntiles = nt * (nt + 1) / 2;
  const int64_t stages = (ntok + bk - 1) / bk;
  int64_t want = (2048 + p->ntiles - 1) / p->ntiles;    // ~8 workgroups per CU
  int64_t maxs = stages / 8 > 0 ? stages / 8 : 1;       // >= 8 stages per split
  int64_t ns = want < maxs ? want : maxs;
  if (ns < 1) ns = 1;
  if (ns > 64) ns = 64;
  int64_t kps = ((stages + ns - 1) / ns) * bk;
  if (kps < bk) kps = bk;           // ntok == 0: one empty split
  ns = (ntok + kps - 1) / kps;
  if (ns < 1) ns = 1;
  p->nsplit = ns;
  p->kps = kps;
  p->partial_bytes = ns > 1 ? (size_t)ns * p->ntiles * BM * BM * sizeof(float) : 0;
}

hipError_t launch_hessian(float* H, int64_t n, const void* X, int32_t xdtype,
                          int64_t ntok, int64_t ldx, int32_t accumulate,
                          const SyrkPlan& p, void* partial, hipStream_t st) {
  const bool aligned =
      ((uintptr_t)X % 16 == 0) && ((ldx * (xdtype == 1 ? 2 : 4)) % 16 == 0);
  const int direct = p.nsplit == 1;
  dim3 grid((unsigned)p.ntiles, (unsigned)p.nsplit);
  if (xdtype == 1)
    syrk_tiles<uint16_t><<<grid, NT, 0, st>>>((const uint16_t*)X, (int)n, ntok, ldx,
                                              p.kps, aligned, (float*)partial, H,
                                              direct, accumulate);
  else
    syrk_tiles<float><<<grid, NT, 0, st>>>((const float*)X, (int)n, ntok, ldx, p.kps,
                                           aligned, (float*)partial, H, direct,
                                           accumulate);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || direct) return e;
  syrk_reduce<<<(unsigned)(p.ntiles * 4), 256, 0, st>>>((const float*)partial,
                                                        (int)p.ntiles, (int)p.nsplit,
                                                        (int)n, H, accumulate);
  return hipGetLastError();
}

}  // namespace pwq
