// H (+)= 2 X X^T for calibration activations X, stored either channel-major
// ([n, ntok], tokens contiguous) or token-major ([ntok, n], one row per
// token with the channels contiguous, as activations are usually captured).
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

__device__ __forceinline__ void tri_index(int t, int& a, int& b) {
  // t enumerates a lower triangle row by row: (0,0),(1,0),(1,1),(2,0),...
  int r = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while ((r + 1) * (r + 2) / 2 <= t) ++r;
  while (r * (r + 1) / 2 > t) --r;
  a = r;
  b = t - r * (r + 1) / 2;
}

// Tile order: lower-triangular 8x8 super-blocks of 128x128 tiles, each
// super-block's tiles consecutive.  Workgroups that run together on one XCD
// take consecutive positions, so they share at most 16 row panels of X in
// that XCD's L2.
constexpr int SUPER = 8;
__device__ __forceinline__ void tile_coords(int pos, int nt, int& ti, int& tj) {
  const int ns = (nt + SUPER - 1) / SUPER;
  int base = 0;
  for (int I = 0; I < ns; ++I) {
    const int rows = min(SUPER, nt - SUPER * I);
    for (int J = 0; J <= I; ++J) {
      const int cols = min(SUPER, nt - SUPER * J);
      const int cnt = (I == J) ? rows * (rows + 1) / 2 : rows * cols;
      if (pos < base + cnt) {
        const int local = pos - base;
        int a, b;
        if (I == J) {
          tri_index(local, a, b);
        } else {
          a = local / cols;
          b = local % cols;
        }
        ti = SUPER * I + a;
        tj = SUPER * J + b;
        return;
      }
      base += cnt;
    }
  }
  ti = tj = 0;  // not reached for pos < nt (nt + 1) / 2
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

// Token-major X: the same 16-byte vector (channel `row`, tokens k ..
// k+VEC-1) gathered element by element; consecutive lanes take consecutive
// channels, so every element load is coalesced across the wave.
template <typename XT>
__device__ __forceinline__ uint4 load_vec_tm(const XT* X, int64_t ldx, int row, int n,
                                             int64_t k, int64_t kend) {
  constexpr int VEC = SyrkCfg<XT>::VEC;
  XT tmp[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e)
    tmp[e] = (row < n && k + e < kend) ? X[(k + e) * ldx + row] : (XT)0;
  uint4 v;
  __builtin_memcpy(&v, tmp, sizeof(v));
  return v;
}

// Work item = (split, tile position), split-major.  Workgroup w runs on XCD
// w % 8 (round-robin dispatch); XCD x takes items [x Q, (x+1) Q), so with 8
// splits each XCD owns one token range of every tile.
template <typename XT, bool TM>
__global__ __launch_bounds__(NT) void syrk_tiles(
    const XT* __restrict__ X, int n, int64_t ntok, int64_t ldx, int64_t kps,
    int aligned, float* __restrict__ partial, float* __restrict__ H,
    int direct, int accumulate, int ntiles, int nsplit, int per_xcd) {
  constexpr int BK = SyrkCfg<XT>::BK, PAD = SyrkCfg<XT>::PAD,
                VEC = SyrkCfg<XT>::VEC, LD = BK + PAD;
  constexpr int VPR = BK / VEC;                 // vectors per tile row
  constexpr int NV = BM * VPR / NT;             // vectors per thread per panel
  __shared__ __attribute__((aligned(16))) XT As[2][BM * LD];
  __shared__ __attribute__((aligned(16))) XT Bs[2][BM * LD];

  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= ntiles * nsplit) return;
  const int split = item / ntiles, tile = item % ntiles;
  const int nt = (n + BM - 1) / BM;
  int ti, tj;
  tile_coords(tile, nt, ti, tj);
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
  // vector v of a panel stage: channel row, token vector cv (channel-major:
  // consecutive threads walk along the tokens of a row; token-major: along
  // the channels)
  auto vrow = [](int v) { return TM ? v % BM : v / VPR; };
  auto vcol = [](int v) { return TM ? v / BM : v % VPR; };
  auto gload = [&](int stage) {
    const int64_t k0 = kbeg + (int64_t)stage * BK;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + NT * i, row = vrow(v), cv = vcol(v);
      if constexpr (TM) {
        ra[i] = load_vec_tm<XT>(X, ldx, r0 + row, n, k0 + cv * VEC, kend);
        if (!diag) rb[i] = load_vec_tm<XT>(X, ldx, c0 + row, n, k0 + cv * VEC, kend);
      } else {
        ra[i] = load_vec<XT>(X, ldx, r0 + row, n, k0 + cv * VEC, kend, aligned);
        if (!diag) rb[i] = load_vec<XT>(X, ldx, c0 + row, n, k0 + cv * VEC, kend, aligned);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int v = tid + NT * i, row = vrow(v), cv = vcol(v);
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
    float* P = partial + ((int64_t)split * ntiles + tile) * (BM * BM);
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

// Large-tile variant for bf16 X: 256x256 output tiles computed by 8 waves,
// each 64x128 (2x4 v_mfma_f32_32x32x16_bf16 accumulators), two waves per
// SIMD so one wave's LDS waits hide behind the other's MFMAs; 32 tokens per
// stage.  Twice the arithmetic per byte moved from L2 of a 128x128 tile.
// X streams HBM -> LDS with global_load_lds_dwordx4 (no register staging)
// through a ring of 5 stages (the whole 160 KB LDS), issued 4 stages ahead,
// so about 2 us of load latency is covered.  LDS rows are 64 B (four 16-byte
// chunks) with the chunk index XOR-swizzled by bits 2..3 of the row: 16
// consecutive rows read at one logical chunk hit 16 distinct bank groups.
constexpr int BL = 256;        // large tile edge
constexpr int BKL = 32;        // tokens per stage
constexpr int NSLOT = 5;       // LDS ring slots
constexpr int AHEAD = 4;       // stages in flight ahead of the one computed
// 8 waves of 64x128 (two per SIMD) measured faster than 4 waves of 128x128:
// the second wave per SIMD hides LDS latency better than the halved LDS
// traffic of the larger wave tile saves.
constexpr int NWL = 8;         // waves per workgroup
constexpr int NTL = 64 * NWL;  // threads

__device__ __forceinline__ int swz(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

// Token-major X: an LDS panel stage is 32 token rows of 512 B (256 channels,
// 32 chunks of 16 B); logical chunk c of token row r is stored at chunk
// c ^ tm_swz(r).  The MFMA operands (8 consecutive tokens of one channel per
// lane) come from pairs of ds_read_b64_tr_b16: within each 16-lane group,
// lane i receives element i % 4 of the 8 bytes addressed by lane
// 4 j + i / 4 as its element j.  When source lane 4 j + a addresses token
// row t0 + j, channels f0 + 4a .. f0 + 4a + 3, lane i therefore receives
// tokens t0 .. t0 + 3 of channel f0 + i.  A group reads 4 consecutive token
// rows at the same channels; the swizzle moves those rows' 32-byte pieces
// to distinct banks.
#ifndef PWQ_TM_SWZ
#define PWQ_TM_SWZ 4
#endif
__device__ __forceinline__ int tm_swz(int r) { return PWQ_TM_SWZ * (r & 3); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// The twelve MFMA operands of one stage (two token steps of 16; each
// operand is 8 consecutive tokens t0 .. t0 + 7 of channel f0 + lane % 16)
// from the LDS addresses p[0..5] of the first step: two transposed reads 4
// token rows (2048 B) apart per operand, the second step 16 rows (8192 B)
// further.  All 24 reads are issued together and waited for (lgkmcnt(0))
// inside the same asm block, so every output is complete when the block
// ends.  (Written as asm because the compiler, not seeing which LDS bytes
// the builtin reads, would otherwise wait for every LDS copy still in
// flight before the first read.)
__device__ __forceinline__ void tr_operands12(const uint32_t (&p)[6], bf16x8_t (&out)[12]) {
  v4i16 lo[12], hi[12];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %24\n\t"
      "ds_read_b64_tr_b16 %1, %24 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %25\n\t"
      "ds_read_b64_tr_b16 %3, %25 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %26\n\t"
      "ds_read_b64_tr_b16 %5, %26 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %27\n\t"
      "ds_read_b64_tr_b16 %7, %27 offset:2048\n\t"
      "ds_read_b64_tr_b16 %8, %28\n\t"
      "ds_read_b64_tr_b16 %9, %28 offset:2048\n\t"
      "ds_read_b64_tr_b16 %10, %29\n\t"
      "ds_read_b64_tr_b16 %11, %29 offset:2048\n\t"
      "ds_read_b64_tr_b16 %12, %24 offset:8192\n\t"
      "ds_read_b64_tr_b16 %13, %24 offset:10240\n\t"
      "ds_read_b64_tr_b16 %14, %25 offset:8192\n\t"
      "ds_read_b64_tr_b16 %15, %25 offset:10240\n\t"
      "ds_read_b64_tr_b16 %16, %26 offset:8192\n\t"
      "ds_read_b64_tr_b16 %17, %26 offset:10240\n\t"
      "ds_read_b64_tr_b16 %18, %27 offset:8192\n\t"
      "ds_read_b64_tr_b16 %19, %27 offset:10240\n\t"
      "ds_read_b64_tr_b16 %20, %28 offset:8192\n\t"
      "ds_read_b64_tr_b16 %21, %28 offset:10240\n\t"
      "ds_read_b64_tr_b16 %22, %29 offset:8192\n\t"
      "ds_read_b64_tr_b16 %23, %29 offset:10240\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
        "=&v"(lo[3]), "=&v"(hi[3]), "=&v"(lo[4]), "=&v"(hi[4]), "=&v"(lo[5]), "=&v"(hi[5]),
        "=&v"(lo[6]), "=&v"(hi[6]), "=&v"(lo[7]), "=&v"(hi[7]), "=&v"(lo[8]), "=&v"(hi[8]),
        "=&v"(lo[9]), "=&v"(hi[9]), "=&v"(lo[10]), "=&v"(hi[10]), "=&v"(lo[11]), "=&v"(hi[11])
      : "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]), "v"(p[4]), "v"(p[5])
      : "memory");
#pragma unroll
  for (int t = 0; t < 12; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[t][e] = lo[t][e];
      out[t][4 + e] = hi[t][e];
    }
}

// s_waitcnt immediate (gfx9 encoding) waiting for vmcnt <= v and lgkmcnt = 0.
constexpr int wait_vm_lgkm0(int v) { return (v & 15) | (((v >> 4) & 3) << 14) | 0x70; }

template <bool TM>
__global__ __launch_bounds__(NTL, 1) void syrk_tiles256(
    const uint16_t* __restrict__ X, int n, int64_t ntok, int64_t ldx, int64_t kps,
    int aligned, float* __restrict__ partial, float* __restrict__ H, int direct,
    int accumulate, int ntiles, int nsplit, int per_xcd) {
  constexpr int WR = 512 / NWL;        // rows per wave (the wave grid is (NWL/2) x 2)
  constexpr int TI = WR / 32;          // 32-row accumulator blocks per wave
  constexpr int CPW = 16 / NWL;        // 1 KB DMA chunks per wave per panel and stage
  __shared__ __attribute__((aligned(16))) uint4 Ls[NSLOT][2][BL * 4];
  const int item = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (item >= ntiles * nsplit) return;
  const int split = item / ntiles, tile = item % ntiles;
  const int nt = (n + BL - 1) / BL;
  int ti, tj;
  tile_coords(tile, nt, ti, tj);
  const bool diag = ti == tj;
  const int r0 = ti * BL, c0 = tj * BL;
  const int64_t kbeg = (int64_t)split * kps;
  const int64_t kend = min(ntok, kbeg + kps);
  const int nstage = (int)((kend - kbeg + BKL - 1) / BKL);
  const int nfull = (int)((kend - kbeg) / BKL);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;      // rows WR wm, cols 128 wn
  // waves entirely above the diagonal of a diagonal tile have nothing to do
  const bool skip = diag && (WR * wm + WR - 1 < 128 * wn);

  f32x16_t acc[TI][4];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // DMA: each stage and panel is 16 wave-chunks of 1 KB (64 lanes x 16 B);
  // wave w fills chunks CPW w .. CPW w + CPW-1, and lane l of chunk q fills
  // LDS unit u = 64 q + l.
  // Channel-major: unit u = channel row u/4, physical chunk u%4, i.e.
  // logical chunk (u%4) ^ ((row>>2)&3) of 8 tokens.  Rows past n read row
  // n-1 (those products only reach outputs >= n, which are never stored).
  // Token-major: unit u = token row u/32, physical chunk u%32, logical chunk
  // (u%32) ^ tm_swz(row) of 8 channels; channels past n read channels n-8 ..
  // n-1 (n is a multiple of 8 on this path), again only reaching outputs
  // that are never stored.
  const uint16_t* ga[CPW];
  const uint16_t* gb[CPW];
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const int u = (CPW * wave + q) * 64 + lane;
    if constexpr (TM) {
      const int t = u >> 5, c = (u & 31) ^ tm_swz(u >> 5);
      ga[q] = X + (kbeg + t) * ldx + min(r0 + 8 * c, n - 8);
      gb[q] = X + (kbeg + t) * ldx + min(c0 + 8 * c, n - 8);
    } else {
      const int r = u >> 2, c = (u & 3) ^ ((r >> 2) & 3);
      ga[q] = X + (int64_t)min(r0 + r, n - 1) * ldx + kbeg + 8 * c;
      gb[q] = X + (int64_t)min(c0 + r, n - 1) * ldx + kbeg + 8 * c;
    }
  }
  const int64_t kstep = TM ? (int64_t)BKL * ldx : (int64_t)BKL;   // elements per stage
  // token-major operand reads: lane-constant byte offsets of the A (t < TI)
  // and B (t >= TI) fragments within a slot, for tokens 8 (lane/32) .. + 3
  // of the stage's first 16 (the other reads add constant row offsets)
  int toff[TM ? TI + 4 : 1];
  if constexpr (TM) {
    const int g = lane >> 4, j = (lane >> 2) & 3, a = lane & 3;
#pragma unroll
    for (int t = 0; t < TI + 4; ++t) {
      const int f = (t < TI ? wm * WR + 32 * t : wn * 128 + 32 * (t - TI)) + 16 * (g & 1) + 4 * a;
      toff[t] = (t < TI ? 0 : BL * 64) + (8 * (g >> 1) + j) * 512 +
                (((f >> 3) ^ tm_swz(j)) << 4) + 2 * (f & 7);
    }
  }
  auto issue = [&](int stage) {
    const int slot = stage % NSLOT;
    const int64_t ko = (int64_t)stage * kstep;
#pragma unroll
    for (int q = 0; q < CPW; ++q) {
      __builtin_amdgcn_global_load_lds(
          (const void*)(ga[q] + ko),
          (__attribute__((address_space(3))) void*)&Ls[slot][0][(CPW * wave + q) * 64], 16, 0,
          0);
      __builtin_amdgcn_global_load_lds(
          (const void*)(gb[q] + ko),
          (__attribute__((address_space(3))) void*)&Ls[slot][1][(CPW * wave + q) * 64], 16, 0,
          0);
    }
  };
  auto compute = [&](int slot) {
    if (skip) return;
    const uint4* A = Ls[slot][0];
    const uint4* B = Ls[slot][1];
    if constexpr (TM) {
      // both token steps' operands in one block of transposed reads
      static_assert(TI + 4 == 6, "six operands per token step");
      const uint32_t sb = (uint32_t)(uintptr_t)(const lds_char*)&Ls[slot][0][0];
      uint32_t p[6];
      bf16x8_t o[12];
#pragma unroll
      for (int t = 0; t < 6; ++t) p[t] = sb + toff[t];
      tr_operands12(p, o);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(o[6 * ks + i], o[6 * ks + TI + j],
                                                                acc[i][j], 0, 0, 0);
      return;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      bf16x8_t a[TI], b[4];
#pragma unroll
      for (int t = 0; t < TI; ++t)
        a[t] = __builtin_bit_cast(bf16x8_t, A[swz(wm * WR + 32 * t + (lane & 31), c)]);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[t] = __builtin_bit_cast(bf16x8_t, B[swz(wn * 128 + 32 * t + (lane & 31), c)]);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };
  // Wait until this wave's DMA for the stage about to be computed has landed
  // (`later` stages, 2 CPW instructions each, may stay in flight) and its own
  // LDS reads are done, then meet the other waves.
  auto sync_stage = [&](int later) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    switch (later) {
      case 0: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0)); break;
      case 1: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(2 * CPW)); break;
      case 2: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(4 * CPW)); break;
      default: __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(6 * CPW)); break;
    }
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };

  for (int s = 0; s < AHEAD && s < nfull; ++s) issue(s);
  int s = 0;
  // steady state: stages s+1..s+3 in flight while stage s is waited for;
  // stage s+4 goes into the slot computed in the previous iteration, which
  // every wave has finished reading (barrier above)
  for (; s + AHEAD < nfull; ++s) {
    sync_stage(AHEAD - 1);
    issue(s + AHEAD);
    compute(s % NSLOT);
  }
  for (; s < nfull; ++s) {
    sync_stage(nfull - 1 - s);
    compute(s % NSLOT);
  }
  if (nstage > nfull) {
    // ragged token tail: one masked stage through registers
    sync_stage(0);
    const int slot = nfull % NSLOT;
    const int64_t k0 = kbeg + (int64_t)nfull * BKL;
#pragma unroll
    for (int i = 0; i < 1024 / NTL; ++i) {
      if constexpr (TM) {
        const int u = tid + NTL * i, t = u >> 5, c = (u & 31) ^ tm_swz(t);
        uint4 va = make_uint4(0, 0, 0, 0), vb = va;
        if (k0 + t < kend) {
          va = *(const uint4*)(X + (k0 + t) * ldx + min(r0 + 8 * c, n - 8));
          vb = *(const uint4*)(X + (k0 + t) * ldx + min(c0 + 8 * c, n - 8));
        }
        Ls[slot][0][u] = va;
        Ls[slot][1][u] = vb;
      } else {
        const int row = (tid >> 2) + (NTL / 4) * i;
        const int64_t kk = k0 + (tid & 3) * 8;
        Ls[slot][0][swz(row, tid & 3)] = load_vec<uint16_t>(X, ldx, r0 + row, n, kk, kend, aligned);
        Ls[slot][1][swz(row, tid & 3)] = load_vec<uint16_t>(X, ldx, c0 + row, n, kk, kend, aligned);
      }
    }
    __syncthreads();
    compute(slot);
  }

  if (!direct) {
    float* P = partial + ((int64_t)split * ntiles + tile) * (BL * BL);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * WR + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const int col = wn * 128 + j * 32 + (lane & 31);
          P[row * BL + col] = acc[i][j][r];
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int gr = r0 + wm * WR + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int gc = c0 + wn * 128 + j * 32 + (lane & 31);
        if (gr < n && gc <= gr) {
          float v = 2.0f * acc[i][j][r];
          if (accumulate) v += H[(int64_t)gr * n + gc];
          H[(int64_t)gr * n + gc] = v;
          if (gc != gr) H[(int64_t)gc * n + gr] = v;
        }
      }
}

// Sum split partials in split order, x2, (+H), write lower and mirror.
// One workgroup per 64x64 sub-block of a TE x TE output tile.
template <int TE>
__global__ __launch_bounds__(256) void syrk_reduce(
    const float* __restrict__ partial, int ntiles, int nsplit, int n,
    float* __restrict__ H, int accumulate) {
  constexpr int QB = TE / 64;           // sub-blocks per tile edge
  __shared__ float T[64][65];
  const int tile = blockIdx.x / (QB * QB), q = blockIdx.x % (QB * QB);
  int ti, tj;
  tile_coords(tile, (n + TE - 1) / TE, ti, tj);
  const int qr = (q / QB) * 64, qc = (q % QB) * 64;
  const int r0 = ti * TE + qr, c0 = tj * TE + qc;
  if (ti == tj && qr < qc) return;  // strictly-upper sub-block of a diagonal tile
  const int tid = threadIdx.x;
  const int64_t split_stride = (int64_t)ntiles * (TE * TE) / 4;   // float4 units
  // four float4 per thread; every split's loads of them in flight together,
  // summed in split order
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int e4 = tid + 256 * v;
    const int lr = e4 >> 4, lc = (e4 & 15) * 4;
    const float4* src = (const float4*)(partial + (int64_t)tile * (TE * TE) +
                                        (int64_t)(qr + lr) * TE + qc + lc);
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 8
    for (int sp = 0; sp < nsplit; ++sp) {
      const float4 p = src[sp * split_stride];
      s.x += p.x;
      s.y += p.y;
      s.z += p.z;
      s.w += p.w;
    }
    const float sv[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int gr = r0 + lr, gc = c0 + lc + u;
      float val = 2.0f * sv[u];
      if (gr < n && gc < n && gc <= gr) {
        if (accumulate) val += H[(int64_t)gr * n + gc];
        H[(int64_t)gr * n + gc] = val;
      }
      T[lr][lc + u] = val;
    }
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

bool syrk_aligned(const void* X, int64_t n, int64_t ldx, int32_t xdtype) {
  const int64_t es = (xdtype & kXTypeMask) == 1 ? 2 : 4;
  // token-major rows are read in 16-byte pieces of channels, so n must fill
  // whole pieces as well
  const bool tm = (xdtype & kXTokenMajor) != 0;
  return ((uintptr_t)X % 16 == 0) && ((ldx * es) % 16 == 0) && (!tm || (n * es) % 16 == 0);
}

void syrk_plan(int64_t n, int64_t ntok, int32_t xdtype, bool aligned, SyrkPlan* p) {
  // bf16 inputs on layers of >= 1024 channels (16-byte aligned rows) use the
  // 256x256 tile
  xdtype &= kXTypeMask;
  const bool big = xdtype == 1 && n >= 1024 && aligned;
  const int te = big ? BL : BM;
  const int bk = big ? BKL : (xdtype == 1 ? SyrkCfg<uint16_t>::BK : SyrkCfg<float>::BK);
  const int64_t nt = (n + te - 1) / te;
  p->tile = te;
  p->ntiles = nt * (nt + 1) / 2;
  const int64_t stages = (ntok + bk - 1) / bk;
  // Enough work items for a few rounds of workgroups; below that, a multiple
  // of 8 splits so that each XCD streams its own token range.
  const int64_t slots = big ? 256 : 512;      // resident workgroups
  const int64_t maxs = stages / 8 > 0 ? stages / 8 : 1;  // >= 8 stages per split
  int64_t ns = 1;
  if (p->ntiles < 3 * slots && big) {
    // 8..16 splits: the count whose last round of workgroups is fullest,
    // i.e. the least rounds x stages-per-split (ties: fewer partials)
    int64_t best = -1;
    for (int64_t c = 8; c <= 16; ++c) {
      const int64_t cost = ((p->ntiles * c + slots - 1) / slots) * ((stages + c - 1) / c);
      if (best < 0 || cost < best) {
        best = cost;
        ns = c;
      }
    }
  } else if (p->ntiles < 3 * slots) {
    const int64_t want = (4 * slots + p->ntiles - 1) / p->ntiles;
    ns = (want + 7) / 8 * 8;
  }
  if (ns > maxs) ns = maxs;
  if (ns > 64) ns = 64;
  if (ns < 1) ns = 1;
  int64_t kps = ((stages + ns - 1) / ns) * bk;
  if (kps < bk) kps = bk;           // ntok == 0: one empty split
  ns = (ntok + kps - 1) / kps;
  if (ns < 1) ns = 1;
  p->nsplit = ns;
  p->kps = kps;
  p->partial_bytes = ns > 1 ? (size_t)ns * p->ntiles * te * te * sizeof(float) : 0;
}

hipError_t launch_hessian(float* H, int64_t n, const void* X, int32_t xdtype,
                          int64_t ntok, int64_t ldx, int32_t accumulate,
                          const SyrkPlan& p, void* partial, hipStream_t st) {
  const bool aligned = syrk_aligned(X, n, ldx, xdtype);
  const bool tm = (xdtype & kXTokenMajor) != 0;
  xdtype &= kXTypeMask;
  const int direct = p.nsplit == 1;
  const int64_t items = p.ntiles * p.nsplit;
  const int per_xcd = (int)((items + 7) / 8);
  const unsigned grid = (unsigned)(8 * per_xcd);
  if (p.tile == BL && !aligned) return hipErrorInvalidValue;  // checked by the caller
  KernelTimer& timer = g_timers[PWQ_TIMER_HESSIAN_TILES];
  hipError_t te = hipSuccess;
  const int64_t ti = timer.begin(st, &te);
  if (te != hipSuccess) return te;
  const float* Xf = (const float*)X;
  const uint16_t* Xh = (const uint16_t*)X;
  float* P = (float*)partial;
  const int nti = (int)p.ntiles, nsp = (int)p.nsplit;
  if (p.tile == BL && tm)
    syrk_tiles256<true><<<grid, NTL, 0, st>>>(Xh, (int)n, ntok, ldx, p.kps, aligned, P, H,
                                              direct, accumulate, nti, nsp, per_xcd);
  else if (p.tile == BL)
    syrk_tiles256<false><<<grid, NTL, 0, st>>>(Xh, (int)n, ntok, ldx, p.kps, aligned, P, H,
                                               direct, accumulate, nti, nsp, per_xcd);
  else if (xdtype == 1 && tm)
    syrk_tiles<uint16_t, true><<<grid, NT, 0, st>>>(Xh, (int)n, ntok, ldx, p.kps, aligned, P,
                                                    H, direct, accumulate, nti, nsp, per_xcd);
  else if (xdtype == 1)
    syrk_tiles<uint16_t, false><<<grid, NT, 0, st>>>(Xh, (int)n, ntok, ldx, p.kps, aligned, P,
                                                     H, direct, accumulate, nti, nsp, per_xcd);
  else if (tm)
    syrk_tiles<float, true><<<grid, NT, 0, st>>>(Xf, (int)n, ntok, ldx, p.kps, aligned, P, H,
                                                 direct, accumulate, nti, nsp, per_xcd);
  else
    syrk_tiles<float, false><<<grid, NT, 0, st>>>(Xf, (int)n, ntok, ldx, p.kps, aligned, P, H,
                                                  direct, accumulate, nti, nsp, per_xcd);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = timer.end(ti, st);
  if (e != hipSuccess || direct) return e;
  if (p.tile == BL)
    syrk_reduce<BL><<<(unsigned)(p.ntiles * 16), 256, 0, st>>>(
        (const float*)partial, (int)p.ntiles, (int)p.nsplit, (int)n, H, accumulate);
  else
    syrk_reduce<BM><<<(unsigned)(p.ntiles * 4), 256, 0, st>>>(
        (const float*)partial, (int)p.ntiles, (int)p.nsplit, (int)n, H, accumulate);
  return hipGetLastError();
}

}  // namespace pwq
