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
// lower-triangular output tiles are computed.  bf16 X on layers of >= 1024
// channels (16-byte aligned rows) takes syrk_tiles256: 256x256 tiles, X
// streamed HBM -> LDS in 32-token stages by asynchronous copies through a
// five-slot ring, MFMA operands read from LDS one stage ahead of the
// v_mfma_f32_16x16x32_bf16 that use them (bf16 products are exact in
// fp32).  Each XCD owns a
// contiguous range of tiles; it computes whole rounds of them in one pass
// over the token axis and splits the remainder over the token axis so its
// 32 CUs finish together.  fp32 X, small or unaligned layers take
// syrk_tiles: 128x128 tiles with register-staged double buffering and
// v_mfma_f32_32x32x16_bf16 or v_mfma_f32_32x32x2f32.  Split tiles are summed
// in a fixed order by a reduction kernel (no float atomics, so results are
// bitwise reproducible), which also applies the factor 2, the optional
// accumulation into the previous H and the mirror into the upper triangle.
#include "pwq_device.h"
#include "pwq_internal.h"

#include <algorithm>

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

// Large-tile kernel for bf16 X: 256x256 output tiles, 8 waves of 64x128
// (4x8 v_mfma_f32_16x16x32_bf16 accumulators), two waves per SIMD.  A
// long launch of this kernel runs at the chip's power limit: the clock and
// the share of cycles the MFMA pipe is busy trade against each other, and
// the rate follows from the bytes moved per flop, which the 256x256 tile
// fixes.  The 16x16x32 form (a quarter of the accumulator data per
// instruction of the 32x32x16 form) and copies addressed from a scalar
// base (no 64-bit per-lane pointers to spill) come out a little ahead.
//
// Stages of 32 tokens (one MFMA K step) stream HBM -> LDS through a ring of
// NSLOT slots of 32 KB (the A and B panels, 16 KB each; 160 KB in all) with
// AHEAD stages in flight.  The copies are global_load_lds_dwordx4 issued
// from inline asm: the compiler then does not see an asynchronous LDS
// writer, so it neither drains the copy queue before LDS reads nor reorders
// them, and each wave waits for exactly its own copies (vmcnt) before the
// stage barrier.  The operands of stage s + 1 are read right after that
// barrier and before the MFMAs of stage s, so the LDS reads of one stage run
// under the MFMAs of the previous one (two operand register sets in turn).
// The ring is safe because the slot refilled after barrier s + 1 held stage
// s - 2, which every wave finished reading before it arrived there.
//
// Token-major X (TM): a panel stage is 32 token rows of 512 B (256
// channels); the MFMA operand (8 consecutive tokens of one channel per
// lane) comes from two ds_read_b64_tr_b16 (within each 16-lane group, lane i
// receives element i % 4 of the 8 bytes addressed by lane 4 j + i / 4 as
// its element j, so source lane 4 j + a addressing token row t0 + j,
// channels f0 + 4 a .. f0 + 4 a + 3 gives lane i tokens t0 .. t0 + 3 of
// channel f0 + i).  The 16-byte chunks of a token row are XOR-swizzled by
// 4 (row % 4) so the four rows a group reads fall in distinct banks.
// Channel-major X: a panel stage is 256 channel rows of 64 B (32 tokens);
// the operand is one ds_read_b128 of 8 tokens; the four chunks of a row are
// XOR-swizzled by bits 2-3 of the row, so 16 consecutive rows at one
// logical chunk cover all banks.  Both layouts feed the same values to the
// same MFMAs in the same order: H is bitwise the same.
//
// A 16x16x32 operand holds row (or column) l % 16 and the 8 tokens
// 8 (l / 16) .. 8 (l / 16) + 7 of the stage in lane l, for A and B alike,
// so the instruction sums exactly the stage's 32 token products of each
// output.  Result layout: lane l, register r -> row 4 (l / 16) + r,
// column l % 16 of the 16x16 block.
constexpr int BL = 256;        // tile edge
constexpr int BKS = 32;        // tokens per stage
constexpr int PANEL = BL * BKS * 2;   // bytes of one panel stage
constexpr int NSLOT = 5;       // LDS ring slots of two panels
constexpr int AHEAD = 3;       // stages in flight (<= NSLOT - 2)
constexpr int TRIP = 2 * NSLOT;   // stages per steady-state trip (operand sets alternate)
constexpr int NWL = 8;         // waves per workgroup, (NWL / 2) x 2 over the tile
constexpr int NTL = 64 * NWL;  // threads
constexpr int WR = 2 * BL / NWL;   // rows of a wave's sub-tile (columns: 128)
constexpr int FA = WR / 16;    // A operand fragments per stage and wave
constexpr int NFR = FA + 8;    // operand fragments per stage and wave (FA A, 8 B)
constexpr int NCPY = PANEL / (NTL * 16);   // 16-byte copies per lane and panel stage
static_assert(NSLOT * 2 * PANEL <= 160 * 1024, "ring fits the LDS");
static_assert(AHEAD <= NSLOT - 2, "refilled slot is two stages old");
static_assert(NCPY * NTL * 16 == PANEL, "whole copies per panel stage");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ int tm_swz(int r) { return 4 * (r & 3); }
__device__ __forceinline__ int cm_swz(int r) { return (r >> 2) & 3; }

// Copy 16 bytes per lane from global memory at sbase + voff into LDS at
// lds + 16 lane: a wave-uniform base in scalar registers plus a 32-bit
// per-lane byte offset, so no 64-bit per-lane address is kept (lds
// wave-uniform).  M0 holds the LDS base for the copy and is restored.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// Wait until at most `later` stages of this wave's copies (P instructions
// each) are still in flight, then meet the other waves.
template <int P>
__device__ __forceinline__ void stage_barrier(int later) {
  switch (later) {
#define PWQ_SB(L) \
    case L: asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(P * L) : "memory"); break;
    PWQ_SB(1) PWQ_SB(2) PWQ_SB(3) PWQ_SB(4) PWQ_SB(5) PWQ_SB(6) PWQ_SB(7)
#undef PWQ_SB
    default: asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
}
static_assert(AHEAD - 1 <= 7 && 2 * NCPY * 7 <= 63, "stage_barrier covers every count");

__device__ __forceinline__ bf16x8_t tr_operand(uint32_t a) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)a);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t)(a + 4 * 512));
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = lo[e];
    r[4 + e] = hi[e];
  }
  return r;
}

// 256 tiles: the XCD x owns tiles [tb, tb + cnt) of the super-block order;
// the first `d` of them are computed whole, the other `rem` are split.
__host__ __device__ __forceinline__ void xcd_tiles(int64_t T, int x, int mode, int& tb, int& d,
                                                   int& rem) {
  tb = (int)(T * x / 8);
  const int cnt = (int)(T * (x + 1) / 8) - tb;
  d = mode == 2 ? cnt : (mode == 1 ? 32 * (cnt / 32) : 0);
  rem = cnt - d;
}

template <bool TM, bool DIAG>
__device__ __forceinline__ void syrk256_tile(const uint16_t* __restrict__ X, int n, int64_t ldx,
                                             int r0, int c0, int64_t kbeg, int64_t kend,
                                             lds_char* Ls, f32x4_t (&acc)[FA][8]) {
  constexpr int NP = DIAG ? 1 : 2;          // panels copied per stage
  constexpr int P = NCPY * NP;              // copies per wave and stage
  constexpr uint32_t BOFF = DIAG ? 0 : PANEL;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;   // rows WR wm, columns 128 wn of the tile
  // waves entirely above the diagonal of a diagonal tile only copy
  const bool skip = DIAG && (WR * wm + WR - 1 < 128 * wn);
  const int nfull = (int)((kend - kbeg) / BKS);
  const int nstage = (int)((kend - kbeg + BKS - 1) / BKS);
  const uint32_t lbase = (uint32_t)(uintptr_t)Ls;

  // copy sources: copy h of lane l of wave w fills LDS unit
  // u = NTL h + 64 w + l of a panel stage, from a wave-uniform base plus a
  // per-lane byte offset (below 2^32: the host routes layers whose offsets
  // would not fit to the 128-tile kernel).  Token-major: copy h covers
  // token rows (NTL / 32) h + u / 32 with the same swizzle (it depends on
  // the row mod 4), so one offset per panel and a uniform row step serve
  // all of them.  Channel-major: rows (NTL / 4) h + u / 4, each clamped
  // into the matrix.
  const int u = 64 * wave + lane;
  constexpr int NPTR = TM ? 1 : NCPY;
  const uint16_t* ga[1];
  const uint16_t* gb[1];
  uint32_t oa_[NPTR], ob_[NPTR];   // byte offsets from the panel bases
  int64_t kstep, hstep;
  if constexpr (TM) {
    // token row u / 32, physical chunk u % 32 holding logical chunk
    // c = (u % 32) ^ tm_swz(row) of 8 channels; channels past n read
    // channels n - 8 .. n - 1 (only outputs past n, never stored, use them)
    const int t = u >> 5, c = (u & 31) ^ tm_swz(u >> 5);
    ga[0] = gb[0] = X + kbeg * ldx;
    oa_[0] = (uint32_t)(2 * ((int64_t)t * ldx + min(r0 + 8 * c, n - 8)));
    ob_[0] = (uint32_t)(2 * ((int64_t)t * ldx + min(c0 + 8 * c, n - 8)));
    kstep = (int64_t)BKS * ldx;
    hstep = (int64_t)(NTL / 32) * ldx;
  } else {
    // uniform panel bases; per-lane offsets within 256 rows of X
    ga[0] = X + (int64_t)r0 * ldx + kbeg;
    gb[0] = X + (int64_t)c0 * ldx + kbeg;
#pragma unroll
    for (int h = 0; h < NCPY; ++h) {
      // channel row uh / 4, physical chunk uh % 4 holding logical chunk
      // (uh % 4) ^ cm_swz(row) (8 tokens); rows past n read row n - 1
      const int uh = u + NTL * h;
      const int r = uh >> 2, c = (uh & 3) ^ cm_swz(r);
      oa_[h] = (uint32_t)(2 * ((min(r0 + r, n - 1) - r0) * ldx + 8 * c));
      ob_[h] = (uint32_t)(2 * ((min(c0 + r, n - 1) - c0) * ldx + 8 * c));
    }
    kstep = BKS;
    hstep = 0;
  }
  auto copy_stage = [&](int64_t ofs, uint32_t dst) {
#pragma unroll
    for (int h = 0; h < NCPY; ++h)
      dma16s(oa_[TM ? 0 : h], ga[0] + ofs + h * hstep, dst + 1024u * NWL * h);
    if constexpr (!DIAG) {
#pragma unroll
      for (int h = 0; h < NCPY; ++h)
        dma16s(ob_[TM ? 0 : h], gb[0] + ofs + h * hstep, dst + PANEL + 1024u * NWL * h);
    }
  };
  auto issue = [&](int stage) {
    copy_stage(stage * kstep, lbase + (uint32_t)(stage % NSLOT) * (2 * PANEL) + 1024u * wave);
  };
  // operand addresses within a slot: A fragments t < FA (rows WR wm + 16 t),
  // B fragments t >= FA (columns 128 wn + 16 (t - FA))
  uint32_t off[NFR];
#pragma unroll
  for (int t = 0; t < NFR; ++t) {
    const int f0 = t < FA ? wm * WR + 16 * t : wn * 128 + 16 * (t - FA);
    const uint32_t pb = t < FA ? 0u : BOFF;
    if constexpr (TM) {
      const int g = lane >> 4, j = (lane >> 2) & 3, a = lane & 3;
      const int f = f0 + 4 * a, row = 8 * g + j;
      off[t] = pb + (uint32_t)(row * 512 + (((f >> 3) ^ tm_swz(row)) << 4) + 2 * (f & 7));
    } else {
      const int row = f0 + (lane & 15), c = (lane >> 4) ^ cm_swz(row);
      off[t] = pb + (uint32_t)(row * 64 + 16 * c);
    }
  }
  // The slot base is made opaque per read pass: slot offsets past 64 KB do
  // not fit the LDS instructions' offset field, and the compiler would
  // otherwise keep a precomputed address per fragment and slot live.
  auto read = [&](int slot, bf16x8_t (&o)[NFR]) {
    uint32_t sb = lbase + (uint32_t)slot * (2 * PANEL);
    asm volatile("" : "+v"(sb));
#pragma unroll
    for (int t = 0; t < NFR; ++t) {
      if constexpr (TM)
        o[t] = tr_operand(sb + off[t]);
      else
        o[t] = *(const bf16x8_t*)(Ls + (sb - lbase) + off[t]);
    }
  };
  auto mfma = [&](const bf16x8_t (&o)[NFR]) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < FA; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o[i], o[FA + j], acc[i][j], 0, 0, 0);
  };
  // Interleave of one stage's work: one MFMA, one LDS read, ... while the
  // reads last, then the remaining MFMAs, so the LDS reads and the matrix
  // pipe run side by side.
  auto interleave = [&]() {
    constexpr int NRD = TM ? 2 * NFR : NFR;
#pragma unroll
    for (int i = 0; i < 8 * FA; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
      if (i < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
  };
  // one stage in the steady state, its ring slot K % NSLOT known at compile
  // time (the LDS offsets fold into the instructions): wait for stage
  // s + 1 and meet, refill the slot of stage s - 2 with stage s + AHEAD
  // from the running copy offset, read stage s + 1, multiply stage s
  int64_t pofs = AHEAD * kstep;
  auto step = [&](auto KK, bf16x8_t (&cur)[NFR], bf16x8_t (&nxt)[NFR]) {
    constexpr int K = decltype(KK)::value;
    stage_barrier<P>(AHEAD - 2);
    copy_stage(pofs, lbase + (uint32_t)((K + AHEAD) % NSLOT) * (2 * PANEL) + 1024u * wave);
    pofs += kstep;
    if (!skip) {
      read((K + 1) % NSLOT, nxt);
      mfma(cur);
      interleave();
    }
  };
  // the same near the end of the range, where fewer copies are in flight
  auto step_tail = [&](int s, bf16x8_t (&cur)[NFR], bf16x8_t (&nxt)[NFR]) {
    if (s + 1 < nfull) {
      stage_barrier<P>(min(nfull, s + AHEAD) - (s + 2));
      if (s + AHEAD < nfull) issue(s + AHEAD);
      if (!skip) read((s + 1) % NSLOT, nxt);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!skip) mfma(cur);
    __builtin_amdgcn_sched_barrier(0);
  };

  bf16x8_t oa[NFR], ob[NFR];
  if (nfull > 0) {
    const int first = min(nfull, AHEAD);
    for (int s = 0; s < first; ++s) issue(s);
    stage_barrier<P>(first - 1);
    if (!skip) read(0, oa);
  }
  int s = 0;
  // steady state: TRIP stages per trip (two turns of the ring, so the
  // operand sets alternate within it), every one issuing its copy
  static_assert(TRIP % 2 == 0 && TRIP % NSLOT == 0, "trip = whole turns, even length");
  for (; s + TRIP + AHEAD <= nfull; s += TRIP) {
    static_for_up<TRIP>([&](auto KK) {
      constexpr int K = decltype(KK)::value;
      if constexpr (K % 2 == 0)
        step(KK, oa, ob);
      else
        step(KK, ob, oa);
    });
  }
  for (; s < nfull; s += 2) {
    step_tail(s, oa, ob);
    if (s + 1 < nfull) step_tail(s + 1, ob, oa);
  }
  if (nstage > nfull) {
    // ragged token tail: one masked stage through registers into the slot
    // after the last full stage (every copy has landed: the last waits
    // above left none in flight)
    __syncthreads();
    const uint32_t sl = (uint32_t)(nfull % NSLOT) * (2 * PANEL);
    const int64_t k0 = kbeg + (int64_t)nfull * BKS;
#pragma unroll
    for (int pnl = 0; pnl < NP; ++pnl) {
      const int base = pnl ? c0 : r0;
#pragma unroll
      for (int h = 0; h < NCPY; ++h) {
        const int uh = u + NTL * h;
        uint4 v = make_uint4(0, 0, 0, 0);
        if constexpr (TM) {
          const int t = uh >> 5, c = (uh & 31) ^ tm_swz(uh >> 5);
          if (k0 + t < kend) v = *(const uint4*)(X + (k0 + t) * ldx + min(base + 8 * c, n - 8));
        } else {
          const int r = uh >> 2, c = (uh & 3) ^ cm_swz(r);
          const uint16_t* src = X + (int64_t)min(base + r, n - 1) * ldx + k0 + 8 * c;
          uint16_t tmp[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) tmp[e] = (k0 + 8 * c + e < kend) ? src[e] : (uint16_t)0;
          __builtin_memcpy(&v, tmp, sizeof(v));
        }
        *(uint4*)(Ls + sl + pnl * PANEL + 16 * uh) = v;
      }
    }
    __syncthreads();
    if (!skip) {
      read(nfull % NSLOT, oa);
      mfma(oa);
    }
  }
}

// Work item of workgroup blockIdx: XCD x = blockIdx % 8 (round-robin
// dispatch) takes its items in order: its whole tiles, then its split tiles
// split by split.  Whole tiles write H (x2, optional accumulation, lower
// triangle and its mirror); split tiles write their partial sum.
template <bool TM>
__global__ __launch_bounds__(NTL, 1) void syrk_tiles256(
    const uint16_t* __restrict__ X, int n, int64_t ntok, int64_t ldx, int64_t kps,
    float* __restrict__ partial, float* __restrict__ H, int accumulate, int64_t T, int nsplit,
    int mode, int nrem) {
  __shared__ __attribute__((aligned(16))) char Lsm[NSLOT * 2 * PANEL];
  lds_char* Ls = (lds_char*)Lsm;
  const int x = blockIdx.x & 7, l = blockIdx.x >> 3;
  int tb, d, rem;
  xcd_tiles(T, x, mode, tb, d, rem);
  int tile, pslot = -1;
  int64_t kbeg = 0, kend = ntok;
  if (l < d) {
    tile = tb + l;
  } else {
    const int j = l - d;
    if (j >= rem * nsplit) return;
    const int split = j / rem, r = j % rem;
    tile = tb + d + r;
    kbeg = (int64_t)split * kps;
    kend = min(ntok, kbeg + kps);
    int pre = 0;
    for (int y = 0; y < x; ++y) {
      int a, b, c;
      xcd_tiles(T, y, mode, a, b, c);
      pre += c;
    }
    pslot = split * nrem + pre + r;
  }
  const int nt = (n + BL - 1) / BL;
  int ti, tj;
  tile_coords(tile, nt, ti, tj);
  const int r0 = ti * BL, c0 = tj * BL;
  f32x4_t acc[FA][8];
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;
  if (ti == tj)
    syrk256_tile<TM, true>(X, n, ldx, r0, c0, kbeg, kend, Ls, acc);
  else
    syrk256_tile<TM, false>(X, n, ldx, r0, c0, kbeg, kend, Ls, acc);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // 16x16 result layout: lane l, register r -> row 4 (l / 16) + r, col l % 16
  if (pslot >= 0) {
    float* Pt = partial + (int64_t)pslot * (BL * BL);
#pragma unroll
    for (int i = 0; i < FA; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * WR + i * 16 + 4 * (lane >> 4) + r;
          const int col = wn * 128 + j * 16 + (lane & 15);
          Pt[row * BL + col] = acc[i][j][r];
        }
    return;
  }
#pragma unroll
  for (int i = 0; i < FA; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int gr = r0 + wm * WR + i * 16 + 4 * (lane >> 4) + r;
        const int gc = c0 + wn * 128 + j * 16 + (lane & 15);
        if (gr < n && gc <= gr) {
          float v = 2.0f * acc[i][j][r];
          if (accumulate) v += H[(int64_t)gr * n + gc];
          H[(int64_t)gr * n + gc] = v;
          if (gc != gr) H[(int64_t)gc * n + gr] = v;
        }
      }
}

// Sum the split partials of the split tiles in split order, x2, (+H), write
// the lower triangle and its mirror.  One workgroup per 64x64 sub-block of
// a split tile (split tile R of the list ordered by XCD, then position).
__global__ __launch_bounds__(256) void syrk_reduce_split(const float* __restrict__ partial,
                                                         int64_t T, int mode, int nsplit,
                                                         int nrem, int n, float* __restrict__ H,
                                                         int accumulate) {
  __shared__ float Tt[64][65];
  const int R = blockIdx.x / 16, q = blockIdx.x % 16;
  int tile = 0, pre = 0;
  for (int y = 0; y < 8; ++y) {
    int tb, d, rem;
    xcd_tiles(T, y, mode, tb, d, rem);
    if (R < pre + rem) {
      tile = tb + d + (R - pre);
      break;
    }
    pre += rem;
  }
  int ti, tj;
  tile_coords(tile, (n + BL - 1) / BL, ti, tj);
  const int qr = (q / 4) * 64, qc = (q % 4) * 64;
  const int r0 = ti * BL + qr, c0 = tj * BL + qc;
  if (ti == tj && qr < qc) return;  // strictly-upper sub-block of a diagonal tile
  const int tid = threadIdx.x;
  const int64_t split_stride = (int64_t)nrem * (BL * BL) / 4;   // float4 units
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int e4 = tid + 256 * v;
    const int lr = e4 >> 4, lc = (e4 & 15) * 4;
    const float4* src = (const float4*)(partial + (int64_t)R * (BL * BL) +
                                        (int64_t)(qr + lr) * BL + qc + lc);
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
      Tt[lr][lc + u] = val;
    }
  }
  __syncthreads();
  // mirrored writes, coalesced along the destination row
  for (int e = tid; e < 64 * 64; e += 256) {
    const int lr = e >> 6, lc = e & 63;   // destination row c0+lr, col r0+lc
    const int gr = r0 + lc, gc = c0 + lr; // source lower element (gr, gc)
    if (gr < n && gc < n && gc < gr) H[(int64_t)gc * n + gr] = Tt[lc][lr];
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
  // the 256-tile kernel addresses its copies by 32-bit byte offsets within
  // NTL / 32 token rows (token-major) or 256 channel rows (channel-major)
  // of X; a larger row stride takes the 128-tile kernel
  const int64_t span = (tm ? NTL / 32 : BL) * ldx * es;
  return ((uintptr_t)X % 16 == 0) && ((ldx * es) % 16 == 0) && (!tm || (n * es) % 16 == 0) &&
         span < ((int64_t)1 << 32);
}

void syrk_plan(int64_t n, int64_t ntok, int32_t xdtype, bool aligned, SyrkPlan* p) {
  xdtype &= kXTypeMask;
  const bool big = xdtype == 1 && n >= 1024 && aligned;
  p->mode = -1;
  p->nrem = 0;
  if (big) {
    // 256 tiles (bf16, >= 1024 channels, 16-byte rows): per-XCD tile ranges
    const int64_t nt = (n + BL - 1) / BL;
    const int64_t T = nt * (nt + 1) / 2;
    const int64_t stages = (ntok + BKS - 1) / BKS;
    p->tile = BL;
    p->ntiles = T;
    // time of one whole tile on one CU, and of writing and reading back one
    // partial tile, as estimates for choosing the decomposition
    const double t_tile = 2.0 * BL * BL * (double)ntok / 6.0e12;
    const double t_part = 2.0 * BL * BL * 4.0 / 4.0e12;
    double best = -1.0;
    int bmode = 2;
    int64_t bs = 1;
    for (int mode = 0; mode <= 2; ++mode) {
      const int64_t smax = mode == 2 ? 1 : std::max<int64_t>(1, std::min<int64_t>(64, stages / 16));
      for (int64_t S = (mode == 2 ? 1 : 2); S <= smax; ++S) {
        double worst = 0.0;
        int64_t nrem = 0;
        for (int x = 0; x < 8; ++x) {
          int tb, d, rem;
          xcd_tiles(T, x, mode, tb, d, rem);
          const double rounds = (double)((d + 31) / 32) +
                                (rem ? (double)((rem * S + 31) / 32) / (double)S : 0.0);
          worst = std::max(worst, rounds);
          nrem += rem;
        }
        const double cost = worst * t_tile + (S > 1 ? (double)(S * nrem) * t_part : 0.0);
        if (best < 0.0 || cost < best * (1.0 - 1e-9)) {
          best = cost;
          bmode = mode;
          bs = S;
        }
      }
    }
    int64_t kps = ((stages + bs - 1) / bs) * BKS;
    if (kps < BKS) kps = BKS;
    int64_t S = std::max<int64_t>(1, (ntok + kps - 1) / kps);
    if (S == 1) bmode = 2;
    p->mode = bmode;
    p->nsplit = bmode == 2 ? 1 : S;
    p->kps = bmode == 2 ? std::max<int64_t>(ntok, 1) : kps;
    int64_t nrem = 0, items = 0;
    for (int x = 0; x < 8; ++x) {
      int tb, d, rem;
      xcd_tiles(T, x, bmode, tb, d, rem);
      nrem += rem;
      items = std::max<int64_t>(items, d + rem * p->nsplit);
    }
    p->nrem = nrem;
    p->grid = 8 * std::max<int64_t>(items, 1);
    p->partial_bytes = nrem > 0 ? (size_t)p->nsplit * nrem * BL * BL * sizeof(float) : 0;
    return;
  }
  const int te = BM;
  const int bk = xdtype == 1 ? SyrkCfg<uint16_t>::BK : SyrkCfg<float>::BK;
  const int64_t nt = (n + te - 1) / te;
  p->tile = te;
  p->ntiles = nt * (nt + 1) / 2;
  const int64_t stages = (ntok + bk - 1) / bk;
  // enough work items for a few rounds of workgroups: a multiple of 8
  // splits, so that each XCD streams its own token range
  const int64_t slots = 512;                                // resident workgroups
  const int64_t maxs = stages / 8 > 0 ? stages / 8 : 1;     // >= 8 stages per split
  int64_t ns = 1;
  if (p->ntiles < 3 * slots) {
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
  p->grid = 8 * ((p->ntiles * ns + 7) / 8);
}

hipError_t launch_hessian(float* H, int64_t n, const void* X, int32_t xdtype,
                          int64_t ntok, int64_t ldx, int32_t accumulate,
                          const SyrkPlan& p, void* partial, hipStream_t st) {
  const bool aligned = syrk_aligned(X, n, ldx, xdtype);
  const bool tm = (xdtype & kXTokenMajor) != 0;
  xdtype &= kXTypeMask;
  if (p.tile == BL && !aligned) return hipErrorInvalidValue;  // checked by the caller
  KernelTimer& timer = g_timers[PWQ_TIMER_HESSIAN_TILES];
  hipError_t te = hipSuccess;
  const int64_t ti = timer.begin(st, &te);
  if (te != hipSuccess) return te;
  const float* Xf = (const float*)X;
  const uint16_t* Xh = (const uint16_t*)X;
  float* P = (float*)partial;
  const unsigned grid = (unsigned)p.grid;
  if (p.tile == BL) {
    if (tm)
      syrk_tiles256<true><<<grid, NTL, 0, st>>>(Xh, (int)n, ntok, ldx, p.kps, P, H, accumulate,
                                                p.ntiles, (int)p.nsplit, p.mode, (int)p.nrem);
    else
      syrk_tiles256<false><<<grid, NTL, 0, st>>>(Xh, (int)n, ntok, ldx, p.kps, P, H, accumulate,
                                                 p.ntiles, (int)p.nsplit, p.mode, (int)p.nrem);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = timer.end(ti, st);
    if (e != hipSuccess || p.nrem == 0) return e;
    syrk_reduce_split<<<(unsigned)(p.nrem * 16), 256, 0, st>>>(
        P, p.ntiles, p.mode, (int)p.nsplit, (int)p.nrem, (int)n, H, accumulate);
    return hipGetLastError();
  }
  const int direct = p.nsplit == 1;
  const int per_xcd = (int)(p.grid / 8);
  const int nti = (int)p.ntiles, nsp = (int)p.nsplit;
  if (xdtype == 1 && tm)
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
  syrk_reduce<BM><<<(unsigned)(p.ntiles * 4), 256, 0, st>>>(
      (const float*)partial, (int)p.ntiles, (int)p.nsplit, (int)n, H, accumulate);
  return hipGetLastError();
}

}  // namespace pwq
