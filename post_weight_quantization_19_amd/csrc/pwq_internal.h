// Host-side declarations shared by the libpwq translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pwq.h"
#include "pwq_device.h"

namespace pwq {

struct SyrkPlan {
  int tile;              // output tile edge (128 or 256)
  int64_t ntiles;
  int64_t nsplit;        // splits of the token axis (of every split tile)
  int64_t kps;           // tokens per split (multiple of the LDS stage)
  size_t partial_bytes;  // 0 when every tile writes H directly
  // 256 tiles: each XCD owns a contiguous range of tiles; `mode` says which
  // of them are computed whole (written straight into H) and which are
  // split over the token axis (partials, summed by the reduction).
  //   0: every tile split; 1: whole rounds of 32 tiles direct, the rest
  //   split; 2: every tile direct.
  int mode;
  int64_t nrem;          // split tiles over all XCDs
  int64_t grid;          // workgroups launched
};

// Overflow entries (SSQR): per-row counts, offsets and total; the sorted
// (row, column, value) list.
hipError_t launch_overflow_count(const int32_t* codes, int64_t m, int64_t n, int64_t ldc,
                                 int kind, int bits, int32_t* row_count, int64_t* row_off,
                                 int64_t* total, hipStream_t st);
hipError_t launch_overflow_write(const int32_t* codes, int64_t m, int64_t n, int64_t ldc,
                                 int kind, int bits, const float* scales, const int32_t* zeros,
                                 int G, const int64_t* row_off, int64_t max_out,
                                 int32_t* rows, int32_t* cols, float* vals, hipStream_t st);

// xdtype as at the boundary: element type in the low bits, kXTokenMajor
// when X is stored ntok x n.
constexpr int32_t kXTypeMask = 0xff;
constexpr int32_t kXTokenMajor = 0x100;
bool syrk_aligned(const void* X, int64_t n, int64_t ldx, int32_t xdtype);
void syrk_plan(int64_t n, int64_t ntok, int32_t xdtype, bool aligned, SyrkPlan* p);
hipError_t launch_hessian(float* H, int64_t n, const void* X, int32_t xdtype, int64_t ntok,
                          int64_t ldx, int32_t accumulate, const SyrkPlan& p, void* partial,
                          hipStream_t st);

// dscratch: kCholScratchBytes of workspace (diagonal blocks in flight).
constexpr size_t kCholScratchBytes = 2 * 64 * 64 * sizeof(double);
hipError_t launch_damp_cholesky(const float* H, int64_t n, double damp, int32_t prec,
                                const int32_t* perm, void* L, int32_t* dead, pwq_result* res,
                                DevFlags* flags, double* lam, void* dscratch, hipStream_t st);
// The same for fp32 in natural order with H already in the working copy A
// (both triangles or the lower one; the upper is overwritten with zeros).
hipError_t launch_damp_cholesky_in_place(float* A, int64_t n, double damp, int32_t* dead,
                                         pwq_result* res, DevFlags* flags, double* lam,
                                         void* dscratch, hipStream_t st);

// OA-EM codebook initialisation (all float64).  Workspace: Hb ng g g,
// R m n, Q ng K, S ng K g doubles, cnt ng K int32, part
// oaem_objective_parts(m, n, g) doubles.
constexpr int kOaemMaxG = 16;
constexpr int kOaemMaxLds = 8192;   // K (g + 1) doubles of codebook and norms in LDS
struct OaemWs {
  double* Hb;
  double* R;
  double* Q;
  double* S;
  int32_t* cnt;
  double* part;
};
int64_t oaem_objective_parts(int64_t m, int64_t n, int32_t g);
hipError_t launch_oaem(const void* W, int32_t wdtype, int64_t m, int64_t n, int64_t ldw,
                       const float* H, const double* lam, int32_t g, int32_t K, int32_t M,
                       int32_t iters, const int64_t* seeds, double* books, int32_t* codes,
                       double* obj, pwq_result* res, const OaemWs& w, hipStream_t st);

// Dead inputs and lambda = damp * mean(diag H after the dead fix), as the
// first stage of launch_damp_cholesky (writes res->lambda, res->ndead).
hipError_t launch_damp_lambda(const float* H, int64_t n, double damp, int32_t* dead,
                              pwq_result* res, DevFlags* flags, double* lam, hipStream_t st);

hipError_t launch_grid_steps(const void* W, int32_t wdtype, int64_t m, int64_t n, int64_t ldw,
                             const int32_t* dead, int kind, int bits, int G, float* scales,
                             int32_t* zeros, const DevFlags* flags, hipStream_t st,
                             float kappa = 1.0f);

// Columns of a lazy-update group: the sweep applies a block's errors to the
// rest of its group at once and a whole group's errors to the columns before
// it in one pass; the sweep workspace holds one group of errors per row.
// fp32: 256 (the register-resident E of the group kernel); fp64: 512 (the
// generic kernel stages any K through LDS).  A multiple of every block size.
inline int update_group_cols(int32_t prec) { return prec == PWQ_F64 ? 512 : 256; }

struct SweepLaunch {
  const void* W;
  int32_t wdtype;
  int64_t ldw, m, n;
  int32_t prec, block;
  const void* L;
  void* invd;
  void* dg;
  void* alpha;
  int colspacing;
  double c;
  float* scales;       // SYM/ASYM input
  float* scales_out;   // COLSPACING output (per original column)
  const int32_t* zeros;
  int ng, G;
  const int32_t* colmap;
  const int32_t* dead;
  void* acc;
  void* E;
  int32_t* codes;
  double* partials;
  pwq_result* result;
  const DevFlags* flags;
};

size_t sweep_partials_bytes(int64_t m, int64_t n, int32_t block, int32_t prec);
hipError_t launch_sweep(const SweepLaunch& sl, hipStream_t st);

hipError_t launch_order(int32_t order_kind, const float* H, int64_t n, const int32_t* perm_in,
                        int32_t* perm_out, int32_t* seen, pwq_result* res, DevFlags* flags,
                        hipStream_t st);
// perm[k] = k (a valid map for every later kernel whatever happens after).
hipError_t launch_identity_perm(int32_t* perm, int64_t n, hipStream_t st);
hipError_t launch_init_flags(DevFlags* flags, pwq_result* res, int reset_info, hipStream_t st);

// Min-pivot order (pivoted LDL^T in fp64).  Workspace: A n x n doubles,
// P n x kMinPivotPanel doubles, d n doubles, pos and rem n int32 each, and
// 2 ceil(n / 256) (double, int32) partial minima.
constexpr int kMinPivotPanel = 32;
struct MinPivotWs {
  double* A;
  double* P;
  double* d;
  int32_t* pos;
  int32_t* rem;
  double* part_v;
  int32_t* part_i;
};
// perm[k] = column of position k; piv[k] = D_kk (may be NULL).  lam: the
// damping (device double, from launch_damp_lambda).  A pivot that is not
// positive sets flags->info = res->info = k + 1 and ends the work.
hipError_t launch_min_pivot(const float* H, int64_t n, const double* lam, const MinPivotWs& w,
                            int32_t* perm, double* piv, DevFlags* flags, pwq_result* res,
                            hipStream_t st);

// cmin / cmax: n int32 each of workspace.
hipError_t launch_column_entropy(const int32_t* codes, int64_t m, int64_t n, int64_t ldc,
                                 double* bits, double* mean, int64_t* huff, int32_t* cmin,
                                 int32_t* cmax, hipStream_t st);

// Event pairs recorded around launches of one kernel (pwq_kernel_timer_attach).
struct KernelTimer {
  hipEvent_t* starts = nullptr;
  hipEvent_t* stops = nullptr;
  int64_t capacity = 0;
  int64_t used = 0;
  // Returns the pair index to record, or -1 when not attached / full.
  int64_t next() { return used < capacity ? used++ : -1; }
  // Start event of the next pair on `st` (if attached); returns its index.
  int64_t begin(hipStream_t st, hipError_t* err) {
    const int64_t i = next();
    if (i >= 0) *err = hipEventRecord(starts[i], st);
    return i;
  }
  hipError_t end(int64_t i, hipStream_t st) {
    return i >= 0 ? hipEventRecord(stops[i], st) : hipSuccess;
  }
};
// indexed by pwq_timed_kernel
constexpr int kNumTimers = 3;
extern KernelTimer g_timers[kNumTimers];

}  // namespace pwq
