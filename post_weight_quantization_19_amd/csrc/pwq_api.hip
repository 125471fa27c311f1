// extern "C" entry points of libpwq: argument validation, workspace carving
// and stage orchestration.  Every argument check runs before any HIP call,
// so invalid requests return without touching the device.
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "pwq_internal.h"

#include <algorithm>
#include <cmath>
#include <mutex>

using namespace pwq;

namespace pwq {
KernelTimer g_timers[kNumTimers];
}

namespace {

thread_local std::string g_last_error;

pwq_status fail(pwq_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

pwq_status ok() {
  g_last_error.clear();
  return PWQ_OK;
}

pwq_status hip_fail(hipError_t e, const char* where) {
  return fail(PWQ_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;

// Bump allocator over the caller's workspace; with base == nullptr it only
// measures, so sizing and carving share one code path.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    off = (off + kAlign - 1) / kAlign * kAlign;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
  size_t size() const { return (off + kAlign - 1) / kAlign * kAlign; }
};

size_t elem(int32_t prec) { return prec == PWQ_F64 ? 8 : 4; }

// Scratch of pwq_damp_cholesky_static: the status flags, lambda and the
// side buffer of diagonal blocks that pwq_damp_cholesky otherwise carves from
// the caller's workspace.  One copy per GPU, held until the process ends;
// host code uses only the device address looked up below, never the name.
constexpr size_t kStaticScratchBytes = 68 * 1024;
__device__ __align__(256) char scratch[kStaticScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch copy on the GPU that runs `st` (the current
// GPU for the null stream), looked up once per GPU with that GPU current.
hipError_t static_scratch(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

bool valid_block(int32_t b) { return b == 32 || b == 64 || b == 128 || b == 256; }

pwq_status check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return PWQ_OK;
  if (!ws) return fail(PWQ_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if ((uintptr_t)ws % kAlign)
    return fail(PWQ_ERR_WORKSPACE, "workspace must be %zu-byte aligned", kAlign);
  if (ws_bytes < need)
    return fail(PWQ_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, need);
  return PWQ_OK;
}

pwq_status check_grid(const pwq_grid* g, int64_t n, bool allow_colspacing) {
  if (!g) return fail(PWQ_ERR_INVALID_ARG, "grid is NULL");
  if (g->reserved != 0) return fail(PWQ_ERR_INVALID_ARG, "grid.reserved must be 0");
  if (g->kind == PWQ_GRID_SYM || g->kind == PWQ_GRID_ASYM) {
    if (g->bits < 2 || g->bits > 16)
      return fail(PWQ_ERR_INVALID_ARG, "bits must be in [2, 16] (got %d)", g->bits);
    if (g->group_size < 0) return fail(PWQ_ERR_INVALID_ARG, "group_size must be >= 0");
    if (g->group_size > 0 && n % g->group_size)
      return fail(PWQ_ERR_INVALID_ARG, "group_size %d does not divide n = %lld", g->group_size,
                  (long long)n);
    if (g->c != 0.0)
      return fail(PWQ_ERR_INVALID_ARG, "grid.c is the COLSPACING constant: 0 for SYM / ASYM");
    if (!(g->kappa >= 0.0) || !(g->kappa < 1e30))
      return fail(PWQ_ERR_INVALID_ARG, "the step multiplier kappa must be 0 (none) or finite > 0");
    return PWQ_OK;
  }
  if (g->kind == PWQ_GRID_COLSPACING) {
    if (!allow_colspacing) return fail(PWQ_ERR_INVALID_ARG, "COLSPACING steps need the factor");
    if (!(g->c > 0.0) || !(g->c < 1e300))
      return fail(PWQ_ERR_INVALID_ARG, "COLSPACING needs a finite c > 0");
    if (g->kappa != 0.0)
      return fail(PWQ_ERR_INVALID_ARG, "grid.kappa is for SYM / ASYM: 0 for COLSPACING");
    return PWQ_OK;
  }
  return fail(PWQ_ERR_INVALID_ARG, "unknown grid kind %d", g->kind);
}

int group_of(const pwq_grid* g, int64_t n) { return g->group_size > 0 ? g->group_size : (int)n; }

// SYM / ASYM: kappa is a multiplier on every step (0 means none).
float step_multiplier(const pwq_grid* g) { return g->kappa > 0.0 ? (float)g->kappa : 1.0f; }

// ---- workspace layouts (shared by sizing and carving)

struct SweepWs {
  DevFlags* flags;
  void *invd, *dg, *alpha, *acc, *E;
  double* partials;
};

void carve_sweep(Carver& c, int64_t m, int64_t n, int32_t block, int32_t prec, SweepWs* w) {
  w->invd = c.take((size_t)n * elem(prec));
  w->dg = c.take((size_t)n * elem(prec));
  w->alpha = c.take((size_t)n * elem(prec));
  w->acc = c.take((size_t)m * n * elem(prec));
  w->E = c.take((size_t)m * update_group_cols(prec) * elem(prec));   // a group of errors per row
  w->partials = (double*)c.take(sweep_partials_bytes(m, n, block, prec));
}

void carve_min_pivot(Carver& c, int64_t n, MinPivotWs* w) {
  const int64_t g = (n + 255) / 256;
  w->A = (double*)c.take((size_t)n * n * sizeof(double));
  w->P = (double*)c.take((size_t)n * kMinPivotPanel * sizeof(double));
  w->d = (double*)c.take((size_t)n * sizeof(double));
  w->pos = (int32_t*)c.take((size_t)n * 4);
  w->rem = (int32_t*)c.take((size_t)n * 4);
  w->part_v = (double*)c.take((size_t)2 * g * sizeof(double));
  w->part_i = (int32_t*)c.take((size_t)2 * g * 4);
}

struct LayerWs {
  DevFlags* flags;
  double* lam;
  int32_t* perm;
  int32_t* seen;
  int32_t* dead;
  float* H;
  void* partial;
  void* L;
  void* dscratch;
  SweepWs sw;
  MinPivotWs mp;
};

void carve_layer(Carver& c, int64_t m, int64_t n, int64_t ntok, bool has_x, bool need_h,
                 bool need_l, int32_t xdtype, bool x_aligned, int32_t block, int32_t prec,
                 bool min_pivot, LayerWs* w) {
  w->flags = (DevFlags*)c.take(sizeof(DevFlags));
  w->lam = (double*)c.take(sizeof(double));
  w->perm = (int32_t*)c.take((size_t)n * 4);
  w->seen = (int32_t*)c.take((size_t)n * 4);
  w->dead = (int32_t*)c.take((size_t)n * 4);
  w->H = need_h ? (float*)c.take((size_t)n * n * 4) : nullptr;
  w->partial = nullptr;
  if (has_x) {
    SyrkPlan p;
    syrk_plan(n, ntok, xdtype, x_aligned, &p);
    w->partial = p.partial_bytes ? c.take(p.partial_bytes) : nullptr;
  }
  w->L = need_l ? c.take((size_t)n * n * elem(prec)) : nullptr;
  w->dscratch = c.take(kCholScratchBytes);
  carve_sweep(c, m, n, block, prec, &w->sw);
  w->mp = MinPivotWs{};
  if (min_pivot) carve_min_pivot(c, n, &w->mp);
}

}  // namespace

extern "C" {

const char* pwq_status_string(pwq_status s) {
  // A C caller may pass any integer; an enum object holding a value outside
  // its enumerators' range may not be read as the enum in C++, so its bytes
  // are read as an integer.
  int32_t v;
  static_assert(sizeof(s) == sizeof(v), "pwq_status is 32-bit");
  __builtin_memcpy(&v, &s, sizeof(v));
  switch (v) {
    case PWQ_OK: return "PWQ_OK";
    case PWQ_ERR_INVALID_ARG: return "PWQ_ERR_INVALID_ARG";
    case PWQ_ERR_UNSUPPORTED: return "PWQ_ERR_UNSUPPORTED";
    case PWQ_ERR_WORKSPACE: return "PWQ_ERR_WORKSPACE";
    case PWQ_ERR_HIP: return "PWQ_ERR_HIP";
  }
  return "PWQ_ERR_UNKNOWN";
}

const char* pwq_last_error(void) { return g_last_error.c_str(); }

// ------------------------------------------------------------------ Hessian

// Element type and layout of X (xdtype = PWQ_BF16 / PWQ_F32, optionally
// | PWQ_X_TOKEN_MAJOR) and its row stride.
static pwq_status check_x(int64_t n, int64_t ntok, int32_t xdtype, int64_t ldx) {
  const int32_t el = xdtype & ~PWQ_X_TOKEN_MAJOR;
  if (el != PWQ_BF16 && el != PWQ_F32)
    return fail(PWQ_ERR_INVALID_ARG,
                "X dtype must be PWQ_BF16 or PWQ_F32 (optionally | PWQ_X_TOKEN_MAJOR)");
  if (xdtype & PWQ_X_TOKEN_MAJOR) {
    if (ldx < n) return fail(PWQ_ERR_INVALID_ARG, "token-major X needs ldx >= n");
  } else if (ldx < ntok) {
    return fail(PWQ_ERR_INVALID_ARG, "ldx < ntok");
  }
  return PWQ_OK;
}

size_t pwq_hessian_workspace_size(int64_t n, int64_t ntok) {
  if (n <= 0 || ntok < 0) return 0;
  size_t need = 0;
  for (int dt = 0; dt < 2; ++dt)
    for (int al = 0; al < 2; ++al) {
      SyrkPlan p;
      syrk_plan(n, ntok, dt == 0 ? PWQ_BF16 : PWQ_F32, al != 0, &p);
      if (p.partial_bytes > need) need = p.partial_bytes;
    }
  return (need + kAlign - 1) / kAlign * kAlign;
}

pwq_status pwq_hessian_accum(float* H, int64_t n, const void* X, int32_t xdtype, int64_t ntok,
                             int64_t ldx, int32_t accumulate, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!H) return fail(PWQ_ERR_INVALID_ARG, "H is NULL");
  if (n <= 0 || n > 65536) return fail(PWQ_ERR_INVALID_ARG, "n must be in [1, 65536]");
  if (ntok < 0) return fail(PWQ_ERR_INVALID_ARG, "ntok must be >= 0");
  if (ntok > 0 && !X) return fail(PWQ_ERR_INVALID_ARG, "X is NULL");
  pwq_status s = check_x(n, ntok, xdtype, ldx);
  if (s != PWQ_OK) return s;
  SyrkPlan p;
  syrk_plan(n, ntok, xdtype, syrk_aligned(X, n, ldx, xdtype), &p);
  s = check_ws(ws, ws_bytes, p.partial_bytes);
  if (s != PWQ_OK) return s;
  hipError_t e = launch_hessian(H, n, X, xdtype, ntok, ldx, accumulate, p, ws,
                                (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hessian_accum launch");
  return ok();
}

// ----------------------------------------------------------------- Cholesky

size_t pwq_cholesky_workspace_size(int64_t n, int32_t prec) {
  (void)n;
  (void)prec;
  Carver c(nullptr);
  c.take(sizeof(DevFlags));
  c.take(sizeof(double));
  c.take(kCholScratchBytes);
  return c.size();
}

static pwq_status check_damp_cholesky(const float* H, int64_t n, double damp, int32_t prec,
                                      const void* L, const pwq_result* result) {
  if (!H || !L || !result) return fail(PWQ_ERR_INVALID_ARG, "H, L and result must be non-NULL");
  if (n <= 0 || n > 65536) return fail(PWQ_ERR_INVALID_ARG, "n must be in [1, 65536]");
  if (prec != PWQ_F32 && prec != PWQ_F64)
    return fail(PWQ_ERR_INVALID_ARG, "prec must be PWQ_F32 or PWQ_F64");
  if (!(damp >= 0.0) || !(damp < 1e30)) return fail(PWQ_ERR_INVALID_ARG, "damp must be >= 0");
  return PWQ_OK;
}

pwq_status pwq_damp_cholesky(const float* H, int64_t n, double damp, int32_t prec, void* L,
                             int32_t* dead, pwq_result* result, void* ws, size_t ws_bytes,
                             void* stream) {
  pwq_status s = check_damp_cholesky(H, n, damp, prec, L, result);
  if (s != PWQ_OK) return s;
  s = check_ws(ws, ws_bytes, pwq_cholesky_workspace_size(n, prec));
  if (s != PWQ_OK) return s;
  Carver c(ws);
  DevFlags* flags = (DevFlags*)c.take(sizeof(DevFlags));
  double* lam = (double*)c.take(sizeof(double));
  void* dscratch = c.take(kCholScratchBytes);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_init_flags(flags, result, 1, st);
  if (e == hipSuccess)
    e = launch_damp_cholesky(H, n, damp, prec, nullptr, L, dead, result, flags, lam, dscratch,
                             st);
  if (e != hipSuccess) return hip_fail(e, "damp_cholesky launch");
  return ok();
}

pwq_status pwq_damp_cholesky_static(const float* H, int64_t n, double damp, int32_t prec,
                                    void* L, int32_t* dead, pwq_result* result, void* stream) {
  pwq_status s = check_damp_cholesky(H, n, damp, prec, L, result);
  if (s != PWQ_OK) return s;
  const size_t need = pwq_cholesky_workspace_size(n, prec);
  if (need > kStaticScratchBytes)
    return fail(PWQ_ERR_WORKSPACE, "needs %zu bytes of scratch; the static scratch holds %zu",
                need, kStaticScratchBytes);
  void* ws = nullptr;
  const hipError_t e = static_scratch((hipStream_t)stream, &ws);
  if (e != hipSuccess) return hip_fail(e, "static scratch lookup");
  return pwq_damp_cholesky(H, n, damp, prec, L, dead, result, ws, kStaticScratchBytes, stream);
}

// -------------------------------------------------------------------- steps

pwq_status pwq_grid_steps(const void* W, int32_t wdtype, int64_t m, int64_t n, int64_t ldw,
                          const int32_t* dead, const pwq_grid* grid, float* scales,
                          int32_t* zeros, void* stream) {
  if (!W || !scales) return fail(PWQ_ERR_INVALID_ARG, "W and scales must be non-NULL");
  if (m <= 0 || n <= 0) return fail(PWQ_ERR_INVALID_ARG, "m and n must be positive");
  if (wdtype != PWQ_BF16 && wdtype != PWQ_F32)
    return fail(PWQ_ERR_INVALID_ARG, "W dtype must be PWQ_BF16 or PWQ_F32");
  if (ldw < n) return fail(PWQ_ERR_INVALID_ARG, "ldw < n");
  pwq_status s = check_grid(grid, n, false);
  if (s != PWQ_OK) return s;
  if (grid->kind == PWQ_GRID_ASYM && !zeros)
    return fail(PWQ_ERR_INVALID_ARG, "ASYM grid needs zeros");
  hipError_t e = launch_grid_steps(W, wdtype, m, n, ldw, dead, grid->kind, grid->bits,
                                   group_of(grid, n), scales, zeros, nullptr,
                                   (hipStream_t)stream, step_multiplier(grid));
  if (e != hipSuccess) return hip_fail(e, "grid_steps launch");
  return ok();
}

// -------------------------------------------------------------------- sweep

size_t pwq_sweep_workspace_size(int64_t m, int64_t n, int32_t block, int32_t prec) {
  if (m < 0 || n <= 0 || !valid_block(block)) return 0;
  if (prec != PWQ_F32 && prec != PWQ_F64) return 0;
  Carver c(nullptr);
  c.take(sizeof(DevFlags));
  SweepWs w;
  carve_sweep(c, m, n, block, prec, &w);
  return c.size();
}

static pwq_status check_sweep_common(const void* W, int32_t wdtype, int64_t m, int64_t n,
                                     int64_t ldw, int32_t prec, const pwq_grid* grid,
                                     float* scales, const int32_t* zeros, int32_t block,
                                     int32_t* codes, pwq_result* result) {
  if (!W && m > 0) return fail(PWQ_ERR_INVALID_ARG, "W is NULL");
  if (!codes && m > 0) return fail(PWQ_ERR_INVALID_ARG, "codes is NULL");
  if (!result) return fail(PWQ_ERR_INVALID_ARG, "result is NULL");
  if (m < 0 || m > (1 << 30)) return fail(PWQ_ERR_INVALID_ARG, "m out of range");
  if (n <= 0 || n > 65536) return fail(PWQ_ERR_INVALID_ARG, "n must be in [1, 65536]");
  if (wdtype != PWQ_BF16 && wdtype != PWQ_F32)
    return fail(PWQ_ERR_INVALID_ARG, "W dtype must be PWQ_BF16 or PWQ_F32");
  if (ldw < n) return fail(PWQ_ERR_INVALID_ARG, "ldw < n");
  if (prec != PWQ_F32 && prec != PWQ_F64)
    return fail(PWQ_ERR_INVALID_ARG, "prec must be PWQ_F32 or PWQ_F64");
  if (!valid_block(block))
    return fail(PWQ_ERR_UNSUPPORTED, "block must be 32, 64, 128 or 256 (got %d)", block);
  pwq_status s = check_grid(grid, n, true);
  if (s != PWQ_OK) return s;
  if (!scales && (m > 0 || grid->kind == PWQ_GRID_COLSPACING))
    return fail(PWQ_ERR_INVALID_ARG, "scales is NULL");
  if (grid->kind == PWQ_GRID_ASYM && !zeros)
    return fail(PWQ_ERR_INVALID_ARG, "ASYM grid needs zeros");
  return PWQ_OK;
}

pwq_status pwq_babai_sweep(const void* W, int32_t wdtype, int64_t m, int64_t n, int64_t ldw,
                           const void* L, int32_t prec, const int32_t* dead,
                           const pwq_grid* grid, float* scales, const int32_t* zeros,
                           int32_t block, int32_t* codes, pwq_result* result, void* ws,
                           size_t ws_bytes, void* stream) {
  pwq_status s = check_sweep_common(W, wdtype, m, n, ldw, prec, grid, scales, zeros, block,
                                    codes, result);
  if (s != PWQ_OK) return s;
  if (!L) return fail(PWQ_ERR_INVALID_ARG, "L is NULL");
  s = check_ws(ws, ws_bytes, pwq_sweep_workspace_size(m, n, block, prec));
  if (s != PWQ_OK) return s;
  Carver c(ws);
  DevFlags* flags = (DevFlags*)c.take(sizeof(DevFlags));
  SweepWs w;
  carve_sweep(c, m, n, block, prec, &w);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_init_flags(flags, result, 1, st);
  if (e != hipSuccess) return hip_fail(e, "babai_sweep launch");
  SweepLaunch sl{};
  sl.W = W; sl.wdtype = wdtype; sl.ldw = ldw; sl.m = m; sl.n = n; sl.prec = prec;
  sl.block = block; sl.L = L; sl.invd = w.invd; sl.dg = w.dg; sl.alpha = w.alpha;
  sl.colspacing = grid->kind == PWQ_GRID_COLSPACING; sl.c = grid->c;
  sl.scales = scales; sl.scales_out = scales;
  sl.zeros = grid->kind == PWQ_GRID_ASYM ? zeros : nullptr;
  const int G = sl.colspacing ? 1 : group_of(grid, n);
  sl.G = G; sl.ng = (int)(n / G);
  sl.colmap = nullptr; sl.dead = dead; sl.acc = w.acc; sl.E = w.E; sl.codes = codes;
  sl.partials = w.partials; sl.result = result; sl.flags = flags;
  e = launch_sweep(sl, st);
  if (e != hipSuccess) return hip_fail(e, "babai_sweep launch");
  return ok();
}

// -------------------------------------------------------------- whole layer

size_t pwq_quant_layer_workspace_size(int64_t m, int64_t n, int64_t ntok, int32_t has_x,
                                      int32_t order_kind, int32_t block, int32_t prec) {
  if (m < 0 || n <= 0 || !valid_block(block)) return 0;
  const bool mp = order_kind == PWQ_ORDER_MIN_PIVOT;
  // size for the worst case: H and L kept in the workspace, any X dtype and
  // alignment
  size_t need = 0;
  for (int dt = 0; dt < 2; ++dt)
    for (int al = 0; al < 2; ++al) {
      Carver c(nullptr);
      LayerWs w;
      carve_layer(c, m, n, ntok, has_x != 0, has_x != 0, true, dt == 0 ? PWQ_BF16 : PWQ_F32,
                  al != 0, block, prec, mp, &w);
      if (c.size() > need) need = c.size();
    }
  return need;
}

pwq_status pwq_quant_layer(const void* W, int32_t wdtype, int64_t m, int64_t n, int64_t ldw,
                           const void* X, int32_t xdtype, int64_t ntok, int64_t ldx,
                           const float* H, const pwq_grid* grid, int32_t order_kind,
                           const int32_t* perm, double damp, int32_t block, int32_t prec,
                           int32_t* codes, float* scales, int32_t* zeros, pwq_result* result,
                           float* H_out, void* L_out, void* ws, size_t ws_bytes,
                           void* stream) {
  pwq_status s = check_sweep_common(W, wdtype, m, n, ldw, prec, grid, scales, zeros, block,
                                    codes, result);
  if (s != PWQ_OK) return s;
  const bool has_x = X != nullptr;
  if (has_x == (H != nullptr)) return fail(PWQ_ERR_INVALID_ARG, "give exactly one of X and H");
  if (has_x) {
    if (ntok < 0) return fail(PWQ_ERR_INVALID_ARG, "ntok must be >= 0");
    s = check_x(n, ntok, xdtype, ldx);
    if (s != PWQ_OK) return s;
  } else if (H_out) {
    return fail(PWQ_ERR_INVALID_ARG, "H_out is only produced when X is given");
  }
  if (order_kind < PWQ_ORDER_BACK_TO_FRONT || order_kind > PWQ_ORDER_MIN_PIVOT)
    return fail(PWQ_ERR_INVALID_ARG, "unknown order %d", order_kind);
  if (order_kind == PWQ_ORDER_PERM && !perm)
    return fail(PWQ_ERR_INVALID_ARG, "PERM order needs perm");
  if (!(damp >= 0.0) || !(damp < 1e30)) return fail(PWQ_ERR_INVALID_ARG, "damp must be >= 0");

  const bool need_h = has_x && !H_out;
  const bool need_l = !L_out;
  const bool xal = has_x && syrk_aligned(X, n, ldx, xdtype);
  Carver measure(nullptr);
  LayerWs w;
  const bool mp = order_kind == PWQ_ORDER_MIN_PIVOT;
  carve_layer(measure, m, n, ntok, has_x, need_h, need_l, xdtype, xal, block, prec, mp, &w);
  s = check_ws(ws, ws_bytes, measure.size());
  if (s != PWQ_OK) return s;
  Carver c(ws);
  carve_layer(c, m, n, ntok, has_x, need_h, need_l, xdtype, xal, block, prec, mp, &w);
  hipStream_t st = (hipStream_t)stream;
  void* Lm = L_out ? L_out : w.L;
  // fp32, natural order, H not asked for: the Hessian is accumulated
  // straight into the factor's working copy, which is damped and factored
  // in place (no n x n copy)
  const bool in_place = has_x && !H_out && prec == PWQ_F32 &&
                        order_kind == PWQ_ORDER_BACK_TO_FRONT;
  float* Hm = has_x ? (H_out ? H_out : (in_place ? (float*)Lm : w.H)) : (float*)H;

  hipError_t e = launch_init_flags(w.flags, result, 1, st);
  if (e == hipSuccess && has_x) {
    SyrkPlan p;
    syrk_plan(n, ntok, xdtype, xal, &p);
    e = launch_hessian(Hm, n, X, xdtype, ntok, ldx, 0, p, w.partial, st);
  }
  const int32_t* colmap = nullptr;
  if (e == hipSuccess && mp) {
    // the order is taken on the damped matrix: lambda first
    e = launch_damp_lambda(Hm, n, damp, w.dead, result, w.flags, w.lam, st);
    // a failing pivot leaves the positions after it unwritten: start from
    // the identity so the map never holds workspace garbage
    if (e == hipSuccess) e = launch_identity_perm(w.perm, n, st);
    if (e == hipSuccess)
      e = launch_min_pivot(Hm, n, w.lam, w.mp, w.perm, nullptr, w.flags, result, st);
    colmap = w.perm;
  } else if (e == hipSuccess && order_kind != PWQ_ORDER_BACK_TO_FRONT) {
    e = launch_order(order_kind, Hm, n, perm, w.perm, w.seen, result, w.flags, st);
    colmap = order_kind == PWQ_ORDER_PERM ? perm : w.perm;
  }
  if (e == hipSuccess && in_place)
    e = launch_damp_cholesky_in_place((float*)Lm, n, damp, w.dead, result, w.flags, w.lam,
                                      w.dscratch, st);
  else if (e == hipSuccess)
    e = launch_damp_cholesky(Hm, n, damp, prec, colmap, Lm, w.dead, result, w.flags, w.lam,
                             w.dscratch, st);
  const bool colsp = grid->kind == PWQ_GRID_COLSPACING;
  const int G = colsp ? 1 : group_of(grid, n);
  if (e == hipSuccess && !colsp && m > 0)
    e = launch_grid_steps(W, wdtype, m, n, ldw, w.dead, grid->kind, grid->bits, G, scales,
                          zeros, w.flags, st, step_multiplier(grid));
  if (e == hipSuccess) {
    SweepLaunch sl{};
    sl.W = W; sl.wdtype = wdtype; sl.ldw = ldw; sl.m = m; sl.n = n; sl.prec = prec;
    sl.block = block; sl.L = Lm; sl.invd = w.sw.invd; sl.dg = w.sw.dg; sl.alpha = w.sw.alpha;
    sl.colspacing = colsp; sl.c = grid->c;
    sl.scales = scales; sl.scales_out = scales;
    sl.zeros = grid->kind == PWQ_GRID_ASYM ? zeros : nullptr;
    sl.G = G; sl.ng = (int)(n / G);
    sl.colmap = colmap; sl.dead = w.dead; sl.acc = w.sw.acc; sl.E = w.sw.E; sl.codes = codes;
    sl.partials = w.sw.partials; sl.result = result; sl.flags = w.flags;
    e = launch_sweep(sl, st);
  }
  if (e != hipSuccess) return hip_fail(e, "quant_layer launch");
  return ok();
}

size_t pwq_min_pivot_workspace_size(int64_t n) {
  if (n <= 0 || n > 65536) return 0;
  Carver c(nullptr);
  c.take(sizeof(DevFlags));
  c.take(sizeof(double));
  MinPivotWs w;
  carve_min_pivot(c, n, &w);
  return c.size();
}

pwq_status pwq_min_pivot_order(const float* H, int64_t n, double damp, int32_t* perm,
                               double* pivots, pwq_result* result, void* ws, size_t ws_bytes,
                               void* stream) {
  if (n <= 0 || n > 65536) return fail(PWQ_ERR_INVALID_ARG, "n must be in [1, 65536]");
  if (!H || !perm || !result)
    return fail(PWQ_ERR_INVALID_ARG, "H, perm and result must be non-NULL");
  if (!(damp >= 0.0) || !(damp < 1e30)) return fail(PWQ_ERR_INVALID_ARG, "damp must be >= 0");
  pwq_status s = check_ws(ws, ws_bytes, pwq_min_pivot_workspace_size(n));
  if (s != PWQ_OK) return s;
  Carver c(ws);
  DevFlags* flags = (DevFlags*)c.take(sizeof(DevFlags));
  double* lam = (double*)c.take(sizeof(double));
  MinPivotWs w;
  carve_min_pivot(c, n, &w);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_init_flags(flags, result, 1, st);
  if (e == hipSuccess) e = launch_damp_lambda(H, n, damp, nullptr, result, flags, lam, st);
  if (e == hipSuccess) e = launch_min_pivot(H, n, lam, w, perm, pivots, flags, result, st);
  if (e != hipSuccess) return hip_fail(e, "min_pivot_order launch");
  return ok();
}

static void carve_oaem(Carver& c, int64_t m, int64_t n, int32_t g, int32_t K, OaemWs* w) {
  const int64_t ng = n / g;
  w->Hb = (double*)c.take((size_t)ng * g * g * sizeof(double));
  w->R = (double*)c.take((size_t)m * n * sizeof(double));
  w->Q = (double*)c.take((size_t)ng * K * sizeof(double));
  w->S = (double*)c.take((size_t)ng * K * g * sizeof(double));
  w->cnt = (int32_t*)c.take((size_t)ng * K * 4);
  w->part = (double*)c.take((size_t)oaem_objective_parts(m, n, g) * sizeof(double));
}

static bool oaem_shape_ok(int64_t m, int64_t n, int32_t g, int32_t K) {
  return m >= 1 && n >= 1 && m <= INT32_MAX && n <= 65536 && g >= 1 && g <= kOaemMaxG &&
         n % g == 0 && K >= 1 && (int64_t)K * (g + 1) <= kOaemMaxLds &&
         m * (n / g) <= INT32_MAX;
}

size_t pwq_oaem_workspace_size(int64_t m, int64_t n, int32_t g, int32_t K) {
  if (!oaem_shape_ok(m, n, g, K)) return 0;
  Carver c(nullptr);
  c.take(sizeof(DevFlags));
  c.take(sizeof(double));
  OaemWs w;
  carve_oaem(c, m, n, g, K, &w);
  return c.size();
}

pwq_status pwq_oaem_init(const void* W, int32_t wdtype, int64_t m, int64_t n, int64_t ldw,
                         const float* H, double damp, int32_t g, int32_t K, int32_t M,
                         int32_t iters, const int64_t* seeds, double* codebooks, int32_t* codes,
                         double* objective, pwq_result* result, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!W || !H || !seeds || !codebooks || !codes || !result)
    return fail(PWQ_ERR_INVALID_ARG, "W, H, seeds, codebooks, codes and result must be non-NULL");
  if (wdtype != PWQ_F32 && wdtype != PWQ_BF16)
    return fail(PWQ_ERR_INVALID_ARG, "W dtype must be PWQ_F32 or PWQ_BF16");
  if (!oaem_shape_ok(m, n, g, K))
    return fail(PWQ_ERR_INVALID_ARG,
                "need m >= 1, 1 <= n <= 65536, 1 <= g <= %d dividing n, K >= 1 with "
                "K (g + 1) <= %d "
                "(got m %lld n %lld g %d K %d)", kOaemMaxG, kOaemMaxLds, (long long)m,
                (long long)n, g, K);
  if (ldw < n) return fail(PWQ_ERR_INVALID_ARG, "ldw < n");
  if (M < 1 || iters < 0) return fail(PWQ_ERR_INVALID_ARG, "need M >= 1 and iters >= 0");
  if (!(damp >= 0.0) || !(damp < 1e30)) return fail(PWQ_ERR_INVALID_ARG, "damp must be >= 0");
  pwq_status s = check_ws(ws, ws_bytes, pwq_oaem_workspace_size(m, n, g, K));
  if (s != PWQ_OK) return s;
  Carver c(ws);
  DevFlags* flags = (DevFlags*)c.take(sizeof(DevFlags));
  double* lam = (double*)c.take(sizeof(double));
  OaemWs w;
  carve_oaem(c, m, n, g, K, &w);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_init_flags(flags, result, 1, st);
  if (e == hipSuccess) e = launch_damp_lambda(H, n, damp, nullptr, result, flags, lam, st);
  if (e == hipSuccess)
    e = launch_oaem(W, wdtype, m, n, ldw, H, lam, g, K, M, iters, seeds, codebooks, codes,
                    objective, result, w, st);
  if (e != hipSuccess) return hip_fail(e, "oaem_init launch");
  return ok();
}

size_t pwq_rate_workspace_size(int64_t n) {
  if (n <= 0) return 0;
  Carver c(nullptr);
  c.take((size_t)n * 4);
  c.take((size_t)n * 4);
  return c.size();
}

pwq_status pwq_column_entropy(const int32_t* codes, int64_t m, int64_t n, int64_t ldc,
                              double* bits, double* mean, int64_t* huff, void* ws,
                              size_t ws_bytes, void* stream) {
  if (m < 0 || n < 0 || m > INT32_MAX || n > INT32_MAX)
    return fail(PWQ_ERR_INVALID_ARG, "m and n must be in [0, 2^31)");
  if (ldc < n) return fail(PWQ_ERR_INVALID_ARG, "ldc (%lld) < n (%lld)", (long long)ldc,
                           (long long)n);
  if (n > 0 && (!bits || (m > 0 && !codes)))
    return fail(PWQ_ERR_INVALID_ARG, "codes and bits must be non-NULL");
  pwq_status s = check_ws(ws, ws_bytes, pwq_rate_workspace_size(n));
  if (s != PWQ_OK) return s;
  Carver c(ws);
  int32_t* cmin = n > 0 ? (int32_t*)c.take((size_t)n * 4) : nullptr;
  int32_t* cmax = n > 0 ? (int32_t*)c.take((size_t)n * 4) : nullptr;
  const hipError_t e = launch_column_entropy(codes, m, n, ldc, bits, mean, huff, cmin, cmax,
                                             (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "column_entropy launch");
  return ok();
}

pwq_status pwq_kernel_timer_attach(int32_t kernel, void* const* starts, void* const* stops,
                                   int64_t capacity) {
  if (kernel < 0 || kernel >= kNumTimers)
    return fail(PWQ_ERR_INVALID_ARG, "unknown timed kernel %d", kernel);
  if (capacity < 0) return fail(PWQ_ERR_INVALID_ARG, "capacity must be >= 0");
  if (capacity > 0 && (!starts || !stops))
    return fail(PWQ_ERR_INVALID_ARG, "event arrays are NULL");
  KernelTimer& t = g_timers[kernel];
  t.starts = capacity ? (hipEvent_t*)starts : nullptr;
  t.stops = capacity ? (hipEvent_t*)stops : nullptr;
  t.capacity = capacity;
  t.used = 0;
  return ok();
}

int64_t pwq_kernel_timer_count(int32_t kernel) {
  return (kernel >= 0 && kernel < kNumTimers) ? g_timers[kernel].used : -1;
}

// ------------------------------------------------------------ SSQR outliers

size_t pwq_overflow_workspace_size(int64_t m) {
  if (m < 0) return 0;
  Carver c(nullptr);
  c.take((size_t)m * 4);
  c.take((size_t)m * 8);
  c.take(8);
  return c.size();
}

pwq_status pwq_overflow_entries(const int32_t* codes, int64_t m, int64_t n, int64_t ldc,
                                const pwq_grid* grid, const float* scales,
                                const int32_t* zeros, int64_t max_out, int32_t* rows,
                                int32_t* cols, float* vals, int64_t* count, void* ws,
                                size_t ws_bytes, void* stream) {
  if (m < 0 || n <= 0 || m > INT32_MAX || n > INT32_MAX)
    return fail(PWQ_ERR_INVALID_ARG, "bad m / n");
  if (m > 0 && (!codes || !scales)) return fail(PWQ_ERR_INVALID_ARG, "codes / scales NULL");
  if (m > 0 && ldc < n) return fail(PWQ_ERR_INVALID_ARG, "ldc < n");
  if (!count) return fail(PWQ_ERR_INVALID_ARG, "count is NULL");
  if (max_out < 0) return fail(PWQ_ERR_INVALID_ARG, "max_out must be >= 0");
  if (max_out > 0 && (!rows || !cols || !vals))
    return fail(PWQ_ERR_INVALID_ARG, "rows / cols / vals NULL");
  pwq_status s = check_grid(grid, n, false);
  if (s != PWQ_OK) return s;
  if (grid->kind == PWQ_GRID_ASYM && !zeros)
    return fail(PWQ_ERR_INVALID_ARG, "ASYM grid needs zeros");
  s = check_ws(ws, ws_bytes, pwq_overflow_workspace_size(m));
  if (s != PWQ_OK) return s;
  Carver c(ws);
  int32_t* rc = (int32_t*)c.take((size_t)m * 4);
  int64_t* ro = (int64_t*)c.take((size_t)m * 8);
  (void)c.take(8);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = launch_overflow_count(codes, m, n, ldc, grid->kind, grid->bits, rc, ro, count, st);
  if (e == hipSuccess)
    e = launch_overflow_write(codes, m, n, ldc, grid->kind, grid->bits, scales,
                              grid->kind == PWQ_GRID_ASYM ? zeros : nullptr, group_of(grid, n),
                              ro, max_out, rows, cols, vals, st);
  if (e != hipSuccess) return hip_fail(e, "overflow launch");
  return ok();
}

size_t pwq_ssqr_workspace_size(int64_t m, int64_t n, int64_t ntok, int32_t has_x, int32_t block,
                               int32_t prec) {
  if (m < 0 || n <= 0 || !valid_block(block)) return 0;
  Carver c(nullptr);
  if (has_x) c.take((size_t)n * n * 4);                               // H
  c.take((size_t)n * n * elem(prec));                                 // L
  c.take((size_t)n * 4);                                              // dead flags
  size_t inner = pwq_sweep_workspace_size(m, n, block, prec);
  inner = std::max(inner, pwq_cholesky_workspace_size(n, prec));
  if (has_x) inner = std::max(inner, pwq_hessian_workspace_size(n, ntok));
  c.take(inner);
  c.take(pwq_overflow_workspace_size(m));
  return c.size();
}

pwq_status pwq_ssqr_quant_layer(const void* W, int32_t wdtype, int64_t m, int64_t n,
                                int64_t ldw, const void* X, int32_t xdtype, int64_t ntok,
                                int64_t ldx, const float* H, const pwq_grid* grid, double damp,
                                int32_t block, int32_t prec, double density, int32_t iters,
                                double log2_lo, int32_t* codes, float* scales, int32_t* zeros,
                                pwq_result* result, int64_t max_out, int32_t* rows,
                                int32_t* cols, float* vals, int64_t* n_out, double* kappa,
                                void* ws, size_t ws_bytes, void* stream) {
  if (!grid || (grid->kind != PWQ_GRID_SYM && grid->kind != PWQ_GRID_ASYM))
    return fail(PWQ_ERR_INVALID_ARG, "SSQR needs a SYM or ASYM grid");
  if (!(density >= 0.0) || !(density <= 1.0))
    return fail(PWQ_ERR_INVALID_ARG, "density must be in [0, 1]");
  if (iters < 0 || iters > 60) return fail(PWQ_ERR_INVALID_ARG, "iters must be in [0, 60]");
  if (!(log2_lo < 0.0) || !(log2_lo >= -60.0))
    return fail(PWQ_ERR_INVALID_ARG, "log2_lo must be in [-60, 0)");
  if (!n_out || !kappa) return fail(PWQ_ERR_INVALID_ARG, "n_out / kappa NULL");
  if (max_out < 0 || (max_out > 0 && (!rows || !cols || !vals)))
    return fail(PWQ_ERR_INVALID_ARG, "bad outlier arrays");
  const bool has_x = X != nullptr;
  if (has_x == (H != nullptr)) return fail(PWQ_ERR_INVALID_ARG, "give exactly one of X and H");
  if (m <= 0 || n <= 0) return fail(PWQ_ERR_INVALID_ARG, "m and n must be positive");
  if (!valid_block(block)) return fail(PWQ_ERR_UNSUPPORTED, "block must be 32, 64, 128 or 256");
  pwq_status s = check_ws(ws, ws_bytes, pwq_ssqr_workspace_size(m, n, ntok, has_x, block, prec));
  if (s != PWQ_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  Carver c(ws);
  float* Hw = has_x ? (float*)c.take((size_t)n * n * 4) : nullptr;
  void* L = c.take((size_t)n * n * elem(prec));
  int32_t* dead = (int32_t*)c.take((size_t)n * 4);
  size_t inner = pwq_sweep_workspace_size(m, n, block, prec);
  inner = std::max(inner, pwq_cholesky_workspace_size(n, prec));
  if (has_x) inner = std::max(inner, pwq_hessian_workspace_size(n, ntok));
  void* iws = c.take(inner);
  int32_t* rc = (int32_t*)c.take((size_t)m * 4);
  int64_t* ro = (int64_t*)c.take((size_t)m * 8);
  int64_t* tot = (int64_t*)c.take(8);
  // The Hessian and its factor do not depend on the steps: once.
  if (has_x) {
    s = pwq_hessian_accum(Hw, n, X, xdtype, ntok, ldx, 0, iws, inner, stream);
    if (s != PWQ_OK) return s;
  }
  s = pwq_damp_cholesky(has_x ? Hw : H, n, damp, prec, L, dead, result, iws, inner, stream);
  if (s != PWQ_OK) return s;
  pwq_result r0;
  hipError_t e = hipMemcpyAsync(&r0, result, sizeof(r0), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "ssqr factor");
  if (r0.info != 0) {               // the factorization failed: result->info says where
    *n_out = 0;
    *kappa = 1.0;
    return ok();
  }
  const int64_t target = (int64_t)std::floor(density * (double)m * (double)n);
  // steps at multiplier k, the sweep, and its outlier count (on the host)
  double last = -1.0;
  auto evaluate = [&](double k, int64_t* cnt) -> pwq_status {
    pwq_grid g = *grid;
    g.kappa = k;
    pwq_status q = pwq_grid_steps(W, wdtype, m, n, ldw, dead, &g, scales, zeros, stream);
    if (q != PWQ_OK) return q;
    q = pwq_babai_sweep(W, wdtype, m, n, ldw, L, prec, dead, &g, scales, zeros, block, codes,
                        result, iws, inner, stream);
    if (q != PWQ_OK) return q;
    hipError_t he = launch_overflow_count(codes, m, n, n, grid->kind, grid->bits, rc, ro, tot, st);
    int64_t t = 0;
    if (he == hipSuccess) he = hipMemcpyAsync(&t, tot, 8, hipMemcpyDeviceToHost, st);
    if (he == hipSuccess) he = hipStreamSynchronize(st);
    if (he != hipSuccess) return hip_fail(he, "ssqr evaluation");
    last = k;
    *cnt = t;
    return PWQ_OK;
  };
  // the multiplier as float32 of 2^x (what the step kernel multiplies by)
  auto kap = [](double x) { return (double)(float)std::exp2(x); };
  int64_t cnt = 0;
  double lo = log2_lo, hi = 0.0, res_k = 1.0;
  s = evaluate(kap(hi), &cnt);
  if (s != PWQ_OK) return s;
  if (cnt <= target) {
    s = evaluate(kap(lo), &cnt);
    if (s != PWQ_OK) return s;
    if (cnt <= target) {
      res_k = kap(lo);
    } else {
      for (int i = 0; i < iters; ++i) {
        const double mid = 0.5 * (lo + hi);
        s = evaluate(kap(mid), &cnt);
        if (s != PWQ_OK) return s;
        if (cnt <= target) hi = mid;
        else lo = mid;
      }
      res_k = kap(hi);
    }
  }
  if (last != res_k) {              // leave the outputs at the chosen multiplier
    s = evaluate(res_k, &cnt);
    if (s != PWQ_OK) return s;
  }
  e = launch_overflow_write(codes, m, n, n, grid->kind, grid->bits, scales,
                            grid->kind == PWQ_GRID_ASYM ? zeros : nullptr, group_of(grid, n),
                            ro, max_out, rows, cols, vals, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "ssqr outliers");
  *n_out = cnt;
  *kappa = res_k;
  return ok();
}

}  // extern "C"
