/*
 * pwq.h -- C ABI of libpwq: Hessian-weighted sequential quantization of one
 * linear layer on an MI355X (gfx950), read as Babai's nearest-plane algorithm.
 *
 * Pages defining the operations (cited by title and section):
 *   [GEOM] "The Geometry of LLM Quantization: GPTQ as Babai's Nearest Plane
 *          Algorithm", technical summary 1 (problem), 2.1 (closest-vector
 *          form, basis X diag(s), Theorem 1), 2.2 (back-to-front GPTQ =
 *          Babai, Theorem 4), 2.3 (no clipping, Theorem 5, pivot order).
 *   [WSIC] "WaterSIC: information-theoretically (near) optimal linear layer
 *          quantization", technical summary 1 (objective) and 2 (Cholesky
 *          Sigma = L L^T, last column first with interference cancellation,
 *          spacing alpha_i = c/|l_ii|, dead-feature erasure).
 *   [OAEM] "Initialisation Determines the Basin: Efficient Codebook
 *          Optimisation for Extreme LLM Quantization", section 3 (damped
 *          Hessian X^T X + lambda I).
 *
 * Conventions for every entry point
 *   - Matrices are row-major.  W is m x n (d_out x d_in), row stride ldw
 *     elements.  X is n x ntok (channels x tokens, tokens contiguous), row
 *     stride ldx elements.  H and L are n x n with row stride n.
 *   - Every pointer except `grid` and the returned strings is a DEVICE
 *     pointer owned by the caller.  The library allocates nothing: scratch
 *     memory is the caller's workspace `ws` of `ws_bytes` bytes (ask the
 *     matching *_workspace_size function), 256-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and the call returns without synchronising.
 *   - Argument errors are reported synchronously, before anything is
 *     enqueued, as a pwq_status (details: pwq_last_error()).  A numerical
 *     failure on the device (Cholesky of a matrix that is not positive
 *     definite) is written to result->info, LAPACK-potrf style: 0 = success,
 *     k > 0 = the leading minor of order k is not positive definite; the
 *     codes, steps and losses are then undefined.  NaN/Inf pivots also
 *     report info = k.
 *   - Same inputs and arguments give bitwise-identical outputs (no float
 *     atomics; every reduction has a fixed order).
 *   - Calls with distinct workspaces may run concurrently on distinct streams.
 */
#ifndef PWQ_H
#define PWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PWQ_OK = 0,
  PWQ_ERR_INVALID_ARG = 1,   /* bad pointer, size, enum or combination      */
  PWQ_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement */
  PWQ_ERR_WORKSPACE = 3,     /* ws NULL, misaligned or smaller than needed  */
  PWQ_ERR_HIP = 4            /* a HIP runtime call failed                   */
} pwq_status;

/* Element types of W and X (PWQ_F32/PWQ_BF16) and the precision of the
 * factor / running target / sweep (PWQ_F32 or PWQ_F64). */
typedef enum { PWQ_F32 = 0, PWQ_BF16 = 1, PWQ_F64 = 2 } pwq_dtype;

/* Layout flag OR'ed into the X dtype (xdtype) of pwq_hessian_accum and
 * pwq_quant_layer: X is stored ntok x n, one row per token with the n
 * channels contiguous (row stride ldx >= n), the layout in which a layer's
 * input activations are usually captured.  Without it X is n x ntok (row
 * stride ldx >= ntok).  Both describe the same matrix X and give the same H. */
enum { PWQ_X_TOKEN_MAJOR = 0x100 };

/* Quantization grid.  The lattice of one row is s * Z per column (no
 * clipping: codes are any int32) [GEOM 2.1, 2.3].
 *   SYM        : s = max|w| / (2^(bits-1) - 1) over each group of
 *                `group_size` consecutive columns of a row (0 = whole row);
 *                stored code = lattice integer.
 *   ASYM       : lo = min(min w, 0), hi = max(max w, 0),
 *                s = (hi - lo) / (2^bits - 1), zero point z0 = rint(-lo/s);
 *                stored code = lattice integer + z0.
 *   COLSPACING : one spacing per column, alpha_k = c / l_kk of the Cholesky
 *                factor [WSIC 2]; stored code = lattice integer.
 * Steps are taken from W (after dead-feature erasure) before the sweep; a
 * zero step becomes 1.  bits in [2, 16] for SYM/ASYM; c > 0 for COLSPACING.
 * Each field belongs to one family of kinds; the other family's field must
 * be 0 (a call that sets it is rejected with PWQ_ERR_INVALID_ARG). */
typedef enum { PWQ_GRID_SYM = 0, PWQ_GRID_ASYM = 1, PWQ_GRID_COLSPACING = 2 } pwq_grid_kind;
typedef struct {
  int32_t kind;        /* pwq_grid_kind                                   */
  int32_t bits;        /* SYM / ASYM                                      */
  int32_t group_size;  /* SYM / ASYM: 0 = one step per row; else divides n */
  int32_t reserved;    /* must be 0                                       */
  double c;            /* COLSPACING only: alpha_k = c / l_kk, finite > 0 */
  double kappa;        /* SYM / ASYM only: a multiplier on every step,    */
                       /* applied in float32 after the step rule (the     */
                       /* asymmetric zero point uses the scaled step);    */
                       /* 0 means none, else finite > 0.  [GEOM 3: SSQR   */
                       /* adjusts the scale to a target outlier density]  */
} pwq_grid;

/* Processing order.  Position k of the permuted problem holds original
 * column perm[k]; positions are processed from n-1 down to 0 [GEOM 2.2].
 *   BACK_TO_FRONT : perm = identity (Babai's natural order)
 *   FRONT_TO_BACK : perm = reversal (standard GPTQ order)
 *   PERM          : caller's device int32 permutation of 0..n-1
 *   ACT_ORDER     : largest diag(H) processed first, ties by lower index
 *                   [GEOM 2.3]
 *   MIN_PIVOT     : the min-pivot order of the damped Hessian (see
 *                   pwq_min_pivot_order) [GEOM 2.3] */
typedef enum {
  PWQ_ORDER_BACK_TO_FRONT = 0,
  PWQ_ORDER_FRONT_TO_BACK = 1,
  PWQ_ORDER_PERM = 2,
  PWQ_ORDER_ACT = 3,
  PWQ_ORDER_MIN_PIVOT = 4
} pwq_order_kind;

/* Device-resident result record (read after a stream synchronisation).
 *   loss        = tr((W - W^) H (W - W^)^T), undamped H [WSIC 1]
 *   loss_damped = the same with H + lambda I; equals sum rho^2 s^2 l_kk^2
 *   bound       = (1/4) sum s^2 l_kk^2, Theorem 5 of [GEOM 2.3]
 *   delta_sq    = ||W - W^||_F^2
 *   lambda      = damp * mean(diag H) after dead-feature erasure [OAEM 3]
 *   info        = 0, or the order of the failing leading minor
 *   ndead       = number of zero-variance inputs erased [WSIC 2]        */
typedef struct {
  double loss;
  double loss_damped;
  double bound;
  double delta_sq;
  double lambda;
  int32_t info;
  int32_t ndead;
  int32_t reserved[2];
} pwq_result;

/* Human-readable name of a status. Never NULL. */
const char* pwq_status_string(pwq_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* pwq_last_error(void);

/* ---------------------------------------------------------------------- *
 * Stage 1: H (+)= 2 X X^T  [GEOM 2.1: the lattice comes from the
 * calibration inputs; WSIC 1: output error of Y = W X].
 *   H        : n x n float32, full symmetric result (both triangles
 *              written; with accumulate != 0 the previous H is added).
 *   X        : n x ntok, xdtype PWQ_BF16 or PWQ_F32, row stride ldx >= ntok;
 *              or, with xdtype | PWQ_X_TOKEN_MAJOR, stored ntok x n with row
 *              stride ldx >= n.
 *   Products are exact in fp32 for bf16 inputs; accumulation is fp32 in a
 *   fixed order.  Calling it once per calibration chunk with accumulate = 1
 *   streams the Hessian over any number of tokens.
 * ---------------------------------------------------------------------- */
size_t pwq_hessian_workspace_size(int64_t n, int64_t ntok);
pwq_status pwq_hessian_accum(float* H, int64_t n, const void* X, int32_t xdtype,
                             int64_t ntok, int64_t ldx, int32_t accumulate,
                             void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------- *
 * Stage 2+3: dead features, damping, Cholesky [WSIC 2; OAEM 3; GEOM 2.1].
 *   H      : n x n float32 (lower triangle read).
 *   L      : n x n output in precision `prec` (PWQ_F32 -> float,
 *            PWQ_F64 -> double): lower factor of H_d = H' + lambda I where
 *            H' is H with H_kk = 1 for every k with H_kk == 0; the strict
 *            upper triangle is written with zeros.
 *   dead   : optional int32 [n] output, 1 where H_kk == 0 (erased input).
 *   result : lambda, ndead and info are written (losses are not).
 * ---------------------------------------------------------------------- */
size_t pwq_cholesky_workspace_size(int64_t n, int32_t prec);
pwq_status pwq_damp_cholesky(const float* H, int64_t n, double damp, int32_t prec,
                             void* L, int32_t* dead, pwq_result* result,
                             void* ws, size_t ws_bytes, void* stream);

/* pwq_damp_cholesky without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Arguments and results as for pwq_damp_cholesky;
 * it calls no allocating routine.  Its scratch (status flags, lambda and the
 * side buffer of diagonal blocks: 68 KB at most, whatever n) is a static
 * device array of the library; each GPU the library runs on holds one copy
 * until the process ends.  Every call on a GPU uses that GPU's copy, so calls
 * that overlap on one GPU (on different streams, or from different threads)
 * race: serialise them.  A size that would need more scratch than the array
 * holds is rejected with PWQ_ERR_WORKSPACE before anything is enqueued. */
pwq_status pwq_damp_cholesky_static(const float* H, int64_t n, double damp, int32_t prec,
                                    void* L, int32_t* dead, pwq_result* result, void* stream);

/* ---------------------------------------------------------------------- *
 * Steps for SYM / ASYM grids from W [GEOM 2.1: fixed basis X diag(s)].
 *   scales : m x (n / G) float32 (G = group_size, or n when 0)
 *   zeros  : m x (n / G) int32 for ASYM, ignored (may be NULL) otherwise.
 *   dead   : optional int32 [n]; flagged columns count as zero weights.
 * ---------------------------------------------------------------------- */
pwq_status pwq_grid_steps(const void* W, int32_t wdtype, int64_t m, int64_t n,
                          int64_t ldw, const int32_t* dead, const pwq_grid* grid,
                          float* scales, int32_t* zeros, void* stream);

/* ---------------------------------------------------------------------- *
 * Stage 4: the back-to-front nearest-plane sweep with lazy block updates,
 * given a factor [GEOM 2.2, Theorem 4; WSIC 2].  Columns are processed in
 * natural order (n-1 first).  For column k, with running target
 * w~_k = w_k + sum_{j>k} (l_jk / l_kk) e_j:
 *     z = rint(w~_k / s)  (half to even),  e_k = w_k - s z,
 * where e is the ORIGINAL weight minus the dequantized weight.
 *   W      : m x n (wdtype), L : n x n lower in `prec` (as written by
 *            pwq_damp_cholesky).  dead: optional int32 [n] flags; columns
 *            flagged non-zero are treated as zero weights.
 *   scales : SYM/ASYM: input, as written by pwq_grid_steps.
 *            COLSPACING: output, float32 [n], alpha_k = c / l_kk.
 *   zeros  : ASYM input zero points (added to the stored codes).
 *   codes  : m x n int32 output (row stride n).
 *   result : loss_damped, bound, delta_sq written; loss = loss_damped -
 *            lambda * delta_sq uses result->lambda as found on entry.
 *   block  : lazy-update block size, one of 32, 64, 128, 256.
 * ---------------------------------------------------------------------- */
size_t pwq_sweep_workspace_size(int64_t m, int64_t n, int32_t block, int32_t prec);
pwq_status pwq_babai_sweep(const void* W, int32_t wdtype, int64_t m, int64_t n,
                           int64_t ldw, const void* L, int32_t prec,
                           const int32_t* dead, const pwq_grid* grid,
                           float* scales, const int32_t* zeros, int32_t block,
                           int32_t* codes, pwq_result* result,
                           void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------- *
 * The whole layer: quant_layer(W, X or H, grid, order, damp) ->
 * codes + steps + proxy loss [GEOM 1, 2.1-2.3; WSIC 1-2; OAEM 3].
 *   Exactly one of X (n x ntok, xdtype, layout as for pwq_hessian_accum)
 *   and H (n x n float32) is non-NULL.
 *   order_kind : pwq_order_kind; perm (device int32 [n]) only for PERM.
 *   damp       : lambda = damp * mean(diag H) (0 for none).
 *   block      : 32, 64, 128 or 256.   prec : PWQ_F32 or PWQ_F64.
 *   codes      : m x n int32 in ORIGINAL column order (row stride n).
 *   scales     : SYM/ASYM m x (n/G) float32; COLSPACING [n] float32 per
 *                original column.
 *   zeros      : m x (n/G) int32 for ASYM, else ignored.
 *   result     : every field written.
 *   H_out      : optional n x n float32 copy of H = 2 X X^T (X given only).
 *   L_out      : optional n x n factor (precision prec) of the PERMUTED
 *                damped Hessian.
 *   The workspace depends on order_kind: MIN_PIVOT adds the n x n fp64
 *   matrix of pwq_min_pivot_order.
 * ---------------------------------------------------------------------- */
size_t pwq_quant_layer_workspace_size(int64_t m, int64_t n, int64_t ntok,
                                      int32_t has_x, int32_t order_kind,
                                      int32_t block, int32_t prec);
pwq_status pwq_quant_layer(const void* W, int32_t wdtype, int64_t m, int64_t n,
                           int64_t ldw, const void* X, int32_t xdtype,
                           int64_t ntok, int64_t ldx, const float* H,
                           const pwq_grid* grid, int32_t order_kind,
                           const int32_t* perm, double damp, int32_t block,
                           int32_t prec, int32_t* codes, float* scales,
                           int32_t* zeros, pwq_result* result, float* H_out,
                           void* L_out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------- *
 * Min-pivot order [GEOM 2.3: the Theorem 5 bound is (1/4) s^T D s with D
 * the LDL pivots of the permuted Hessian; taking the smallest diagonal
 * entry at each LDL step lowers trace D].  A diagonally pivoted LDL^T of
 * H_d = H' + lambda I, H' = H with erased inputs (H_ii = 0) set to 1,
 * lambda = damp * mean(diag H') (the damped matrix of pwq_quant_layer):
 * step k takes the column not yet chosen whose Schur-complement diagonal
 * is smallest (ties: lower column index; NaN counts as smallest) and puts
 * it at position k, so position 0 is processed LAST by the back-to-front
 * sweep.  Computed in float64.
 *   H      : n x n float32 device, lower triangle read; 1 <= n <= 65536.
 *   perm   : n int32 device out: perm[k] = column of position k.
 *   pivots : optional n float64 device out: D_kk (NULL to skip).
 *   result : device; info = 0, or k + 1 when pivot k is not positive (then
 *            perm and pivots are undefined from position k on); lambda and
 *            ndead written; the other fields untouched.
 *   ws     : pwq_min_pivot_workspace_size(n) bytes (n x n float64 inside).
 * One launch per pivot: the time grows with n launches.
 * ---------------------------------------------------------------------- */
size_t pwq_min_pivot_workspace_size(int64_t n);
pwq_status pwq_min_pivot_order(const float* H, int64_t n, double damp,
                               int32_t* perm, double* pivots,
                               pwq_result* result, void* ws, size_t ws_bytes,
                               void* stream);

/* ---------------------------------------------------------------------- *
 * OA-EM codebook initialisation [OAEM 3: inside AQLM's residual framework
 * each codebook is initialised by EM; the M-step moves the centroids to
 * minimise the output reconstruction error weighted by
 * H_i = X_i^T X_i + lambda I, the E-step reassigns every weight group to
 * its nearest centroid in that Mahalanobis distance].
 *   A weight group is g consecutive inputs of one output row,
 *   w_{r,i} = W[r, i g .. i g + g), i < n / g; its metric H_i is the g x g
 *   diagonal block of the damped Hessian H_d = H' + lambda I (erased inputs
 *   and lambda as in pwq_quant_layer).  Stage t < M fits K centroids to the
 *   residual left by stages 0..t-1: initial centroid k is the residual group
 *   seeds[t K + k] (index r (n/g) + i, chosen by the caller); `iters` rounds
 *   of E-step (argmin_k (w - c_k)^T H_i (w - c_k), ties to the lower k) and
 *   M-step (c_k = (sum H_i)^{-1} sum H_i w over the groups assigned to k; a
 *   centroid with no group keeps its value), then a final E-step gives the
 *   stage's codes and the residual loses the chosen centroids.  float64.
 *   W          : m x n float32 or bfloat16 (row stride ldw >= n), device.
 *   H          : n x n float32 device, lower triangle read (undamped);
 *                1 <= n <= 65536, m (n / g) < 2^31.
 *   g, K       : 1 <= g <= 16 dividing n; K >= 1 with K (g + 1) <= 8192.
 *   seeds      : M x K int64 device; an index outside [0, m n / g) sets
 *                result->info = -1 (group 0 is used).
 *   codebooks  : M x K x g float64 device out.
 *   codes      : M x m x (n/g) int32 device out (codes[t][r][i]).
 *   objective  : optional M float64 device out: sum over groups of
 *                e^T H_i e for the residual e after each stage (NULL: skip).
 *   result     : device; info = 0 or -1, lambda and ndead written.
 *   ws         : pwq_oaem_workspace_size(m, n, g, K) bytes (0 for an
 *                unsupported shape).
 * ---------------------------------------------------------------------- */
size_t pwq_oaem_workspace_size(int64_t m, int64_t n, int32_t g, int32_t K);
pwq_status pwq_oaem_init(const void* W, int32_t wdtype, int64_t m, int64_t n,
                         int64_t ldw, const float* H, double damp, int32_t g,
                         int32_t K, int32_t M, int32_t iters,
                         const int64_t* seeds, double* codebooks,
                         int32_t* codes, double* objective,
                         pwq_result* result, void* ws, size_t ws_bytes,
                         void* stream);

/* ---------------------------------------------------------------------- *
 * Rate: the empirical Shannon entropy of each column's codes, in bits
 * [WSIC 2, items 1 and 3: columns get unequal rates and the unclipped codes
 * are entropy coded, so a column's rate is the entropy of its codes], and
 * optionally their Huffman-coded length [GEOM 3, HPTQ: the unconstrained
 * integer codes are Huffman coded].
 *   codes : m x n int32, row stride ldc >= n (as written by pwq_quant_layer
 *           or pwq_babai_sweep; zero points make no difference).
 *   bits  : n doubles: bits[k] = -sum_v p_v log2 p_v over the distinct
 *           values v of column k, p_v = (count of v) / m; 0 when m = 0;
 *           NaN for a column whose codes span more than 32768 values when
 *           m > 16384.
 *   mean  : optional double: the mean of bits over the n columns.
 *   huff  : optional n int64: total length in bits of column k's m codes
 *           under a Huffman code built for that column (codebook not
 *           counted; one distinct value costs 0); -1 where not computed (a
 *           span above 32768 values with m > 16384, or more than 16385
 *           distinct values in a column spanning 513 to 32768 values).
 *   ws    : pwq_rate_workspace_size(n) bytes.
 * Counts are exact (integer), and the sums run in a fixed order; the
 * Huffman totals are exact integers (every optimal prefix code of the same
 * counts has the same total).
 * ---------------------------------------------------------------------- */
size_t pwq_rate_workspace_size(int64_t n);
pwq_status pwq_column_entropy(const int32_t* codes, int64_t m, int64_t n, int64_t ldc,
                              double* bits, double* mean, int64_t* huff, void* ws,
                              size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------- *
 * Overflow-tolerant steps (SSQR) [GEOM 3: a few outlier weights are kept at
 * full precision as sparse floating-point values, the rest quantized at
 * low bit width; a binary search adjusts the scale to meet a target outlier
 * density].  Reading: the sweep never clips [GEOM 2.3], so a stored code
 * may fall outside the b-bit range (SYM: -2^(b-1) .. 2^(b-1)-1, ASYM:
 * 0 .. 2^b-1); those entries are the outliers, listed as (row, column,
 * value = float32(step * (code - zero point))) sorted by row, then column.
 *
 * pwq_overflow_entries: the list for given codes.
 *   codes   : m x n int32, row stride ldc >= n; scales / zeros as written by
 *             pwq_grid_steps or pwq_quant_layer for `grid` (SYM or ASYM).
 *   rows, cols, vals : device arrays of max_out entries; the first
 *             min(count, max_out) entries of the list are written.
 *   count   : device int64: the number of outliers (may exceed max_out).
 *   ws      : pwq_overflow_workspace_size(m) bytes.
 *
 * pwq_ssqr_quant_layer: the whole layer with the scale search.  H (from X,
 * or given), the damping and the factor are computed once; the layer is
 * then quantized as by pwq_quant_layer (back-to-front) at step multiplier
 * kappa (the grid's step multiplier: steps, then the sweep; the caller's
 * grid->kappa is ignored), and log2 kappa is bisected in
 * [log2_lo, 0]: kappa = 1 is tried first (if its outlier count already
 * exceeds floor(density m n) it is kept), then 2^log2_lo (kept if it meets
 * the target), then `iters` halvings of the bracket; the result is the
 * upper end of the final bracket (kappa = float32(2^x)).  On return codes,
 * scales, zeros and result hold the quantization at that kappa and
 * rows / cols / vals its outliers (as above).
 *   density : target fraction of outliers, in [0, 1].
 *   n_out   : host int64: the number of outliers at the chosen kappa.
 *   kappa   : host double: the chosen multiplier.
 *   ws      : pwq_ssqr_workspace_size(m, n, ntok, X != NULL, block, prec).
 * Synchronous: the stream is synchronised after every quantization (the
 * search needs each count on the host).  A failed factorization stops the
 * search with kappa = 1, n_out = 0 and result->info set.
 * ---------------------------------------------------------------------- */
size_t pwq_overflow_workspace_size(int64_t m);
pwq_status pwq_overflow_entries(const int32_t* codes, int64_t m, int64_t n, int64_t ldc,
                                const pwq_grid* grid, const float* scales,
                                const int32_t* zeros, int64_t max_out, int32_t* rows,
                                int32_t* cols, float* vals, int64_t* count, void* ws,
                                size_t ws_bytes, void* stream);
size_t pwq_ssqr_workspace_size(int64_t m, int64_t n, int64_t ntok, int32_t has_x,
                               int32_t block, int32_t prec);
pwq_status pwq_ssqr_quant_layer(const void* W, int32_t wdtype, int64_t m, int64_t n,
                                int64_t ldw, const void* X, int32_t xdtype, int64_t ntok,
                                int64_t ldx, const float* H, const pwq_grid* grid, double damp,
                                int32_t block, int32_t prec, double density, int32_t iters,
                                double log2_lo, int32_t* codes, float* scales, int32_t* zeros,
                                pwq_result* result, int64_t max_out, int32_t* rows,
                                int32_t* cols, float* vals, int64_t* n_out, double* kappa,
                                void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------- *
 * Kernel timing hook (measurement only; no effect on any result).
 * Attaches caller-owned HIP events (hipEvent_t handles) to one kernel:
 * after attach, launch i (i = 0 .. capacity-1) of that kernel records
 * starts[i] immediately before and stops[i] immediately after itself on
 * the stream it is launched on; later launches are not recorded.
 *   kernel   : PWQ_TIMER_HESSIAN_TILES = the Hessian product kernel (the
 *              bf16/fp32 SYRK tiles of pwq_hessian_accum and of
 *              pwq_quant_layer, without the split-K reduction);
 *              PWQ_TIMER_LAZY_UPDATE = one lazy block update of the sweep
 *              (acc[:, cols] += E[:, blk] L[blk, cols]; one pair per update,
 *              which may be several launches of the update kernel);
 *              PWQ_TIMER_SWEEP_BLOCK = one launch of the column sweep of a
 *              block (at most 128 columns) over all rows.
 *   capacity : number of event pairs; 0 (with NULL arrays) detaches.
 * The kernels are timed independently; several may be attached at once.
 * The arrays must stay valid until detach.  Process-wide state, not
 * thread safe: attach, run, synchronise, detach from one thread.
 * pwq_kernel_timer_count returns the pairs recorded for `kernel` since its
 * last attach (-1 for an unknown kernel).
 * ---------------------------------------------------------------------- */
typedef enum {
  PWQ_TIMER_HESSIAN_TILES = 0,
  PWQ_TIMER_LAZY_UPDATE = 1,
  PWQ_TIMER_SWEEP_BLOCK = 2
} pwq_timed_kernel;
pwq_status pwq_kernel_timer_attach(int32_t kernel, void* const* starts, void* const* stops,
                                   int64_t capacity);
int64_t pwq_kernel_timer_count(int32_t kernel);

#ifdef __cplusplus
}
#endif

#endif /* PWQ_H */
