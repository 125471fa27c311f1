"""MI355X-native Hessian-weighted sequential layer quantization.

GPTQ read as Babai's nearest-plane algorithm ("The Geometry of LLM
Quantization: GPTQ as Babai's Nearest Plane Algorithm", technical summary
2.1-2.3) and its successive-interference-cancellation form with per-column
spacing ("WaterSIC: information-theoretically (near) optimal linear layer
quantization", technical summary 2), behind the C ABI of ``libpwq.so``
(``include/pwq.h``).  These wrappers only marshal torch tensors (device
memory) and the current stream into that ABI; the HIP kernels do all the
work and there is no CPU fallback.
"""
import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import PwqError, check, lib, make_grid, parse_result

__all__ = ["Grid", "hessian_accum", "damp_cholesky", "damp_cholesky_static", "grid_steps", "babai_sweep",
           "quant_layer", "column_entropy", "read_result", "PwqError", "KernelTimer",
           "HessianTileTimer", "overflow_entries", "ssqr_quant_layer"]


@dataclass(frozen=True)
class Grid:
    kind: str = "sym"       # "sym" | "asym" | "colspacing"
    bits: int = 4
    group: int = 0          # 0 = one step per row
    c: float = 0.0          # colspacing constant (alpha_k = c / l_kk); colspacing only
    kappa: float = 0.0      # step multiplier (0 = none); sym / asym only

    def c_struct(self):
        return make_grid(self.kind, self.bits, self.group, self.c, self.kappa)


def _stream():
    return torch.cuda.current_stream().cuda_stream or None


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return _lib.PWQ_F32
    if t.dtype == torch.bfloat16:
        return _lib.PWQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _prec(prec: str) -> int:
    return {"f32": _lib.PWQ_F32, "f64": _lib.PWQ_F64}[prec]


def _tdt(prec: str):
    return torch.float64 if prec == "f64" else torch.float32


def _require_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must be on the GPU")


def _row_major(t: torch.Tensor) -> int:
    """Row stride (elements) of a 2-D row-major tensor.  A single row may
    carry any stride in torch; its row stride is then its length."""
    if t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1):
        raise ValueError("expected a 2-D tensor with unit column stride")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1]


def _check(t: Optional[torch.Tensor], name: str, shape, dtypes):
    """A tensor handed to the library as a raw pointer must have exactly the
    shape, element type and (contiguous, row-major) layout the C ABI reads."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_F32 = (torch.float32,)
_I32 = (torch.int32,)


def _check_result(res: Optional[torch.Tensor]):
    if res is None:
        return
    if res.dtype != torch.uint8 or res.numel() < _lib.RESULT_BYTES or not res.is_contiguous():
        raise ValueError(f"result must be a contiguous uint8 tensor of >= {_lib.RESULT_BYTES} "
                         "bytes (see new_result)")


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def new_result(device) -> torch.Tensor:
    return torch.zeros(_lib.RESULT_BYTES, dtype=torch.uint8, device=device)


def read_result(res: torch.Tensor) -> dict:
    """Synchronising read of a device result record."""
    return parse_result(bytes(res.cpu().numpy().tobytes()))


def _x_args(X: torch.Tensor, x_layout: str):
    """(n, ntok, ldx, xdtype) of activations X: ``x_layout`` "channels" for
    X [n, ntok], "tokens" for X [ntok, n] (one row per token)."""
    ldx = _row_major(X)
    if x_layout == "channels":
        n, ntok = X.shape
        return n, ntok, ldx, _dtype_code(X)
    if x_layout == "tokens":
        ntok, n = X.shape
        return n, ntok, ldx, _dtype_code(X) | _lib.PWQ_X_TOKEN_MAJOR
    raise ValueError(f"x_layout must be 'channels' or 'tokens', not {x_layout!r}")


def hessian_accum(X: torch.Tensor, H: Optional[torch.Tensor] = None,
                  accumulate: bool = False, x_layout: str = "channels") -> torch.Tensor:
    """H (+)= 2 X X^T for activations X (bf16 or fp32) stored [n, ntok]
    (``x_layout="channels"``) or [ntok, n] (``x_layout="tokens"``)."""
    _require_cuda(X, H)
    n, ntok, ldx, xdt = _x_args(X, x_layout)
    _check(H, "H", (n, n), _F32)
    if H is None:
        H = torch.empty((n, n), dtype=torch.float32, device=X.device)
    L = lib()
    wsb = L.pwq_hessian_workspace_size(n, ntok)
    ws = _workspace(wsb, X.device)
    check(L.pwq_hessian_accum(H.data_ptr(), n, X.data_ptr(), xdt, ntok, ldx,
                              int(accumulate), ws.data_ptr(), ws.numel(), _stream()))
    return H


def damp_cholesky(H: torch.Tensor, damp: float = 0.01, prec: str = "f32"):
    """(L, dead, result) for H_d = H' + lambda I (lower factor)."""
    _require_cuda(H)
    n = H.shape[0]
    _check(H, "H", (n, n), _F32)
    L_ = lib()
    Lt = torch.empty((n, n), dtype=_tdt(prec), device=H.device)
    dead = torch.empty(n, dtype=torch.int32, device=H.device)
    res = new_result(H.device)
    ws = _workspace(L_.pwq_cholesky_workspace_size(n, _prec(prec)), H.device)
    check(L_.pwq_damp_cholesky(H.data_ptr(), n, float(damp), _prec(prec), Lt.data_ptr(),
                               dead.data_ptr(), res.data_ptr(), ws.data_ptr(), ws.numel(),
                               _stream()))
    return Lt, dead, res


def damp_cholesky_static(H: torch.Tensor, damp: float = 0.01, prec: str = "f32",
                         out: Optional[tuple] = None):
    """damp_cholesky through pwq_damp_cholesky_static: no workspace (the
    library's static device scratch; calls overlapping on one GPU race).
    ``out`` may pass preallocated (L, dead, result) so that the call itself
    allocates nothing."""
    _require_cuda(H)
    n = H.shape[0]
    _check(H, "H", (n, n), _F32)
    if out is None:
        out = (torch.empty((n, n), dtype=_tdt(prec), device=H.device),
               torch.empty(n, dtype=torch.int32, device=H.device), new_result(H.device))
    Lt, dead, res = out
    _require_cuda(Lt, dead, res)
    _check(Lt, "L", (n, n), (_tdt(prec),))
    _check(dead, "dead", (n,), _I32)
    _check_result(res)
    check(lib().pwq_damp_cholesky_static(H.data_ptr(), n, float(damp), _prec(prec),
                                         Lt.data_ptr(), dead.data_ptr(), res.data_ptr(),
                                         _stream()))
    return Lt, dead, res


def min_pivot_order(H: torch.Tensor, damp: float = 0.01, want_pivots: bool = False):
    """Min-pivot order of H_d = H' + lambda I: (perm, pivots or None, result).
    perm[k] (int32) is the column at position k (position 0 is processed
    last); pivots (float64) are the LDL pivots D_kk of the permuted matrix."""
    _require_cuda(H)
    n = H.shape[0]
    if H.dim() != 2 or H.shape[1] != n or H.dtype != torch.float32 or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [n, n] tensor")
    L_ = lib()
    perm = torch.empty(n, dtype=torch.int32, device=H.device)
    piv = torch.empty(n, dtype=torch.float64, device=H.device) if want_pivots else None
    res = new_result(H.device)
    ws = _workspace(L_.pwq_min_pivot_workspace_size(n), H.device)
    check(L_.pwq_min_pivot_order(H.data_ptr(), n, float(damp), perm.data_ptr(), _ptr(piv),
                                 res.data_ptr(), ws.data_ptr(), ws.numel(), _stream()))
    return perm, piv, res


def oaem_init(W: torch.Tensor, H: torch.Tensor, seeds: torch.Tensor, g: int = 8,
              iters: int = 10, damp: float = 0.01, want_objective: bool = True):
    """OA-EM codebook initialisation.  seeds: int64 [M, K] group indices
    r (n/g) + i.  Returns (codebooks float64 [M, K, g], codes int32
    [M, m, n/g], objective float64 [M] or None, result)."""
    _require_cuda(W, H, seeds)
    m, n = W.shape
    if H.shape != (n, n) or H.dtype != torch.float32 or not H.is_contiguous():
        raise ValueError("H must be a contiguous float32 [n, n] tensor")
    if seeds.dim() != 2 or seeds.dtype != torch.int64 or not seeds.is_contiguous():
        raise ValueError("seeds must be a contiguous int64 [M, K] tensor")
    M, K = seeds.shape
    if g <= 0 or n % g:
        raise ValueError("g must divide n")
    dev = W.device
    L_ = lib()
    books = torch.empty((M, K, g), dtype=torch.float64, device=dev)
    codes = torch.empty((M, m, n // g), dtype=torch.int32, device=dev)
    obj = torch.empty(M, dtype=torch.float64, device=dev) if want_objective else None
    res = new_result(dev)
    nb = L_.pwq_oaem_workspace_size(m, n, g, K)
    ws = _workspace(nb, dev) if nb else None
    check(L_.pwq_oaem_init(W.data_ptr(), _dtype_code(W), m, n, _row_major(W), H.data_ptr(),
                           float(damp), int(g), int(K), int(M), int(iters), seeds.data_ptr(),
                           books.data_ptr(), codes.data_ptr(), _ptr(obj), res.data_ptr(),
                           _ptr(ws), 0 if ws is None else ws.numel(), _stream()))
    return books, codes, obj, res


def grid_steps(W: torch.Tensor, grid: Grid, dead: Optional[torch.Tensor] = None):
    """(scales [m, n/G], zeros [m, n/G] or None) for SYM / ASYM grids."""
    _require_cuda(W, dead)
    m, n = W.shape
    _check(dead, "dead", (n,), _I32)
    if grid.group and n % grid.group:
        raise ValueError(f"group {grid.group} does not divide n = {n}")
    G = grid.group or n
    scales = torch.empty((m, n // G), dtype=torch.float32, device=W.device)
    zeros = (torch.empty((m, n // G), dtype=torch.int32, device=W.device)
             if grid.kind == "asym" else None)
    g = grid.c_struct()
    check(lib().pwq_grid_steps(W.data_ptr(), _dtype_code(W), m, n, _row_major(W), _ptr(dead),
                               g, scales.data_ptr(), _ptr(zeros), _stream()))
    return scales, zeros


def babai_sweep(W: torch.Tensor, L: torch.Tensor, grid: Grid, scales=None, zeros=None,
                dead=None, block: int = 128, result: Optional[torch.Tensor] = None):
    """Nearest-plane sweep given a factor L (natural order).  Returns
    (codes, scales, result)."""
    _require_cuda(W, L, scales, zeros, dead)
    m, n = W.shape
    _check(L, "L", (n, n), (torch.float32, torch.float64))
    prec = "f64" if L.dtype == torch.float64 else "f32"
    _check(dead, "dead", (n,), _I32)
    _check_result(result)
    if grid.kind == "colspacing":
        scales = torch.empty(n, dtype=torch.float32, device=W.device)
    elif scales is None:
        raise ValueError("SYM/ASYM sweeps need scales (see grid_steps)")
    else:
        if grid.group and n % grid.group:
            raise ValueError(f"group {grid.group} does not divide n = {n}")
        ng = n // (grid.group or n)
        _check(scales, "scales", (m, ng), _F32)
        _check(zeros, "zeros", (m, ng), _I32)
    codes = torch.empty((m, n), dtype=torch.int32, device=W.device)
    res = new_result(W.device) if result is None else result
    L_ = lib()
    ws = _workspace(L_.pwq_sweep_workspace_size(m, n, block, _prec(prec)), W.device)
    g = grid.c_struct()
    check(L_.pwq_babai_sweep(W.data_ptr(), _dtype_code(W), m, n, _row_major(W), L.data_ptr(),
                             _prec(prec), _ptr(dead), g, scales.data_ptr(), _ptr(zeros),
                             block, codes.data_ptr(), res.data_ptr(), ws.data_ptr(),
                             ws.numel(), _stream()))
    return codes, scales, res


def workspace_for_layer(m, n, ntok, has_x, order, block, prec, device) -> torch.Tensor:
    nb = lib().pwq_quant_layer_workspace_size(m, n, ntok, int(has_x), _lib.ORDERS[order],
                                             block, _prec(prec))
    return _workspace(nb, device)


def quant_layer(W: torch.Tensor, X: Optional[torch.Tensor] = None,
                H: Optional[torch.Tensor] = None, grid: Grid = Grid(),
                order: str = "back_to_front", perm: Optional[torch.Tensor] = None,
                damp: float = 0.01, block: int = 128, prec: str = "f32",
                want_H: bool = False, want_L: bool = False,
                workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None,
                x_layout: str = "channels"):
    """quant_layer(W, X or H, grid, order, damp) -> dict(codes, scales, zeros,
    result[, H, L]).  ``out`` may pass preallocated outputs (same keys);
    ``x_layout`` as for hessian_accum."""
    _require_cuda(W, X, H, perm, workspace)
    m, n = W.shape
    dev = W.device
    ntok, ldx, xdt = 0, 0, 0
    if X is not None:
        nx, ntok, ldx, xdt = _x_args(X, x_layout)
        if nx != n:
            raise ValueError(f"X has {nx} channels, W has {n} columns")
    _check(H, "H", (n, n), _F32)
    _check(perm, "perm", (n,), _I32)
    if grid.kind != "colspacing" and grid.group and n % grid.group:
        raise ValueError(f"group {grid.group} does not divide n = {n}")
    G = n if grid.kind == "colspacing" else (grid.group or n)
    for k, t in (out or {}).items():
        _require_cuda(t)
    if out:
        ng = n // G
        _check(out.get("codes"), "out['codes']", (m, n), _I32)
        _check(out.get("scales"), "out['scales']",
               (n,) if grid.kind == "colspacing" else (m, ng), _F32)
        if grid.kind == "asym":
            _check(out.get("zeros"), "out['zeros']", (m, ng), _I32)
        _check_result(out.get("result"))
        _check(out.get("H"), "out['H']", (n, n), _F32)
        _check(out.get("L"), "out['L']", (n, n), (_tdt(prec),))
    o = dict(out or {})
    if "codes" not in o:
        o["codes"] = torch.empty((m, n), dtype=torch.int32, device=dev)
    if "scales" not in o:
        o["scales"] = (torch.empty(n, dtype=torch.float32, device=dev)
                       if grid.kind == "colspacing"
                       else torch.empty((m, n // G), dtype=torch.float32, device=dev))
    if "zeros" not in o:
        o["zeros"] = (torch.empty((m, n // G), dtype=torch.int32, device=dev)
                      if grid.kind == "asym" else None)
    if "result" not in o:
        o["result"] = new_result(dev)
    if want_H and X is not None and o.get("H") is None:
        o["H"] = torch.empty((n, n), dtype=torch.float32, device=dev)
    if want_L and o.get("L") is None:
        o["L"] = torch.empty((n, n), dtype=_tdt(prec), device=dev)
    ws = workspace if workspace is not None else workspace_for_layer(
        m, n, ntok, X is not None, order, block, prec, dev)
    g = grid.c_struct()
    check(lib().pwq_quant_layer(
        W.data_ptr(), _dtype_code(W), m, n, _row_major(W),
        _ptr(X), xdt, ntok, ldx, _ptr(H), g,
        _lib.ORDERS[order], _ptr(perm), float(damp), int(block), _prec(prec),
        o["codes"].data_ptr(), o["scales"].data_ptr(), _ptr(o["zeros"]),
        o["result"].data_ptr(), _ptr(o.get("H")), _ptr(o.get("L")), ws.data_ptr(),
        ws.numel(), _stream()))
    return o


def column_entropy(codes: torch.Tensor, huffman: bool = False):
    """Per-column empirical entropy (bits) of int32 codes [m, n] and its mean
    over the columns: (bits [n] float64, mean [] float64), both on the GPU;
    with ``huffman`` also each column's Huffman-coded length in bits
    ([n] int64, -1 where not computed) as a third element."""
    _require_cuda(codes)
    if codes.dtype != torch.int32:
        raise TypeError("codes must be int32")
    m, n = codes.shape
    ldc = _row_major(codes) if m > 0 else n
    bits = torch.empty(n, dtype=torch.float64, device=codes.device)
    mean = torch.empty((), dtype=torch.float64, device=codes.device)
    huff = torch.empty(n, dtype=torch.int64, device=codes.device) if huffman else None
    L_ = lib()
    ws = _workspace(L_.pwq_rate_workspace_size(n), codes.device)
    check(L_.pwq_column_entropy(codes.data_ptr(), m, n, ldc, bits.data_ptr(), mean.data_ptr(),
                                _ptr(huff), ws.data_ptr(), ws.numel(), _stream()))
    return (bits, mean, huff) if huffman else (bits, mean)


class KernelTimer:
    """Times one of the library's kernels (pwq_kernel_timer_attach):
    inside the ``with`` block, its first ``capacity`` launches record a pair
    of HIP events on the stream they run on.  ``kernel`` is "hessian_tiles"
    (the SYRK tiles), "lazy_update" (one lazy block update of the sweep) or
    "sweep_block" (one block of the column sweep).  Measurement only."""

    def __init__(self, kernel: str, capacity: int):
        self.kernel = _lib.TIMED_KERNELS[kernel]
        self.starts = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        self.stops = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        for e in self.starts + self.stops:
            e.record()          # torch creates the HIP event on its first record
        arr = ctypes.c_void_p * max(capacity, 1)
        self._s = arr(*[e.cuda_event for e in self.starts])
        self._e = arr(*[e.cuda_event for e in self.stops])
        self.capacity = capacity
        self.count = 0

    def __enter__(self):
        check(lib().pwq_kernel_timer_attach(self.kernel, self._s, self._e, self.capacity))
        return self

    def __exit__(self, *exc):
        self.count = int(lib().pwq_kernel_timer_count(self.kernel))
        check(lib().pwq_kernel_timer_attach(self.kernel, None, None, 0))
        return False

    def durations_ms(self):
        """Per-launch durations (synchronises)."""
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in zip(self.starts[:self.count],
                                                  self.stops[:self.count])]


class HessianTileTimer(KernelTimer):
    """KernelTimer of the Hessian product kernel."""

    def __init__(self, capacity: int):
        super().__init__("hessian_tiles", capacity)


def overflow_entries(codes: torch.Tensor, scales: torch.Tensor, grid: Grid,
                     zeros: Optional[torch.Tensor] = None, max_out: Optional[int] = None):
    """Overflow entries of int32 codes [m, n] for a SYM/ASYM grid (SSQR):
    (rows, cols, vals, count) -- the first min(count, max_out) entries of the
    (row, column)-sorted list, and the device int64 count."""
    _require_cuda(codes, scales, zeros)
    if codes.dtype != torch.int32:
        raise TypeError("codes must be int32")
    m, n = codes.shape
    if grid.group and n % grid.group:
        raise ValueError(f"group {grid.group} does not divide n = {n}")
    ng = n // (grid.group or n)
    _check(scales, "scales", (m, ng), _F32)
    _check(zeros, "zeros", (m, ng), _I32)
    ldc = _row_major(codes) if m > 0 else n
    cap = m * n if max_out is None else int(max_out)
    dev = codes.device
    rows = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    cols = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    vals = torch.empty(max(cap, 1), dtype=torch.float32, device=dev)
    count = torch.zeros((), dtype=torch.int64, device=dev)
    L_ = lib()
    ws = _workspace(L_.pwq_overflow_workspace_size(m), dev)
    g = grid.c_struct()
    check(L_.pwq_overflow_entries(codes.data_ptr(), m, n, ldc, g, scales.data_ptr(),
                                  _ptr(zeros), cap, rows.data_ptr(), cols.data_ptr(),
                                  vals.data_ptr(), count.data_ptr(), ws.data_ptr(), ws.numel(),
                                  _stream()))
    return rows, cols, vals, count


def ssqr_quant_layer(W: torch.Tensor, X: Optional[torch.Tensor] = None,
                     H: Optional[torch.Tensor] = None, grid: Grid = Grid(),
                     damp: float = 0.01, block: int = 128, prec: str = "f32",
                     density: float = 0.01, iters: int = 12, log2_lo: float = -8.0,
                     max_outliers: Optional[int] = None, x_layout: str = "channels"):
    """Overflow-tolerant quantization (SSQR): the step multiplier kappa is
    bisected in log2 for at most ``density`` m n outlier codes.  Returns a
    dict: codes, scales, zeros, result, kappa, n_outliers and the outlier
    list rows / cols / vals (trimmed to min(n_outliers, max_outliers)).
    Synchronous."""
    _require_cuda(W, X, H)
    m, n = W.shape
    dev = W.device
    ntok, ldx, xdt = 0, 0, 0
    if X is not None:
        nx, ntok, ldx, xdt = _x_args(X, x_layout)
        if nx != n:
            raise ValueError(f"X has {nx} channels, W has {n} columns")
    _check(H, "H", (n, n), _F32)
    if grid.group and n % grid.group:
        raise ValueError(f"group {grid.group} does not divide n = {n}")
    G = grid.group or n
    cap = m * n if max_outliers is None else int(max_outliers)
    o = {"codes": torch.empty((m, n), dtype=torch.int32, device=dev),
         "scales": torch.empty((m, n // G), dtype=torch.float32, device=dev),
         "zeros": (torch.empty((m, n // G), dtype=torch.int32, device=dev)
                   if grid.kind == "asym" else None),
         "result": new_result(dev)}
    rows = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    cols = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    vals = torch.empty(max(cap, 1), dtype=torch.float32, device=dev)
    n_out = ctypes.c_int64(0)
    kappa = ctypes.c_double(0.0)
    L_ = lib()
    ws = _workspace(L_.pwq_ssqr_workspace_size(m, n, ntok, int(X is not None), block,
                                               _prec(prec)), dev)
    g = grid.c_struct()
    check(L_.pwq_ssqr_quant_layer(
        W.data_ptr(), _dtype_code(W), m, n, _row_major(W), _ptr(X), xdt, ntok, ldx, _ptr(H),
        g, float(damp), int(block), _prec(prec), float(density), int(iters), float(log2_lo),
        o["codes"].data_ptr(), o["scales"].data_ptr(), _ptr(o["zeros"]),
        o["result"].data_ptr(), cap, rows.data_ptr(), cols.data_ptr(), vals.data_ptr(),
        ctypes.byref(n_out), ctypes.byref(kappa), ws.data_ptr(), ws.numel(), _stream()))
    k = min(int(n_out.value), cap)
    o.update(kappa=float(kappa.value), n_outliers=int(n_out.value), rows=rows[:k],
             cols=cols[:k], vals=vals[:k])
    return o
