"""Seeded generators for W, calibration activations X and the given-H workload.

bf16 arrays are returned as their raw 16-bit patterns (``uint16``), rounded
from float32 to nearest-even; ``bf16_bits_to_f32`` widens them exactly.  The
same bits are uploaded to the GPU and widened to float64 for the oracle, so
both sides see identical inputs.
"""
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .configs import LayerConfig

CHUNK_TOKENS = 8192
_ROOT_SEED = 2026


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    return max(1, min(16, avail))


def _seed(cfg: LayerConfig, full: bool) -> np.random.SeedSequence:
    key = [_ROOT_SEED, cfg.key]
    if not full:
        key += [cfg.m, cfg.n, cfg.ntok]
    return np.random.SeedSequence(key)


@dataclass
class Layer:
    """One seeded workload.

    ``W``/``X`` hold float32 values (exactly bf16-representable when the
    workload's dtype is bf16); ``W_bits``/``X_bits`` hold the bf16 patterns
    for upload.  For the given-H workload ``X`` is None and ``H`` is float32.
    """
    cfg: LayerConfig
    W: np.ndarray
    W_bits: Optional[np.ndarray]
    X: Optional[np.ndarray]
    X_bits: Optional[np.ndarray]
    H: Optional[np.ndarray]

    def W64(self) -> np.ndarray:
        return self.W.astype(np.float64)

    def X64(self) -> np.ndarray:
        return None if self.X is None else self.X.astype(np.float64)


def _store(vals32: np.ndarray, dtype: str):
    if dtype == "bf16":
        bits = f32_to_bf16_bits(vals32)
        return bf16_bits_to_f32(bits), bits
    return np.ascontiguousarray(vals32, dtype=np.float32), None


def make_weight(cfg: LayerConfig, ss: np.random.SeedSequence):
    rng = np.random.Generator(np.random.PCG64(ss))
    w = rng.standard_normal((cfg.m, cfg.n), dtype=np.float32)
    w *= np.float32(cfg.w_std)
    return _store(w, cfg.wdtype)


def make_activations(cfg: LayerConfig, ss_std: np.random.SeedSequence,
                     ss_out: np.random.SeedSequence,
                     ss_x: np.random.SeedSequence, keep_f32: bool = True):
    """X [n, ntok], tokens contiguous (channel-major)."""
    n, ntok = cfg.n, cfg.ntok
    rs = np.random.Generator(np.random.PCG64(ss_std))
    ro = np.random.Generator(np.random.PCG64(ss_out))
    if cfg.x_kind in ("gauss_lognormal", "laplace_lognormal"):
        chan = rs.lognormal(0.0, cfg.x_param, n)
    else:
        chan = np.ones(n)
    if cfg.outliers:
        # (layers narrower than the outlier count: every channel)
        idx = ro.choice(n, size=min(cfg.outliers, n), replace=False)
        chan[idx] *= cfg.outlier_scale
    chan = chan.reshape(n, 1)
    nchunks = (ntok + CHUNK_TOKENS - 1) // CHUNK_TOKENS
    kids = ss_x.spawn(nchunks)
    bf16 = cfg.xdtype == "bf16"
    X_bits = np.empty((n, ntok), np.uint16) if bf16 else None
    X = np.empty((n, ntok), np.float32) if (keep_f32 or not bf16) else None

    def fill(c):
        t0 = c * CHUNK_TOKENS
        w = min(CHUNK_TOKENS, ntok - t0)
        r = np.random.Generator(np.random.PCG64(kids[c]))
        if cfg.x_kind == "gauss_lognormal":
            v = r.standard_normal((n, w))
        elif cfg.x_kind == "student_t":
            v = r.standard_t(cfg.x_param, size=(n, w))
        elif cfg.x_kind == "laplace_lognormal":
            v = r.laplace(0.0, 1.0, size=(n, w))
        else:
            raise ValueError(cfg.x_kind)
        v = (v * chan).astype(np.float32)
        if bf16:
            b = f32_to_bf16_bits(v)
            X_bits[:, t0:t0 + w] = b
            if X is not None:
                X[:, t0:t0 + w] = bf16_bits_to_f32(b)
        else:
            X[:, t0:t0 + w] = v

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nchunks)))
    return X, X_bits


def make_spectral_hessian(cfg: LayerConfig, ss: np.random.SeedSequence,
                          device=None) -> np.ndarray:
    """H = L0 diag(k^-p) L0^T in float64, rounded once to float32.

    L0 is unit lower triangular with strictly-lower entries N(0, 1/n), drawn
    in fixed row blocks.  With ``device`` (a torch device) the float64
    product is formed there; otherwise on the host in row blocks.
    """
    n = cfg.n
    rows = 1024
    nblk = (n + rows - 1) // rows
    kids = ss.spawn(nblk)
    L0 = np.zeros((n, n), np.float64)

    def fill(b):
        r0 = b * rows
        r1 = min(n, r0 + rows)
        r = np.random.Generator(np.random.PCG64(kids[b]))
        blk = r.standard_normal((r1 - r0, n)) / np.sqrt(n)
        L0[r0:r1] = blk

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nblk)))
    L0 = np.tril(L0, -1)
    L0[np.arange(n), np.arange(n)] = 1.0
    spec = np.arange(1, n + 1, dtype=np.float64) ** (-cfg.x_param)
    A = L0 * np.sqrt(spec)[None, :]
    del L0
    if device is not None:
        import torch
        At = torch.from_numpy(A).to(device)
        H = (At @ At.T).to(torch.float32).cpu().numpy()
        del At
        return H
    H = np.empty((n, n), np.float32)
    for r0 in range(0, n, rows):
        r1 = min(n, r0 + rows)
        # rows r0..r1, columns 0..r1 of A A^T; A is lower triangular so only
        # its first r1 columns contribute.
        H[r0:r1, :r1] = (A[r0:r1, :r1] @ A[:r1, :r1].T).astype(np.float32)
    # mirror the lower triangle so H is exactly symmetric
    for r0 in range(0, n, rows):
        r1 = min(n, r0 + rows)
        H[:r0, r0:r1] = H[r0:r1, :r0].T
        blk = H[r0:r1, r0:r1]
        H[r0:r1, r0:r1] = np.tril(blk) + np.tril(blk, -1).T
    return H


def make_layer(cfg: LayerConfig, full: Optional[bool] = None,
               keep_x_f32: bool = True, device=None) -> Layer:
    """Generate one workload.  ``full`` defaults to True when ``cfg`` is the
    unmodified table entry (seed [2026, k]); resized recipes use the seed
    [2026, k, m, n, ntok]."""
    from .configs import CONFIGS
    if full is None:
        full = CONFIGS.get(cfg.key) == cfg or (
            (cfg.m, cfg.n, cfg.ntok) == (CONFIGS[cfg.key].m, CONFIGS[cfg.key].n,
                                         CONFIGS[cfg.key].ntok))
    ss = _seed(cfg, full)
    k_w, k_std, k_out, k_x, k_h = ss.spawn(5)
    W, W_bits = make_weight(cfg, k_w)
    if cfg.x_kind == "spectral_h":
        H = make_spectral_hessian(cfg, k_h, device=device)
        return Layer(cfg, W, W_bits, None, None, H)
    X, X_bits = make_activations(cfg, k_std, k_out, k_x, keep_f32=keep_x_f32)
    return Layer(cfg, W, W_bits, X, X_bits, None)
