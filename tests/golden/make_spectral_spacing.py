"""Writes spectral_layer_spacing.json: the spacing constant c of the spectral
(ZSIC) layer at which the oracle's codes have a mean per-column empirical
entropy of 2.5 bits.

"WaterSIC: information-theoretically (near) optimal linear layer
quantization", technical summary 2: one lattice spacing per input column,
alpha_k = c / |l_kk|, unequal rates across columns, codes entropy-coded, so
the rate of a column is the entropy of its codes.  The layer is 8192 x 28672
with H = L0 diag(k^-1.2) L0^T (damp 0) and block 256.

Only oracle/ and synth/ are called.  The search runs on log2(c): the rate of
a high-resolution lattice quantizer falls by one bit per doubling of the
spacing, so each step moves log2(c) by (rate - target) bits (a secant step
once two points are known, kept inside the bracket), first on a 1024-row
sample and then on every row, until |rate - 2.5| <= 0.002.

    python tests/golden/make_spectral_spacing.py      (from the repository root)
"""
import json
import math
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

TARGET = 2.5
TOL = 0.002
OUT = os.path.join(HERE, "spectral_layer_spacing.json")


def rate_at(W0, L, c, block):
    alpha = O.colspacing_steps(L, c)
    Sp = np.broadcast_to(alpha[None, :], W0.shape)
    Z, _ = O.nearest_plane_sweep_blocked(W0, L, Sp, block)
    return float(np.mean(O.column_entropy_bits(Z)))


def search(W0, L, block, log2c, tol, log):
    pts = []
    lo = hi = None           # log2 c with rate above / below the target
    for _ in range(30):
        t0 = time.time()
        r = rate_at(W0, L, 2.0 ** log2c, block)
        log(f"  rows {W0.shape[0]}: log2 c = {log2c:.6f}  rate = {r:.6f}  "
            f"({time.time() - t0:.1f} s)")
        pts.append((log2c, r))
        if abs(r - TARGET) <= tol:
            return log2c, r, pts
        if r > TARGET:
            lo = log2c if lo is None else max(lo, log2c)
        else:
            hi = log2c if hi is None else min(hi, log2c)
        if len(pts) >= 2 and pts[-1][1] != pts[-2][1]:
            (x0, r0), (x1, r1) = pts[-2], pts[-1]
            nxt = x1 + (TARGET - r1) * (x1 - x0) / (r1 - r0)
        else:
            nxt = log2c + (r - TARGET)
        if lo is not None and hi is not None and not (lo < nxt < hi):
            nxt = 0.5 * (lo + hi)
        log2c = nxt
    raise RuntimeError("rate search did not converge")


def main():
    def log(s):
        print(s, flush=True)
    cfg = synth.config(5)
    t0 = time.time()
    lay = synth.make_layer(cfg)
    log(f"generated {cfg.name} in {time.time() - t0:.1f} s")
    t0 = time.time()
    Hd, W0, lam, dead = O.fix_dead_and_damp(lay.H.astype(np.float64), lay.W64(), cfg.damp)
    del lay
    L, info = O.cholesky_lower(Hd)
    del Hd
    assert info == 0
    log(f"oracle factor in {time.time() - t0:.1f} s")
    rows = np.random.default_rng(0).choice(W0.shape[0], 1024, replace=False)
    rows.sort()
    log2c, r_s, pts_s = search(W0[rows], L, cfg.block, -13.0, 0.01, log)
    log2c, r, pts = search(W0, L, cfg.block, log2c, TOL, log)
    rec = {
        "what": "spacing constant c of the spectral layer (alpha_k = c / l_kk) giving a mean "
                "per-column code entropy of 2.5 bits on the oracle's codes",
        "source": "WaterSIC technical summary 2 (unequal rates, spacing proportional to "
                  "1/|l_kk|, entropy coding); written by tests/golden/make_spectral_spacing.py "
                  "from oracle/ and synth/ only",
        "layer": {"m": cfg.m, "n": cfg.n, "block": cfg.block, "damp": cfg.damp,
                  "H": "L0 diag(k^-1.2) L0^T, synth.make_layer(config 5) on the host"},
        "c": 2.0 ** log2c, "log2_c": log2c, "rate_bits": r, "target_bits": TARGET,
        "tolerance_bits": TOL,
        "search_sample_rows": [list(p) for p in pts_s], "search_all_rows": [list(p) for p in pts],
    }
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    log(json.dumps({"c": rec["c"], "rate": r}))


if __name__ == "__main__":
    main()
