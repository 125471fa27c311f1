"""Precision study for the column-spacing (ZSIC) layer: how far an fp32 factor
or fp32 lazy updates move the sweep's coordinates, in grid units, against
the all-fp64 sweep.

Not a pytest module (the name is not collected); run it as a script:

    python tests/study_spectral_precision.py [m] [n]

The layer is the spectral test layer resized to m x n (H = L0 diag(k^-1.2)
L0^T, damp 0), with the spacing constant c searched for a mean column
entropy of 2.5 bits on the fp64 codes ("WaterSIC: ...", technical summary
2: alpha_i = c / |l_ii|).  The sweep is the oracle's blocked back-to-front
sweep (lazy updates after each block of 256 columns) written out here with
selectable precisions:

  fp32 updates, fp64 target   E L products and their sums in fp32, added to
                              an fp64 running target (the mixed route)
  fp32 updates and target     the running target kept in fp32 as well
  fp32 factor                 the Cholesky factor of the damped H in fp32
  fp32 factor and updates     both, fp64 target

The fp32 factor is LAPACK's spotrf (through scipy).  numpy's float32
Cholesky cannot stand in for it: it factors in fp64 and rounds the result
(bitwise the fp64 factor rounded), about 300 times more accurate than an
fp32 factor of these Hessians.

For each it prints the share of codes equal to the fp64 sweep's, the
mismatches that are not within 1e-5 of a rounding tie, and the drift
|c - c_64| of the coordinates whose codes agree (largest, 99.9th
percentile, and largest per tenth of the columns).  The codes must match to
1e-5 of a tie, so a drift above that in any column is a parity risk.
"""
import os
import sys

import numpy as np
import scipy.linalg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

BLOCK = 256


def sweep(Wp, L, Sp, upd_dtype=np.float64, tgt_dtype=np.float64):
    """Blocked nearest-plane sweep (the oracle's order of operations) with
    the lazy-update products in upd_dtype and the running target in
    tgt_dtype; decisions in fp64.  Returns codes and coordinates c."""
    m, n = Wp.shape
    Wt = np.array(Wp, dtype=tgt_dtype, copy=True)
    Z = np.zeros((m, n))
    C = np.zeros((m, n))
    Lu = (L / np.diag(L)[None, :]).astype(upd_dtype)
    for b in range((n + BLOCK - 1) // BLOCK - 1, -1, -1):
        j0, j1 = b * BLOCK, min(n, b * BLOCK + BLOCK)
        E = np.zeros((m, j1 - j0))
        for k in range(j1 - 1, j0 - 1, -1):
            c = Wt[:, k].astype(np.float64) / Sp[:, k]
            z = np.rint(c)
            Z[:, k] = z
            C[:, k] = c
            e = Wp[:, k] - Sp[:, k] * z
            E[:, k - j0] = e
            if k > j0:
                Wt[:, j0:k] += np.outer(e.astype(upd_dtype), Lu[k, j0:k]).astype(tgt_dtype)
        if j0 > 0:
            Wt[:, :j0] += (E.astype(upd_dtype) @ Lu[j0:j1, :j0]).astype(tgt_dtype)
    return Z, C


def main(m=128, n=2048):
    cfg = synth.config(5).resized(m=m, n=n)
    lay = synth.make_layer(cfg)
    Hd, W0, _, _ = O.fix_dead_and_damp(lay.H.astype(np.float64), lay.W64(), cfg.damp)
    L, info = O.cholesky_lower(Hd)
    assert info == 0

    def steps(Lx, c):
        return np.broadcast_to(O.colspacing_steps(Lx, c)[None, :], (m, n))

    lo, hi = 1e-8, 10.0
    for _ in range(24):
        c = np.sqrt(lo * hi)
        Z, _ = sweep(W0, L, steps(L, c))
        if float(np.mean(O.column_entropy_bits(Z.astype(np.int64)))) > 2.5:
            lo = c
        else:
            hi = c
    c = np.sqrt(lo * hi)
    S = steps(L, c)
    Z64, C64 = sweep(W0, L, S)
    ref, _ = O.nearest_plane_sweep_blocked(W0, L, S, BLOCK)
    assert np.array_equal(ref, Z64), "the study's fp64 sweep differs from the oracle's"
    bits = float(np.mean(O.column_entropy_bits(Z64.astype(np.int64))))
    print(f"m={m} n={n} c={c:.4g} mean bits {bits:.3f} max |code| {np.abs(Z64).max():.0f}")

    L32 = scipy.linalg.cholesky(Hd.astype(np.float32), lower=True,
                                check_finite=False).astype(np.float64)
    assert L32.dtype == np.float64 and np.all(np.triu(L32, 1) == 0)
    print(f"fp32 factor: relative Frobenius difference {np.linalg.norm(L32 - L) / np.linalg.norm(L):.2e}")
    cases = [("fp32 updates, fp64 target", L, np.float32, np.float64),
             ("fp32 updates and target", L, np.float32, np.float32),
             ("fp32 factor", L32, np.float64, np.float64),
             ("fp32 factor and updates", L32, np.float32, np.float64)]
    tie = np.abs(np.abs(C64 - Z64) - 0.5) <= 1e-5
    for name, Lx, ud, td in cases:
        Z, C = sweep(W0, Lx, steps(Lx, c), ud, td)
        diff = Z != Z64
        drift = np.abs(C - C64)
        drift[diff] = np.nan
        deciles = " ".join(f"{np.nanmax(drift[:, i * n // 10:(i + 1) * n // 10]):.1e}"
                           for i in range(10))
        # a code is a parity risk where the coordinate's drift exceeds the
        # 1e-5 window and the coordinate lies between 1e-5 and that drift
        # from a midpoint: with fractional parts spread evenly that has
        # probability 2 (drift - 1e-5); summed, the expected count
        over = np.nan_to_num(drift, nan=0.0)
        risk = float(np.sum(2.0 * np.clip(over - 1e-5, 0.0, None)))
        print(f"{'':28s} coordinates drifting > 1e-5: {int((over > 1e-5).sum())} of {over.size}; "
              f"expected codes outside the window: {risk:.2e} (x{235e6 / over.size:.0f} at 8192 x 28672)")
        print(f"{name:28s} equal {100.0 * (1 - diff.sum() / diff.size):.4f}%  "
              f"not at a tie {int((diff & ~tie).sum())}  drift max {np.nanmax(drift):.2e}  "
              f"99.9% {np.nanpercentile(drift, 99.9):.2e}  by tenth of columns: {deciles}")


if __name__ == "__main__":
    args = [int(a) for a in sys.argv[1:3]]
    main(*args)
