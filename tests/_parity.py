"""Comparison helpers between the HIP path and the fp64 oracle.

Tolerances (stated once, used by every parity test):
  H and L           relative Frobenius error <= 1e-4
  steps             relative error <= 1e-6, zero points exact
  codes             >= 99.9% identical; every code, teacher-forced through
                    the oracle's fp64 factor, is a nearest rounding of its
                    running target within 1e-5 of the grid midpoint
                    (|G| <= 1/2 + 1e-5)
  proxy losses      relative error <= 1e-3
"""
import numpy as np

import oracle as O

TOL_H = 1e-4
TOL_L = 1e-4
TOL_STEP = 1e-6
TOL_TIE = 1e-5
MIN_IDENTICAL = 0.999
TOL_LOSS = 1e-3


def rel_fro(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def lattice_ints(codes, zeros, n):
    """Stored codes -> signed lattice integers (undo the zero point)."""
    Z = np.asarray(codes, np.int64)
    if zeros is not None:
        Z = Z - O.expand_group_steps(np.asarray(zeros, np.float64), n).astype(np.int64)
    return Z


def check_codes(codes_gpu, ref, zeros_gpu=None, label="", min_identical=MIN_IDENTICAL):
    """Compare GPU codes with an oracle result dict ``ref`` (from
    oracle.quant_layer, or the same keys for a row sample: codes, pi, Sp, W0
    and L).  Returns a dict of statistics; raises AssertionError on
    failure.  ``min_identical`` may be lowered for layers of a few hundred
    codes, where a couple of exact ties already exceed 0.1%; the
    nearest-rounding check is the same for every layer."""
    codes_gpu = np.asarray(codes_gpu, np.int64)
    ref_codes = ref["codes"]
    same = float(np.mean(codes_gpu == ref_codes))
    n = codes_gpu.shape[1]
    Zg = lattice_ints(codes_gpu, zeros_gpu, n)
    pi = ref["pi"]
    Sp = ref["Sp"]
    W0 = ref["W0"]
    S = np.empty_like(Sp)
    S[:, pi] = Sp
    Dp = (W0 - S * Zg)[:, pi]
    G = O.certificate(Dp, ref["L"], Sp)
    gmax = float(np.max(np.abs(G))) if G.size else 0.0
    stats = {"identical": same, "max_abs_G": gmax,
             "mismatches": int(np.sum(codes_gpu != ref_codes))}
    assert same >= min_identical, f"{label}: only {same:.6f} of codes identical {stats}"
    assert gmax <= 0.5 + TOL_TIE, f"{label}: a code is not a nearest rounding {stats}"
    return stats


def check_loss(got, want, label=""):
    rel = abs(got - want) / max(abs(want), 1e-300)
    assert rel <= TOL_LOSS, f"{label}: loss {got} vs {want} (rel {rel:.3g})"
    return rel
