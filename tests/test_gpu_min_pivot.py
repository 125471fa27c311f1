"""Min-pivot order through the C ABI, against the oracle.

The order is an integer result decided by floating point, so both sides
decide in float64 on the same float32 Hessian (the GPU's).  Where several
orders are correct (two Schur diagonals within rounding of each other),
the test checks validity instead of identity:

* every pivot of the GPU's order is the smallest Schur diagonal still open
  at its step, within a relative 1e-9 (the Schur diagonals come from numpy's
  Cholesky factor of the permuted damped matrix);
* the GPU's pivots equal that factor's squared diagonal (relative 1e-9);
* where the oracle's own order has no near tie (every step's two smallest
  candidates differ by more than 1e-7 relative), the orders are identical.

The layer with MIN_PIVOT is checked stage-fed: the oracle runs the same
permutation (order "perm"), and the GPU's MIN_PIVOT layer equals its PERM
layer bitwise.
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_19_amd as P
import synth
from _gpu import to_np, upload
from _parity import check_codes, check_loss

pytestmark = pytest.mark.gpu

TOL_PIVOT = 1e-9
CLEAR_GAP = 1e-7


def _schur_table(Hp, L):
    """Schur diagonal of position i at step k, for i >= k (others NaN)."""
    n = Hp.shape[0]
    sq = np.cumsum(L ** 2, axis=1)
    prev = np.zeros((n, n))
    prev[:, 1:] = sq[:, :-1]
    S = np.diag(Hp)[:, None] - prev            # S[i, k]
    S[np.tril_indices(n, -1)[::-1]] = np.nan   # i < k: already chosen
    return S


def _check_valid(Hd, perm, piv=None):
    pi = np.asarray(perm, np.int64)
    n = len(pi)
    assert sorted(pi.tolist()) == list(range(n))
    Hp = Hd[np.ix_(pi, pi)]
    L = np.linalg.cholesky(Hp)
    D = np.diag(L) ** 2
    S = _schur_table(Hp, L)
    worst = 0.0
    for k in range(n):
        m = np.nanmin(S[k:, k])
        worst = max(worst, (D[k] - m) / m)
    assert worst <= TOL_PIVOT, f"a pivot is not the smallest open diagonal ({worst:.3g})"
    if piv is not None:
        rel = np.max(np.abs(piv - D) / D)
        assert rel <= TOL_PIVOT, rel
    return D


def _clear_margin(Hd, pi):
    """Smallest relative gap between the two smallest candidates of a step."""
    Hp = Hd[np.ix_(pi, pi)]
    L = np.linalg.cholesky(Hp)
    S = _schur_table(Hp, L)
    gap = np.inf
    for k in range(len(pi) - 1):
        col = np.sort(S[k:, k])
        gap = min(gap, (col[1] - col[0]) / abs(col[0]))
    return gap


# (config, m, n, ntok, dead inputs)
CASES = [
    (1, 8, 7, 64, ()),             # fewer columns than one panel
    (1, 16, 130, 1000, ()),        # panels + ragged tail
    (2, 16, 300, 3000, (17, 201)),  # erased inputs (H_ii = 0 -> 1)
    (3, 16, 1000, 6000, ()),       # several workgroups per step, many tiles
]


@pytest.mark.parametrize("cfg_id,m,n,ntok,dead", CASES)
def test_min_pivot_order(cfg_id, m, n, ntok, dead):
    cfg = synth.config(cfg_id).resized(m=m, n=n, ntok=ntok)
    lay = synth.make_layer(cfg)
    for i in dead:
        lay.X[i] = 0.0
        lay.X_bits[i] = 0
    _, X, _ = upload(lay)
    H = P.hessian_accum(X)
    print(f"[min-pivot] config {cfg_id} n={n} dead={len(dead)}", flush=True)
    perm, piv, res = P.min_pivot_order(H, damp=cfg.damp, want_pivots=True)
    torch.cuda.synchronize()
    r = P.read_result(res)
    assert r["info"] == 0 and r["ndead"] == len(dead)
    Hd, _, lam, _ = O.fix_dead_and_damp(to_np(H).astype(np.float64), np.zeros((1, n)),
                                        cfg.damp)
    assert r["lambda"] == pytest.approx(lam, rel=1e-12)
    pg = to_np(perm).astype(np.int64)
    _check_valid(Hd, pg, to_np(piv))
    pi_o, piv_o, info_o = O.min_pivot_order(Hd)
    assert info_o == 0
    gap = _clear_margin(Hd, pi_o)
    if gap > CLEAR_GAP:
        assert np.array_equal(pg, pi_o)
        np.testing.assert_allclose(to_np(piv), piv_o, rtol=TOL_PIVOT)
    print(f"[min-pivot] n={n}: valid; oracle margin {gap:.3g}; identical "
          f"{np.array_equal(pg, pi_o)}", flush=True)


@pytest.mark.parametrize("cfg_id,m,n,ntok", [(2, 64, 384, 4096), (1, 40, 130, 1000)])
def test_min_pivot_layer(cfg_id, m, n, ntok):
    cfg = synth.config(cfg_id).resized(m=m, n=n, ntok=ntok)
    lay = synth.make_layer(cfg)
    W, X, _ = upload(lay)
    g = P.Grid(cfg.grid_kind, cfg.bits, cfg.group)
    out = P.quant_layer(W, X=X, grid=g, order="min_pivot", damp=cfg.damp, block=cfg.block,
                        want_H=True)
    torch.cuda.synchronize()
    r = P.read_result(out["result"])
    assert r["info"] == 0
    perm, _, _ = P.min_pivot_order(out["H"], damp=cfg.damp)
    b = P.quant_layer(W, X=X, grid=g, order="perm", perm=perm, damp=cfg.damp,
                      block=cfg.block)
    torch.cuda.synchronize()
    assert torch.equal(out["codes"], b["codes"])
    assert torch.equal(out["result"], b["result"])
    Hg = to_np(out["H"]).astype(np.float64)
    pg = to_np(perm).astype(np.int64)
    ref = O.quant_layer(lay.W64(), H=Hg, grid_kind=cfg.grid_kind, bits=cfg.bits,
                        group=cfg.group, damp=cfg.damp, order="perm", perm=pg)
    zeros = to_np(out["zeros"]) if out["zeros"] is not None else None
    check_codes(to_np(out["codes"]), ref, zeros, label="min_pivot")
    check_loss(r["loss"], ref["loss"], "min_pivot")
    assert r["bound"] == pytest.approx(ref["bound"], rel=1e-3)
    # the order lowers the Theorem 5 bound below the natural order's here
    nat = O.quant_layer(lay.W64(), H=Hg, grid_kind=cfg.grid_kind, bits=cfg.bits,
                        group=cfg.group, damp=cfg.damp)
    print(f"[min-pivot layer] bound {ref['bound']:.6g} vs natural {nat['bound']:.6g}; "
          f"trace D {ref['D'].sum():.6g} vs {nat['D'].sum():.6g}", flush=True)
    assert ref["D"].sum() <= nat["D"].sum()


def test_min_pivot_spectral_layer_f64():
    """The spectral layer (H given, damp 0, column spacing c / l_kk, fp64
    factor and sweep) in min-pivot order: the spacings follow the permuted
    factor, so this checks the order end to end in the other precision."""
    cfg = synth.config(5).resized(m=48, n=512)
    lay = synth.make_layer(cfg)
    W, _, H = upload(lay)
    c = 0.001
    g = P.Grid("colspacing", 0, 0, c)
    out = P.quant_layer(W, H=H, grid=g, order="min_pivot", damp=cfg.damp, block=cfg.block,
                        prec="f64")
    torch.cuda.synchronize()
    r = P.read_result(out["result"])
    assert r["info"] == 0
    perm, _, _ = P.min_pivot_order(H, damp=cfg.damp)
    torch.cuda.synchronize()
    pg = to_np(perm).astype(np.int64)
    Hg = to_np(H).astype(np.float64)
    Hd, _, _, _ = O.fix_dead_and_damp(Hg, np.zeros((1, cfg.n)), cfg.damp)
    _check_valid(Hd, pg)
    ref = O.quant_layer(lay.W64(), H=Hg, grid_kind="colspacing", c=c, damp=cfg.damp,
                        order="perm", perm=pg)
    np.testing.assert_allclose(to_np(out["scales"]).astype(np.float64), ref["scales"],
                               rtol=1e-6)
    check_codes(to_np(out["codes"]), ref, None, label="min_pivot f64")
    check_loss(r["loss"], ref["loss"], "min_pivot f64")
    print(f"[min-pivot] spectral f64: trace D {ref['D'].sum():.6g}", flush=True)


def test_min_pivot_failures():
    n = 64
    # all ones: the first pivot (column 0) leaves a zero Schur complement
    H = torch.ones((n, n), dtype=torch.float32, device="cuda")
    _, _, res = P.min_pivot_order(H, damp=0.0)
    torch.cuda.synchronize()
    assert P.read_result(res)["info"] == 2
    assert O.min_pivot_order(np.ones((n, n)))[2] == 2
    # a negative diagonal entry is the smallest: the first step fails
    d = np.linspace(1.0, 2.0, n)
    d[40] = -0.5
    Hn = torch.from_numpy(np.diag(d).astype(np.float32)).cuda()
    _, _, res = P.min_pivot_order(Hn, damp=0.0)
    torch.cuda.synchronize()
    assert P.read_result(res)["info"] == 1
    # NaN counts as smallest
    Hq = torch.eye(n, dtype=torch.float32, device="cuda")
    Hq[9, 9] = float("nan")
    _, _, res = P.min_pivot_order(Hq, damp=0.0)
    torch.cuda.synchronize()
    assert P.read_result(res)["info"] == 1
    # the layer reports the same step as the oracle's layer
    W = torch.full((8, n), 0.01, dtype=torch.float32, device="cuda")
    out = P.quant_layer(W, H=Hn, grid=P.Grid("sym", 4, 0), order="min_pivot", damp=0.0,
                        block=32)
    torch.cuda.synchronize()
    ref = O.quant_layer(np.full((8, n), 0.01), H=np.diag(d).astype(np.float32).astype(
        np.float64), grid_kind="sym", bits=4, group=0, order="min_pivot", damp=0.0)
    assert P.read_result(out["result"])["info"] == ref["info"] == 1


def test_min_pivot_full_size_qproj():
    """q_proj's Hessian (4096 x 4096 from 131072 bf16 tokens): every pivot
    is the smallest open Schur diagonal and the pivots are the permuted
    factor's."""
    cfg = synth.config(2)
    lay = synth.make_layer(cfg, keep_x_f32=False)
    _, X, _ = upload(lay)
    H = P.hessian_accum(X)
    del X
    perm, piv, res = P.min_pivot_order(H, damp=cfg.damp, want_pivots=True)
    torch.cuda.synchronize()
    assert P.read_result(res)["info"] == 0
    Hd, _, _, _ = O.fix_dead_and_damp(to_np(H).astype(np.float64), np.zeros((1, cfg.n)),
                                      cfg.damp)
    D = _check_valid(Hd, to_np(perm).astype(np.int64), to_np(piv))
    nat = np.diag(np.linalg.cholesky(Hd)) ** 2
    print(f"[min-pivot] q_proj: valid; trace D {D.sum():.6g} vs natural order "
          f"{nat.sum():.6g}", flush=True)
