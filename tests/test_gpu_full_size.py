"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (the layer's own grid, block, damping and precision, X
stored token-major), on outputs the fp64 oracle can compute:

  H      bitwise equal to the Hessian of the same X stored channel-major
         (the two layouts feed the same operands to the same MFMAs in the
         same order); sampled entries 2 sum_t x_it x_jt (all from the same
         bf16 bits), stratified into diagonal and off-diagonal samples; the
         stratified estimate of the relative Frobenius error must be <= 1e-4
  L      the oracle's fp64 Cholesky of the GPU's own H (stage-fed), whole
         matrix, relative Frobenius <= 1e-4; lambda to 1e-12
  steps  whole matrix from the oracle's float32 step rule, <= 1e-6, zero
         points exact
  codes  every row (q_proj, up_proj) or a seeded sample of 1024 rows
         (down_proj, the spectral layer) swept by the oracle (blocked form,
         fp64) with its own factor and steps: >= 99.9% identical and every
         GPU code a nearest rounding (|G| <= 1/2 + 1e-5)
  losses tr(D H D^T) of the GPU's own codes for every row, against the
         GPU's reported loss (1e-3); bound (1/4) sum s^2 l_kk^2 (1e-3)
  rate   (spectral layer) mean per-column code entropy of all GPU codes at
         the oracle-searched spacing constant, within 0.005 bits of 2.5

Each case prints its progress (generation and the long oracle steps).
"""
import json
import os
import time

import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_19_amd as P
import synth
from _gpu import to_np, upload
from _parity import TOL_H, TOL_L, TOL_LOSS, TOL_STEP, check_codes, check_loss, rel_fro

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
SAMPLE_ROWS = 1024        # rows swept by the oracle where not every row is
ALL_ROWS = (2, 3)         # layers whose every row is compared
SAMPLE_H = 512


def log(msg, t0=None):
    extra = f" ({time.time() - t0:.1f} s)" if t0 is not None else ""
    print(f"[full-size] {msg}{extra}", flush=True)


def _grid(cfg, c=None):
    if cfg.grid_kind == "colspacing":
        return P.Grid("colspacing", 0, 0, c)
    return P.Grid(cfg.grid_kind, cfg.bits, cfg.group)


def _row64(bits_row):
    return synth.gen.bf16_bits_to_f32(bits_row).astype(np.float64)


def _check_h_sampled(lay, Hg, seed):
    """Stratified estimate of ||H_gpu - H||_F / ||H||_F from sampled entries."""
    n = lay.cfg.n
    rng = np.random.default_rng(seed)
    di = rng.choice(n, size=min(SAMPLE_H, n), replace=False)
    oi = rng.integers(0, n, size=(SAMPLE_H, 2))
    oi = oi[oi[:, 0] != oi[:, 1]]
    Xb = lay.X_bits

    def ref(i, j):
        a = _row64(Xb[i])
        b = a if i == j else _row64(Xb[j])
        return 2.0 * float(np.dot(a, b))
    d_ref = np.array([ref(i, i) for i in di])
    d_got = Hg[di, di].astype(np.float64)
    o_ref = np.array([ref(i, j) for i, j in oi])
    o_got = Hg[oi[:, 0], oi[:, 1]].astype(np.float64)
    w_d = n / len(di)
    w_o = n * (n - 1) / len(oi)
    err2 = w_d * np.sum((d_got - d_ref) ** 2) + w_o * np.sum((o_got - o_ref) ** 2)
    ref2 = w_d * np.sum(d_ref ** 2) + w_o * np.sum(o_ref ** 2)
    rel = float(np.sqrt(err2 / ref2))
    assert rel <= TOL_H, f"H: estimated relative Frobenius error {rel:.3g}"
    # symmetric storage: the mirrored entries are the same floats
    assert np.array_equal(Hg[oi[:, 0], oi[:, 1]], Hg[oi[:, 1], oi[:, 0]])
    return rel


def _trace_loss(D, H64, chunk=512):
    """tr(D H D^T), row chunks (float64)."""
    tot = 0.0
    for r0 in range(0, D.shape[0], chunk):
        Dc = D[r0:r0 + chunk]
        tot += float(np.sum((Dc @ H64) * Dc))
    return tot


def _run_x_layer(key):
    cfg = synth.config(key)
    t0 = time.time()
    lay = synth.make_layer(cfg, keep_x_f32=False)
    log(f"{cfg.name}: generated W {cfg.m}x{cfg.n}, X {cfg.n}x{cfg.ntok}", t0)
    W, X, _ = upload(lay)
    t0 = time.time()
    Hc = P.hessian_accum(X)                 # channel-major reference H
    Xt = X.t().contiguous()                 # the benchmark's token-major storage
    del X
    out = P.quant_layer(W, X=Xt, grid=_grid(cfg), damp=cfg.damp, block=cfg.block, prec="f32",
                        want_H=True, want_L=True, x_layout="tokens")
    torch.cuda.synchronize()
    res = P.read_result(out["result"])
    log(f"{cfg.name}: GPU quant_layer done (X token-major), info {res['info']}", t0)
    del Xt
    assert res["info"] == 0 and res["ndead"] == 0
    assert torch.equal(out["H"], Hc), "token-major H differs from channel-major H"
    del Hc
    Hg = to_np(out["H"])
    t0 = time.time()
    relH = _check_h_sampled(lay, Hg, seed=key)
    log(f"{cfg.name}: sampled H rel {relH:.3g}", t0)

    # stage-fed oracle: damping, factor and steps from the GPU's H
    t0 = time.time()
    H64 = Hg.astype(np.float64)
    del Hg
    Hd, W0, lam, dead = O.fix_dead_and_damp(H64, lay.W64(), cfg.damp)
    L, info = O.cholesky_lower(Hd)
    del Hd
    assert info == 0
    Lg = to_np(out["L"]).astype(np.float64)
    relL = rel_fro(Lg, L)
    del Lg
    assert relL <= TOL_L, f"L rel {relL}"
    assert abs(res["lambda"] - lam) <= 1e-12 * lam
    log(f"{cfg.name}: oracle factor, L rel {relL:.3g}", t0)

    s_grp, z_grp = O.grid_steps(W0, cfg.grid_kind, cfg.bits, cfg.group)
    sg = to_np(out["scales"]).astype(np.float64)
    assert rel_fro(sg, s_grp) <= TOL_STEP
    zg = None
    if cfg.grid_kind == "asym":
        zg = to_np(out["zeros"])
        assert np.array_equal(zg, z_grp.astype(np.int64))
    S = O.expand_group_steps(s_grp, cfg.n)

    # codes of every row or of a row sample, swept by the oracle with its
    # own factor
    t0 = time.time()
    rows = (np.arange(cfg.m) if key in ALL_ROWS else
            np.sort(np.random.default_rng(100 + key).choice(cfg.m, SAMPLE_ROWS, replace=False)))
    codes = to_np(out["codes"]).astype(np.int64)
    Zr, rho = O.nearest_plane_sweep_blocked(W0[rows], L, S[rows], cfg.block)
    ref = {"codes": Zr.astype(np.int64), "pi": np.arange(cfg.n), "Sp": S[rows],
           "W0": W0[rows], "L": L}
    if zg is not None:
        ref["codes"] = ref["codes"] + O.expand_group_steps(
            z_grp[rows].astype(np.float64), cfg.n).astype(np.int64)
    stats = check_codes(codes[rows], ref, zg[rows] if zg is not None else None,
                        label=cfg.name)
    log(f"{cfg.name}: sampled rows {stats}", t0)

    # losses of the GPU's own codes, every row
    t0 = time.time()
    Zg = codes - (O.expand_group_steps(zg.astype(np.float64), cfg.n).astype(np.int64)
                  if zg is not None else 0)
    D = W0 - S * Zg
    loss = _trace_loss(D, H64)
    check_loss(res["loss"], loss, cfg.name + " loss")
    check_loss(res["loss_damped"], loss + lam * float(np.sum(D * D)), cfg.name + " loss_d")
    check_loss(res["bound"], O.babai_bound(S, np.diag(L) ** 2), cfg.name + " bound")
    assert res["loss_damped"] <= res["bound"]
    log(f"{cfg.name}: losses {res['loss']:.6g} / bound {res['bound']:.6g}", t0)


@pytest.mark.parametrize("key", [2, 3, 4])
def test_full_size_x_layers(key):
    _run_x_layer(key)


def test_full_size_spectral_layer():
    cfg = synth.config(5)
    path = os.path.join(HERE, "golden", "spectral_layer_spacing.json")
    if not os.path.exists(path):
        pytest.skip("spacing constant not searched yet (tests/golden/make_spectral_spacing.py)")
    with open(path) as f:
        spacing = json.load(f)
    c = float(spacing["c"])
    t0 = time.time()
    lay = synth.make_layer(cfg)
    log(f"{cfg.name}: generated W {cfg.m}x{cfg.n} and H {cfg.n}^2", t0)
    W, _, H = upload(lay)
    t0 = time.time()
    out = P.quant_layer(W, H=H, grid=_grid(cfg, c), damp=cfg.damp, block=cfg.block,
                        prec="f64", want_L=True)
    torch.cuda.synchronize()
    res = P.read_result(out["result"])
    log(f"{cfg.name}: GPU quant_layer done, info {res['info']}", t0)
    assert res["info"] == 0 and res["ndead"] == 0 and res["lambda"] == 0.0
    del H

    t0 = time.time()
    H64 = lay.H.astype(np.float64)
    L, info = O.cholesky_lower(H64)
    assert info == 0
    Lg = to_np(out["L"])
    relL = rel_fro(Lg, L)
    del Lg
    assert relL <= TOL_L, f"L rel {relL}"
    log(f"{cfg.name}: oracle factor, L rel {relL:.3g}", t0)
    alpha = O.colspacing_steps(L, c)
    ag = to_np(out["scales"]).astype(np.float64)
    assert rel_fro(ag, alpha) <= TOL_STEP

    t0 = time.time()
    W0 = lay.W64()
    rows = np.sort(np.random.default_rng(105).choice(cfg.m, SAMPLE_ROWS, replace=False))
    codes = to_np(out["codes"]).astype(np.int64)
    Sr = np.broadcast_to(alpha[None, :], (len(rows), cfg.n))
    Zr, _ = O.nearest_plane_sweep_blocked(W0[rows], L, Sr, cfg.block)
    ref = {"codes": Zr.astype(np.int64), "pi": np.arange(cfg.n), "Sp": np.array(Sr),
           "W0": W0[rows], "L": L}
    stats = check_codes(codes[rows], ref, None, label=cfg.name)
    log(f"{cfg.name}: sampled rows {stats}", t0)

    t0 = time.time()
    bits_g, mean_g, huff_g = P.column_entropy(out["codes"], huffman=True)
    torch.cuda.synchronize()
    bits_o = O.column_entropy_bits(codes)
    np.testing.assert_allclose(to_np(bits_g), bits_o, rtol=0, atol=1e-12)
    rate = float(np.mean(bits_o))
    assert abs(float(mean_g.item()) - rate) <= 1e-12
    assert abs(rate - spacing["target_bits"]) <= 0.005, rate
    huff_o = O.column_huffman_bits(codes)
    np.testing.assert_array_equal(to_np(huff_g), huff_o)
    log(f"{cfg.name}: rate {rate:.5f} bits at c = {c:.6g}, Huffman-coded "
        f"{huff_o.sum() / codes.size:.5f} bits/weight (GPU rate kernel agrees)", t0)

    t0 = time.time()
    D = W0 - alpha[None, :] * codes
    del codes
    loss = _trace_loss(D, H64)
    check_loss(res["loss"], loss, "spectral loss")
    check_loss(res["loss_damped"], loss, "spectral loss_d")
    S = np.broadcast_to(alpha[None, :], (cfg.m, cfg.n))
    check_loss(res["bound"], O.babai_bound(S, np.diag(L) ** 2), "spectral bound")
    # every spacing is c / l_kk, so each column's Theorem 5 term is c^2 / 4
    assert abs(res["bound"] - 0.25 * c * c * cfg.m * cfg.n) <= 1e-6 * res["bound"]
    log(f"{cfg.name}: losses {res['loss']:.6g} / bound {res['bound']:.6g}", t0)
