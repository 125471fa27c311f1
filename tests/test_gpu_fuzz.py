"""Seeded random small layers through the whole GPU path, each against the
oracle on the GPU's own Hessian (stage-fed, as the parity tests): shapes
from a single row or column up to several tiles with ragged edges, every
grid kind with random bits and group sizes, every block size, every
processing order, X in fp32 or bf16 stored either way, fp32 or fp64 factor
and sweep.  The case is printed before it runs."""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_19_amd as P
import synth
from _gpu import to_np, upload
from _parity import TOL_L, TOL_STEP, check_codes, check_loss, lattice_ints, rel_fro

pytestmark = pytest.mark.gpu

ORDERS = ["back_to_front", "front_to_back", "act_order", "perm", "min_pivot"]


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    base = int(rng.choice([1, 2, 3, 4, 5]))
    m = int(rng.choice([1, 2, 7, 16, 33, 64, 97]))
    n = int(rng.choice([1, 3, 16, 40, 64, 130, 200, 256, 384, 513, 640]))
    cfg = synth.config(base)
    if base == 5:
        cfg = cfg.resized(m=m, n=n)
        kind, bits, group, c = "colspacing", 0, 0, float(rng.choice([1e-3, 3e-3, 1e-2]))
    else:
        ntok = int(rng.choice([n + 1, 2 * n + 5, 1024, 3000]))
        cfg = cfg.resized(m=m, n=n, ntok=ntok)
        kind = str(rng.choice(["sym", "asym"]))
        bits = int(rng.integers(2, 9))
        groups = [0] + [g for g in (8, 16, 32, 64, 128) if n % g == 0 and g < n]
        group = int(rng.choice(groups))
        c = 0.0
    block = int(rng.choice([32, 64, 128, 256]))
    order = str(rng.choice(ORDERS))
    prec = "f64" if base == 5 or rng.random() < 0.2 else "f32"
    layout = str(rng.choice(["channels", "tokens"]))
    return dict(base=base, cfg=cfg, kind=kind, bits=bits, group=group, c=c, block=block,
                order=order, prec=prec, layout=layout, perm_seed=int(rng.integers(1 << 30)))


@pytest.mark.parametrize("seed", range(64))
def test_random_layer(seed):
    k = _case(seed)
    cfg = k["cfg"]
    print(f"[fuzz {seed}] config {k['base']} m={cfg.m} n={cfg.n} ntok={cfg.ntok} "
          f"{k['kind']} bits={k['bits']} group={k['group']} c={k['c']} block={k['block']} "
          f"order={k['order']} prec={k['prec']} layout={k['layout']}", flush=True)
    lay = synth.make_layer(cfg)
    W, X, H = upload(lay)
    if X is not None and k["layout"] == "tokens":
        X = X.t().contiguous()
    perm = perm_np = None
    if k["order"] == "perm":
        perm_np = np.random.default_rng(k["perm_seed"]).permutation(cfg.n)
        perm = torch.from_numpy(perm_np.astype(np.int32)).cuda()
    grid = P.Grid(k["kind"], k["bits"], k["group"], k["c"])
    out = P.quant_layer(W, X=X, H=H, grid=grid, order=k["order"], perm=perm, damp=cfg.damp,
                        block=k["block"], prec=k["prec"], want_H=X is not None, want_L=True,
                        x_layout=k["layout"] if X is not None else "channels")
    torch.cuda.synchronize()
    r = P.read_result(out["result"])
    assert r["info"] == 0, r
    Hg = to_np(out["H"]).astype(np.float64) if X is not None else lay.H.astype(np.float64)
    ref = O.quant_layer(lay.W64(), H=Hg, grid_kind=k["kind"], bits=k["bits"],
                        group=k["group"], c=k["c"] if k["c"] else 1.0, order=k["order"],
                        perm=perm_np, damp=cfg.damp)
    assert rel_fro(to_np(out["L"]), ref["L"]) <= (TOL_L if k["prec"] == "f32" else 1e-9)
    assert r["lambda"] == pytest.approx(ref["lam"], rel=1e-9, abs=1e-300)
    np.testing.assert_allclose(to_np(out["scales"]), ref["scales"], rtol=TOL_STEP)
    zeros = to_np(out["zeros"]) if out["zeros"] is not None else None
    if zeros is not None:
        np.testing.assert_array_equal(zeros, ref["zeros"])
    # Every code must be a nearest rounding within 1e-5 of a midpoint (the
    # certificate inside check_codes), so every mismatch is a tie.  With bf16
    # weights and steps (max - min) / (2^b - 1), w / s often falls exactly on
    # a midpoint, and the fp32 and fp64 sides then break the tie by their
    # rounding noise: a couple of such codes in a layer of a few hundred
    # exceed 0.1%, so small layers need 98% identical rather than 99.9%.
    codes = to_np(out["codes"])
    stats = check_codes(codes, ref, zeros, label=f"fuzz {seed}",
                        min_identical=0.999 if codes.size >= 10000 else 0.98)
    check_loss(r["bound"], ref["bound"], f"fuzz {seed} bound")
    # The losses of the GPU's own codes, in the oracle's fp64 arithmetic
    # (after a tie the two sides' later codes in that row may differ, and a
    # layer of a few hundred codes feels that in its loss).  Relative
    # tolerance, with an absolute floor of 1e-9 of the Theorem 5 bound: a
    # layer whose weights sit on their lattice points has a loss of zero up
    # to rounding, where no relative tolerance applies.
    n = cfg.n
    S = np.empty_like(ref["Sp"])
    S[:, ref["pi"]] = ref["Sp"]
    D = ref["W0"] - S * lattice_ints(codes, zeros, n)
    loss = float(np.sum((D @ Hg) * D))
    want = {"loss": loss, "loss_damped": loss + ref["lam"] * float(np.sum(D * D))}
    floor = 1e-9 * ref["bound"]
    for key, w in want.items():
        if abs(w) > 1e3 * floor:
            check_loss(r[key], w, f"fuzz {seed} {key}")
        else:
            assert abs(r[key] - w) <= floor, (key, r[key], w)
    print(f"[fuzz {seed}] {stats}", flush=True)
