"""Token-major activations (X stored [ntok, n], one row per token): the
Hessian and the whole layer through the C ABI with PWQ_X_TOKEN_MAJOR.

The matrix is the same X as in the channel-major tests, so H is compared
with the oracle's fp64 Hessian of X to the same tolerance.  Where both
layouts take the same kernel family (both operands reach the MFMA units as
the same 8-token runs in the same order), H is also bitwise equal to the
channel-major result.
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_19_amd as P
import synth
from _gpu import to_np, upload
from _parity import TOL_H, rel_fro

pytestmark = pytest.mark.gpu


def _tm(X):
    """The same matrix stored token-major (a device copy)."""
    return X.t().contiguous()


# (n, ntok, dtype, same kernel family in both layouts)
CASES = [
    (384, 4096, "bf16", True),     # 128 tiles, element-gathered loads
    (130, 1000, "bf16", True),     # ragged channels and tokens
    (1100, 3000, "bf16", False),   # n % 8 != 0: channel-major takes 256 tiles, tokens 128
    (1104, 3000, "bf16", True),    # 256 tiles, transposed LDS reads, ragged both ways
    (2048, 20480, "bf16", True),   # 256 tiles, split over the token axis
    (256, 2000, "f32", True),
]


@pytest.mark.parametrize("n,ntok,dt,same", CASES)
def test_token_major_hessian(n, ntok, dt, same):
    cfg = synth.config(2).resized(m=16, n=n, ntok=ntok)
    lay = synth.make_layer(cfg)
    _, X, _ = upload(lay)
    if dt == "f32":
        X = X.float()
    print(f"[token-major] n={n} ntok={ntok} {dt}", flush=True)
    Hc = P.hessian_accum(X)
    Ht = P.hessian_accum(_tm(X), x_layout="tokens")
    torch.cuda.synchronize()
    Hg = to_np(Ht)
    assert np.array_equal(Hg, Hg.T)
    assert rel_fro(Hg, O.hessian(lay.X64())) <= TOL_H
    if same:
        assert np.array_equal(Hg, to_np(Hc))
    # accumulation into a previous H
    H2 = P.hessian_accum(_tm(X), H=Ht.clone(), accumulate=True, x_layout="tokens")
    torch.cuda.synchronize()
    assert rel_fro(to_np(H2), 2 * Hg) <= 1e-6


def test_token_major_padded_rows_and_empty():
    """Row stride above n (a view into wider rows), and no tokens."""
    cfg = synth.config(2).resized(m=16, n=1024, ntok=640)
    lay = synth.make_layer(cfg)
    _, X, _ = upload(lay)
    wide = torch.zeros((640, 1024 + 64), dtype=X.dtype, device=X.device)
    wide[:, :1024] = X.t()
    Ht = P.hessian_accum(wide[:, :1024], x_layout="tokens")
    torch.cuda.synchronize()
    assert np.array_equal(to_np(Ht), to_np(P.hessian_accum(X)))
    He = P.hessian_accum(torch.empty((0, 96), dtype=torch.bfloat16, device="cuda"),
                         x_layout="tokens")
    torch.cuda.synchronize()
    assert He.shape == (96, 96) and np.all(to_np(He) == 0)


def test_token_major_layer_matches_channel_major():
    """The whole layer from token-major X: same H bitwise, hence the same
    factor, codes and losses as from channel-major X."""
    cfg = synth.config(2).resized(m=96, n=1024, ntok=4096)
    lay = synth.make_layer(cfg)
    W, X, _ = upload(lay)
    g = P.Grid(cfg.grid_kind, cfg.bits, cfg.group)
    a = P.quant_layer(W, X=X, grid=g, damp=cfg.damp, block=cfg.block, want_H=True)
    b = P.quant_layer(W, X=_tm(X), grid=g, damp=cfg.damp, block=cfg.block, want_H=True,
                      x_layout="tokens")
    torch.cuda.synchronize()
    assert np.array_equal(to_np(a["H"]), to_np(b["H"]))
    assert np.array_equal(to_np(a["codes"]), to_np(b["codes"]))
    ra, rb = P.read_result(a["result"]), P.read_result(b["result"])
    assert ra["loss"] == rb["loss"] and ra["bound"] == rb["bound"]
    with pytest.raises(ValueError):
        P.quant_layer(W, X=X, grid=g, x_layout="tokens")      # [n, ntok] read as [ntok, n]
