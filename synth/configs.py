"""The five layer workloads (shapes, distributions, grid, block, damping).

Grid kinds: "sym" (symmetric, per row or per group of columns), "asym"
(asymmetric with an integer zero point), "colspacing" (one lattice spacing per
input column, alpha_i = c / L_ii).  ``group`` 0 means one step per row.
"""
from dataclasses import dataclass, field, replace
from typing import Optional


@dataclass(frozen=True)
class LayerConfig:
    key: int                 # workload number 1..5
    name: str
    m: int                   # d_out, rows of W
    n: int                   # d_in, columns of W
    ntok: int                # calibration tokens (0 when H is given)
    wdtype: str              # "f32" | "bf16"
    xdtype: str              # "f32" | "bf16" | "" (H given)
    w_std: float
    x_kind: str              # "gauss_lognormal" | "student_t" | "laplace_lognormal" | "spectral_h"
    x_param: float           # LogNormal sigma, Student-t nu, or spectral decay exponent
    outliers: int = 0
    outlier_scale: float = 20.0
    grid_kind: str = "sym"
    bits: int = 4
    group: int = 0
    colspacing_c: float = 0.0
    block: int = 128
    damp: float = 0.01
    order: str = "back_to_front"

    def resized(self, m: Optional[int] = None, n: Optional[int] = None,
                ntok: Optional[int] = None, **kw) -> "LayerConfig":
        """Same recipe at another shape (for oracle-sized parity cases)."""
        return replace(self, m=self.m if m is None else m,
                       n=self.n if n is None else n,
                       ntok=self.ntok if ntok is None else ntok, **kw)


CONFIGS = {
    1: LayerConfig(1, "tiny", 64, 128, 2048, "f32", "f32", 0.02,
                   "gauss_lognormal", 0.5, grid_kind="sym", bits=4, group=0,
                   block=32, damp=0.01),
    2: LayerConfig(2, "q_proj", 4096, 4096, 131072, "bf16", "bf16", 0.02,
                   "student_t", 4.0, outliers=8, grid_kind="asym", bits=4,
                   group=128, block=128, damp=0.01),
    3: LayerConfig(3, "up_proj", 14336, 4096, 262144, "bf16", "bf16", 0.015,
                   "student_t", 4.0, outliers=16, grid_kind="sym", bits=3,
                   group=128, block=128, damp=0.01),
    4: LayerConfig(4, "down_proj", 4096, 14336, 262144, "bf16", "bf16", 0.01,
                   "laplace_lognormal", 1.0, grid_kind="sym", bits=2,
                   group=64, block=128, damp=0.01),
    # c is fixed by a rate search (mean per-column code entropy 2.5 bits);
    # the value here is a placeholder replaced by the searched one.
    5: LayerConfig(5, "zsic_down_proj_70b", 8192, 28672, 0, "bf16", "", 0.01,
                   "spectral_h", 1.2, grid_kind="colspacing", bits=0,
                   group=0, colspacing_c=1.0, block=256, damp=0.0),
}


def config(key: int) -> LayerConfig:
    return CONFIGS[key]
