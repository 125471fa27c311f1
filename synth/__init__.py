"""Seeded synthetic layer workloads for Hessian-weighted layer quantization.

This module is shared by the fp64 oracle's tests and by the GPU path's tests
and benchmark.  It holds only random draws, the bf16 storage format of those
draws and the table of workloads; none of the quantizer's arithmetic lives
here.

The pages measure on real LLM layers with WikiText-2 / C4 calibration data,
which are not available here, so seeded synthetic inputs with the shapes and
value distributions of those layers stand in for them:

* W entries are Gaussian (the usual initialisation-scale spread of trained
  projection weights).
* calibration activations X are heavy-tailed (Student-t with nu=4, or
  Laplace) with a few outlier channels scaled by 20, or with a LogNormal
  per-channel spread; the residual-drift page ("Residual-stream drift",
  RDQ) reports most LLM layer inputs to be non-Gaussian, and the GPTQ/Babai
  page (section 3) stresses outlier weights.
* the unequal-rate (ZSIC) workload is given a Hessian H = L0 diag(lam) L0^T
  with L0 unit lower triangular and a spectrum decaying as k^-1.2.

Every array is produced from numpy's PCG64 seeded through
``SeedSequence([2026, workload, ...])``; X is generated in fixed chunks of
8192 tokens, each from its own spawned child stream, so parallel generation
is reproducible bit for bit.
"""
from .configs import CONFIGS, LayerConfig, config
from .gen import (Layer, bf16_bits_to_f32, f32_to_bf16_bits, make_layer,
                  make_weight, make_activations, make_spectral_hessian)

__all__ = ["CONFIGS", "LayerConfig", "config", "Layer", "bf16_bits_to_f32",
           "f32_to_bf16_bits", "make_layer", "make_weight",
           "make_activations", "make_spectral_hessian"]
