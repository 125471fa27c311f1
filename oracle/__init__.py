"""fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The HIP product path never imports, links or
runs anything here, and nothing here imports the HIP path.
"""
from .babai_oracle import (babai_bound, babai_gram_schmidt, certificate,
                           cholesky_lower, colspacing_steps,
                           column_entropy_bits, column_huffman_bits, cvp_box,
                           cvp_enumerate, huffman_cost,
                           expand_group_steps, fix_dead_and_damp,
                           gamma_ratio, gptq_obs_sweep, grid_steps, hessian,
                           nearest_plane_sweep, nearest_plane_sweep_blocked,
                           min_pivot_order, order_permutation, proxy_loss,
                           quant_layer)
from .babai_oracle import code_range, overflow_entries, ssqr_search
from .babai_oracle import (oaem_blocks, oaem_estep, oaem_init, oaem_mstep,
                           oaem_objective)
