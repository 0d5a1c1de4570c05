"""CPU float64 oracle for the Prism estimator and block-sparse attention.

Test infrastructure: imported only by the test suite, the smoke check and the
benchmark's CPU-baseline leg. It imports nothing from the HIP package.
"""
from .prism_oracle import (admissible, attention_block_row, band_dims, band_rms, band_scores, kv_head,
                           block_sparse_attention, estimate, estimate_head, mean_pool, temperature,
                           top_p, top_p_mask, union)

__all__ = ["admissible", "attention_block_row", "band_dims", "band_rms", "band_scores",
           "block_sparse_attention", "estimate", "estimate_head", "kv_head", "mean_pool", "temperature",
           "top_p", "top_p_mask", "union"]
