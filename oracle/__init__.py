"""CPU oracle for DyRA (test infrastructure only; see dyra_oracle)."""
from .dyra_oracle import (OraclePlan, als, dense_product, factors_instance, inference,  # noqa: F401
                          inference_instance, newton_schulz_inv_sqrt, offline_preparation, optimal_rank_error,
                          blast_matrix, offline_preparation_blast,
                          rel_fro, right_factor, right_factor_ns, truncated_svd, weight_only)
