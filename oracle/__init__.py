"""CPU oracle for the small_fc_lopt optimizer step.

TEST INFRASTRUCTURE ONLY: imported by tests/, ``__graft_entry__.smoke()`` and
``bench.py``'s cpu_baseline leg.  Nothing in the product path may import it.
"""
from .small_fc_lopt import (Hyper, Mlp, N_FEATURES, VELO_FEATURES, FEATURE_SETS, HIDDEN, DEFAULT_TIMESCALES, accumulate,
                            as_matrix, cross_index, feature_scales, features, mlp_forward,
                            mlp_size, pack_mlp, step, step_tensor, step_tensor_rows, step_tensor_sub, time_features, unpack_mlp,
                            update_from_output, zero_state)

__all__ = ["Hyper", "Mlp", "N_FEATURES", "VELO_FEATURES", "FEATURE_SETS", "HIDDEN", "DEFAULT_TIMESCALES", "accumulate", "as_matrix",
           "cross_index", "feature_scales", "features", "mlp_forward", "mlp_size", "pack_mlp",
           "step", "step_tensor", "step_tensor_rows", "step_tensor_sub", "time_features", "unpack_mlp", "update_from_output", "zero_state"]
