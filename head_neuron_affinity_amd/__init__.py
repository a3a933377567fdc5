"""MI355X-native head-to-neuron affinity pass.

Computes the calibration scores of "Affinity-Aware Sharding for Delayed Tensor
Parallelism" (section 3, "Affinity scores", eq. (5)) with hand-written HIP
kernels for gfx950 behind the C ABI in include/hna.h.  This package is a thin
ctypes binding: PyTorch provides device memory and streams only.
"""
from ._binding import (HnaError, HNA_BF16, HNA_F32, HNA_ACCUMULATE, hna_dims, hna_down_dims,
                       make_dims, lib, LIB_PATH, EXPORTED, fold_up_weights, down_col_sqnorm,
                       affinity_up, affinity_add, finalize_up, down_weight_norms, down_combine,
                       up_workspace_bytes, down_workspace_bytes, folded_bytes, status_string,
                       last_error, unit_mass, layout_objective, neuron_step,
                       head_step, layout_search, DUAL_ITERS, loo_workspace_bytes,
                       affinity_loo, static_scratch_bytes, affinity_up_static,
                       mfma_rate_probe)
from .pipeline import AffinityPass, StackPass, pass_for_layer, affinity_layer

__all__ = [
    "HnaError", "HNA_BF16", "HNA_F32", "HNA_ACCUMULATE", "hna_dims", "hna_down_dims", "make_dims",
    "lib", "LIB_PATH", "EXPORTED", "fold_up_weights", "down_col_sqnorm", "affinity_up", "affinity_add",
    "finalize_up", "down_weight_norms", "down_combine", "up_workspace_bytes",
    "down_workspace_bytes", "folded_bytes", "status_string", "last_error", "AffinityPass",
    "StackPass",
    "pass_for_layer", "affinity_layer", "unit_mass", "layout_objective",
    "neuron_step", "head_step", "layout_search", "DUAL_ITERS", "loo_workspace_bytes",
    "affinity_loo", "static_scratch_bytes", "affinity_up_static", "mfma_rate_probe",
]
