"""Newton-Schulz orthogonalization for AMD Instinct MI355X (gfx950).

Python face of ``libnsortho.so``: the standard and Gram forms of quintic
Newton-Schulz (Muon's approximate polar factor), a batched launcher for
equal-shape expert matrices, the ROOT soft-threshold split, ROOT's per-shape
coefficient schedules (fitted on the host, run through the per-step
coefficient arrays) and a whole Muon step (momentum, orthogonalization,
weight update).  The HIP
library does all the work; this package only marshals arguments.
"""

from .flops import gram_flops, ns_flops, standard_flops
from ._binding import (NS_MAX_STEPS, TUNED_ABC, NSError, lib, muon_step,
                       muon_workspace_size, orthogonalize,
                       orthogonalize_batched, orthogonalize_grouped,
                       orthogonalize_static, grouped_workspace_size,
                       plan_kernels,
                       soft_threshold_split, status_code, status_string,
                       workspace_size)
from .coeffs import fit_coefficients, root_coefficients

__all__ = [
    "NS_MAX_STEPS", "TUNED_ABC", "NSError", "lib", "muon_step",
    "muon_workspace_size", "orthogonalize",
    "orthogonalize_batched", "orthogonalize_grouped", "orthogonalize_static",
    "grouped_workspace_size", "plan_kernels", "soft_threshold_split",
    "status_code", "status_string",
    "workspace_size", "gram_flops", "ns_flops", "standard_flops",
    "fit_coefficients", "root_coefficients",
]
