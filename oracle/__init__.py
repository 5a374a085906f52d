"""Plain fp64 CPU oracle for quintic Newton-Schulz orthogonalization.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check and the CPU
baseline leg of the benchmark use it.  It shares no code with the HIP
library (no kernels, headers, constants or helpers); the two meet only in
the seeded input generators of ``workloads``, which hold none of the
method's arithmetic.

Sources (web pages; cited by title and section):

* [Gram-NS] "GPU speeds up again! The Gram Newton-Schulz algorithm cuts
  optimizer time of trillion-parameter MoE models by 40-50%" (itsolotime.com,
  a Thai translation of the Dao-lab Gram Newton-Schulz blog post); sections
  "Algorithm advantages: from standard Newton-Schulz to Gram Newton-Schulz",
  "Stability challenges and solutions", "Performance comparison and real
  applications".
* [NanoGPT-Muon] "Training 124M-parameter NanoGPT in 2 minutes: the Muon
  optimizer and engineering reproduction" (blog.hotdry.top); sections "From
  SGD to Muon", "Coefficient tuning of the Newton-Schulz iteration and FLOP
  overhead", "Engineering reproduction checklist", "Monitoring metrics".
* [ROOT] the ROOT optimizer summary on the reportify.cn concept page "large
  model training optimization"; items "limitations of existing optimizers"
  and "technical innovations of ROOT".

What each function follows, and every reading taken where the pages are
silent or garbled, is stated in its docstring.

Pins (tests marked ``not gpu`` check the oracle against facts that do not
come from the oracle itself):

* ``ns_standard``: converges to the Jacobi-SVD polar factor on tiny inputs
  with the (2, -1.5, 0.5) triple; matches the closed form
  ``U diag(p^T(s)) V^T`` on designed spectra; reproduces the ROOT page's
  printed 2048 x 2048 orthogonalization MSE; equivariance invariants.
* ``ns_gram``: equals ``ns_standard`` in fp64 (with and without restart) and
  matches the same closed form.
* ``gram_iterate``: the recurrence ``ns_gram`` runs; started from a Gram
  matrix with one eigenvalue made negative, its action along that
  eigenvector matches the scalar recurrence mu <- mu (a + b mu + c mu^2)^2
  (the naive iteration grows it without bound), and a restart brings the
  result back into the scalar map's band.
* ``jacobi_svd`` / ``polar_jacobi``: against ``numpy.linalg.svd`` and the
  defining properties (orthonormal factors, reconstruction).
* ``polar_eigh``: against ``polar_jacobi`` and the isometry property.
* ``soft_threshold_split``: the closed form of the l1 proximal step, its
  subgradient optimality conditions and Student-t(2) order statistics.
* ``lower_median_abs``: brute-force sort on small inputs.
* ``muon_step`` / ``momentum_update``: the momentum recurrence against its
  geometric-series closed form for a constant gradient, and the whole step
  against ``W - lr U diag(p^T(s/||s||)) V^T`` on a designed spectrum.

No function here is "parity unpinned".
"""

from .ns import (CLASSIC_ABC, TUNED_ABC, coefficient_schedule, frobenius_stage,
                 gram_iterate, ns_gram, ns_standard, scalar_map)
from .svd import jacobi_svd, polar_eigh, polar_jacobi, orthogonalization_mse
from .soft_threshold import lower_median_abs, soft_threshold_split
from .muon import momentum_update, muon_step

__all__ = [
    "CLASSIC_ABC", "TUNED_ABC", "coefficient_schedule", "frobenius_stage",
    "gram_iterate", "ns_gram", "ns_standard", "scalar_map", "jacobi_svd", "polar_eigh",
    "polar_jacobi", "orthogonalization_mse", "lower_median_abs",
    "soft_threshold_split", "momentum_update", "muon_step",
]
