"""Algorithmic FLOP counts of the two Newton-Schulz forms.

Host-side bookkeeping for throughput reports.  n <= m are the small and large
sides of the matrix (X is n x m after orienting it wide), T the step count.

Two conventions:

* ``symmetric=True`` (the default) counts a product whose result is
  symmetric at half the dense cost, because only its upper-triangle tiles
  are computed (n^2 m for X X^T instead of 2 n^2 m);
* ``symmetric=False`` counts every product as a dense 2*rows*cols*inner.

Per step of the standard form ([Gram-NS] "Algorithm advantages: from
standard Newton-Schulz to Gram Newton-Schulz": three products per step):
A = X X^T (symmetric, inner m), A A (symmetric, inner n), B X (n x m, inner
n).

Gram form: one X X^T at the start, per step Z' = b R + c R^2 (one symmetric
n x n product), Q <- a Q + Z' Q (skipped at the first step after the start
or a restart, where Q = a I + Z'), the R update V = a R + Z' R,
R <- a V + Z' V (two symmetric products, skipped when no later step reads R),
per restart X <- Q X (dense) and X X^T, and the output Q X (dense).
"""

from __future__ import annotations

from typing import Iterable


def restart_set(mask: int) -> set:
    """Step numbers k (1-based) whose bit k is set in ``mask``."""
    return {k for k in range(1, 33) if (mask >> k) & 1}


def standard_flops(n: int, m: int, steps: int = 5,
                   symmetric: bool = True) -> float:
    n, m = min(n, m), max(n, m)
    sym = 1.0 if symmetric else 2.0
    per_step = sym * n * n * m + sym * n ** 3 + 2.0 * n * n * m
    return steps * per_step


def gram_flops(n: int, m: int, steps: int = 5,
               restarts: Iterable[int] = (4,),
               symmetric: bool = True) -> float:
    n, m = min(n, m), max(n, m)
    sym = 1.0 if symmetric else 2.0
    rs = {int(k) for k in restarts if int(k) > 1 and int(k) <= steps}
    nn = float(n) ** 3
    nnm = float(n) * n * m
    total = sym * nnm                                  # R = X0 X0^T
    fresh = True
    for k in range(1, steps + 1):
        if k in rs:
            total += 2.0 * nnm + sym * nnm             # X <- Q X ; R <- X X^T
            fresh = True
        total += sym * nn                              # Z' = b R + c R^2
        if not fresh:
            total += sym * nn                          # Q <- a Q + Z' Q
        fresh = False
        if k < steps and (k + 1) not in rs:
            total += 2.0 * sym * nn                    # V, then R
    total += 2.0 * nnm                                 # output Q X
    return total


def ns_flops(rows: int, cols: int, steps: int = 5, mode: str = "standard",
             restart_mask: int = 1 << 4, symmetric: bool = True) -> float:
    """FLOPs of one orthogonalization of a rows x cols matrix."""
    if mode == "standard":
        return standard_flops(rows, cols, steps, symmetric)
    if mode == "gram":
        return gram_flops(rows, cols, steps, restart_set(restart_mask),
                          symmetric)
    raise ValueError("mode must be 'standard' or 'gram'")
