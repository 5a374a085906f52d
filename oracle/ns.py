"""fp64 Newton-Schulz iterations: the standard form and the Gram form.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Standard form ([Gram-NS], "Algorithm advantages: from standard Newton-Schulz
to Gram Newton-Schulz"; [NanoGPT-Muon], "From SGD to Muon" and "Coefficient
tuning of the Newton-Schulz iteration and FLOP overhead").  The displayed
iteration did not survive extraction; what survives fixes it:

* each iteration uses three matrix products;
* the update is an odd polynomial p(t) = a t + b t^3 + c t^5 applied to the
  singular values (p(t) = t q(t^2));
* the coefficients come as a triple (a, b, c), tuned (3.4445, -4.7750,
  2.0315) or classic (2, -1.5, 0.5), five steps.

The one odd quintic matrix polynomial with a coefficient triple and three
products is ``X <- a X + (b A + c A^2) X`` with ``A = X X^T``.

Readings taken where the pages are silent:

* orientation: X is n x m with n <= m (the Gram-NS article's X in R^{n x m},
  aspect alpha = m/n > 1); a tall input is transposed first and the result is
  transposed back; a square input is not transposed;
* normalization: Frobenius, ``X / (||X||_F + eps)`` with eps = 1e-7, which
  puts every singular value in [0, 1];
* coefficients: the same triple every step unless a per-step list is given.

Gram form ([Gram-NS], "Algorithm advantages ..." and "Stability challenges
and solutions").  The article states that the iteration is moved onto the
Gram matrix R = X X^T by writing the odd polynomial as t q(t^2), that the
accumulated matrix approximates R^{-1/2}, and that the stabilized version
adds a restart that re-initializes the Gram matrix.  Written out:

* X_k = Q_k X_0 with Q_k a polynomial in R_0 (so all of them commute);
* Z_k = a I + b R_k + c R_k^2, X_{k+1} = Z_k X_k, so Q_{k+1} = Z_k Q_k;
* R_{k+1} = X_{k+1} X_{k+1}^T = Z_k R_k Z_k;
* restart before step k (reading: the plainest one): X <- Q X, R <- X X^T
  recomputed from scratch, Q <- I;
* output Q X.

Default restart set {4} (restart once, before step 4 of 5).  The article
does not say when to restart; before step 4 costs the same as before step 3
and, in fp16 storage, is as accurate as restarting twice ({2, 4}).  An empty
set is the naive Gram iteration.
"""

from __future__ import annotations

from typing import Iterable, List, Sequence, Tuple, Union

import numpy as np

TUNED_ABC = (3.4445, -4.7750, 2.0315)
CLASSIC_ABC = (2.0, -1.5, 0.5)
DEFAULT_EPS = 1e-7

Triple = Tuple[float, float, float]


def coefficient_schedule(abc: Union[Triple, Sequence[Triple]],
                         steps: int) -> List[Triple]:
    """Per-step (a, b, c): one triple repeated, or an explicit list."""
    arr = np.asarray(abc, dtype=np.float64)
    if arr.shape == (3,):
        return [tuple(float(v) for v in arr)] * steps
    if arr.ndim != 2 or arr.shape[1] != 3 or arr.shape[0] != steps:
        raise ValueError("abc must be one triple or `steps` triples")
    return [tuple(float(v) for v in row) for row in arr]


def frobenius_stage(m: np.ndarray, eps: float = DEFAULT_EPS):
    """Orient to wide (rows <= cols) and divide by ||X||_F + eps.

    Returns (X0, transposed).  The input is taken as stored values upcast to
    fp64, exactly as the device sees them.
    """
    x = np.asarray(m, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("expects a 2-D matrix")
    transposed = x.shape[0] > x.shape[1]
    if transposed:
        x = x.T
    nrm = np.sqrt(np.sum(x * x))
    return x / (nrm + eps), transposed


def scalar_map(sigma, abc: Union[Triple, Sequence[Triple]] = TUNED_ABC,
               steps: int = 5):
    """The iteration's action on one singular value: p applied ``steps`` times.

    ``sigma`` is a singular value of the normalized matrix.  Used by the
    closed-form checks: for M = U diag(s) V^T the standard iteration returns
    U diag(scalar_map(s / ||s||_2)) V^T.
    """
    y = np.asarray(sigma, dtype=np.float64).copy()
    for a, b, c in coefficient_schedule(abc, steps):
        y = a * y + b * y ** 3 + c * y ** 5
    return y


def ns_standard(m: np.ndarray, steps: int = 5,
                abc: Union[Triple, Sequence[Triple]] = TUNED_ABC,
                eps: float = DEFAULT_EPS) -> np.ndarray:
    """Standard quintic Newton-Schulz in fp64.

    For each step: A = X X^T; B = b A + c A A; X <- a X + B X.  Three matrix
    products per step, as the Gram-NS article counts them.
    """
    x, transposed = frobenius_stage(m, eps)
    for a, b, c in coefficient_schedule(abc, steps):
        gram = x @ x.T
        poly = b * gram + c * (gram @ gram)
        x = a * x + poly @ x
    return x.T if transposed else x


def ns_gram(m: np.ndarray, steps: int = 5,
            abc: Union[Triple, Sequence[Triple]] = TUNED_ABC,
            restart: Iterable[int] = (4,),
            eps: float = DEFAULT_EPS) -> np.ndarray:
    """Gram Newton-Schulz in fp64, with restarts before the listed steps.

    ``restart`` holds 1-based step numbers; a restart before step 1 is a
    no-op.  Returns Q X, oriented like the input.
    """
    x, transposed = frobenius_stage(m, eps)
    out = gram_iterate(x, x @ x.T, coefficient_schedule(abc, steps), restart)
    return out.T if transposed else out


def gram_iterate(x: np.ndarray, r: np.ndarray, sched: Sequence[Triple],
                 restart: Iterable[int] = (4,)) -> np.ndarray:
    """The Gram recurrence from a given start: Q X after ``len(sched)`` steps.

    ``x`` is the wide, normalized iterate and ``r`` the Gram matrix the
    iteration starts from (X X^T for ns_gram).  Taking ``r`` as an argument
    lets a test start from a Gram matrix that lost positive
    semi-definiteness, the failure the Gram-NS article describes for naive
    Gram iterations in float16 ("Stability challenges and solutions"); a
    restart recomputes R from X and so discards it.
    """
    restart = set(int(k) for k in restart)
    n = x.shape[0]
    eye = np.eye(n)
    q = eye.copy()
    for k, (a, b, c) in enumerate(sched, start=1):
        if k in restart and k > 1:
            x = q @ x
            r = x @ x.T
            q = eye.copy()
        z = a * eye + b * r + c * (r @ r)
        q = z @ q
        r = z @ r @ z
    return q @ x
