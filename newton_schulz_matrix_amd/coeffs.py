"""Per-shape Newton-Schulz coefficients (ROOT's adaptive iteration).

[ROOT] "technical innovations of ROOT": instead of one fixed triple for
every matrix, the iteration gets fine-grained coefficients tailored to the
matrix size (m, n); on 2048 x 8192 the page reports the orthogonalization
MSE falling from 0.0761 to 0.00033.  The page gives no fitting procedure;
this module fits them as follows (host side, offline; the kernels only
receive the per-step arrays).

* After Frobenius normalization the iteration acts on each singular value
  sigma of X independently: sigma -> p_T(...p_1(sigma)), with
  p_k(x) = a_k x + b_k x^3 + c_k x^5.  The page's MSE (the squared
  Frobenius error against polar(M), per singular value) is therefore the
  mean of (p_T o ... o p_1(sigma_i) - 1)^2 over the singular values.
* For an i.i.d. Gaussian r x c matrix (n = min, m = max, lambda = n / m)
  the eigenvalues mu of X X^T / m follow the Marchenko-Pastur law on
  [(1 - sqrt(lambda))^2, (1 + sqrt(lambda))^2] with mean 1, so after
  normalization sigma_i = sqrt(mu_i / n).  `mp_singular_values` returns
  `count` quantiles of that law.
* `fit_coefficients` minimizes the mean squared error over those quantiles
  (scipy least squares, started from the tuned triple) plus a penalty on
  any intermediate value of the composed map outside [0, bound] for sigma
  in [0, 1] (the fitted maps stay within about [-0.002, bound + 0.02]): a
  real matrix's singular values need not follow the law, and bounded
  intermediates keep the fp16 state of the kernels safe.

`root_coefficients(rows, cols)` returns the stored fit for a shape from
``coeff_table.json`` (written by ``python -m newton_schulz_matrix_amd.coeffs
--write``), fitting on the spot (seconds to a minute) for shapes not in it.
"""

from __future__ import annotations

import argparse
import json
import os
from typing import Dict, List, Sequence, Tuple

import numpy as np

from ._binding import TUNED_ABC

TABLE_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "coeff_table.json")

# Shapes of the bench workloads and of the pages' examples, (rows, cols).
TABLE_SHAPES = [
    (2048, 2048), (2048, 8192), (4096, 4096), (4096, 14336), (1408, 2048),
    (768, 768), (768, 3072), (256, 1024),
]

Triple = Tuple[float, float, float]


def mp_singular_values(rows: int, cols: int, count: int = 256, grid: int = 8001) -> np.ndarray:
    """`count` quantiles of the normalized singular values of a Gaussian matrix.

    Quantile i is at probability (i + 1/2) / count of the Marchenko-Pastur
    law with ratio n / m, mapped to sigma = sqrt(mu / n).  The density is
    integrated in the angle theta of mu = lo + (hi - lo)(1 - cos theta) / 2,
    where it has no endpoint singularity.
    """
    n, m = min(rows, cols), max(rows, cols)
    if n < 1:
        raise ValueError("empty shape")
    lam = n / m
    lo, hi = (1.0 - np.sqrt(lam)) ** 2, (1.0 + np.sqrt(lam)) ** 2
    theta = np.linspace(0.0, np.pi, grid)
    mu = lo + (hi - lo) * (1.0 - np.cos(theta)) / 2.0
    if lo > 0.0:
        dens = (hi - lo) ** 2 / 4.0 * np.sin(theta) ** 2 / (2.0 * np.pi * lam * mu)
    else:  # lambda = 1: the 1/mu factor cancels against sin^2 / (1 - cos)
        dens = (1.0 + np.cos(theta)) / np.pi
    cdf = np.concatenate([[0.0], np.cumsum((dens[1:] + dens[:-1]) / 2.0 * np.diff(theta))])
    cdf /= cdf[-1]
    probs = (np.arange(count) + 0.5) / count
    return np.sqrt(np.interp(probs, cdf, mu) / n)


def composed(coeffs: Sequence[Triple], x: np.ndarray, clip: float = 4.0) -> List[np.ndarray]:
    """Values after each step of the scalar map (clipped to +-clip for the fit)."""
    out = []
    y = np.asarray(x, dtype=np.float64)
    for a, b, c in coeffs:
        y = np.clip(a * y + b * y ** 3 + c * y ** 5, -clip, clip)
        out.append(y)
    return out


def predicted_mse(coeffs: Sequence[Triple], sigma: np.ndarray) -> float:
    """Mean of (p_T o ... o p_1(sigma) - 1)^2: the page's MSE for that spectrum."""
    y = composed(coeffs, sigma, clip=np.inf)[-1]
    return float(np.mean((y - 1.0) ** 2))


def fit_coefficients(rows: int, cols: int, steps: int = 5, bound: float = 1.3,
                     count: int = 256, weight: float = 10.0) -> List[Triple]:
    """Per-step (a, b, c) minimizing the predicted MSE for a Gaussian rows x cols matrix."""
    from scipy.optimize import least_squares

    sigma = mp_singular_values(rows, cols, count)
    guard = np.linspace(0.0, 1.0, 201)

    def residuals(p):
        cf = p.reshape(steps, 3)
        r = [(composed(cf, sigma)[-1] - 1.0) / np.sqrt(count)]
        for y in composed(cf, guard):
            r.append(weight * np.maximum(y - bound, 0.0))
            r.append(weight * np.maximum(-y, 0.0))
        return np.concatenate(r)

    best = None
    for scale in (1.0, 1.2):
        x0 = np.array(TUNED_ABC * steps, dtype=np.float64)
        x0[0::3] *= scale
        res = least_squares(residuals, x0, method="trf", max_nfev=4000, xtol=1e-12, ftol=1e-14)
        if best is None or res.cost < best.cost:
            best = res
    return [tuple(float(v) for v in row) for row in best.x.reshape(steps, 3)]


def _key(rows: int, cols: int, steps: int) -> str:
    return f"{min(rows, cols)}x{max(rows, cols)}/T{steps}"


_cache: Dict[str, List[Triple]] = {}


def load_table(path: str = TABLE_PATH) -> dict:
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        return json.load(f)["entries"]


def root_coefficients(rows: int, cols: int, steps: int = 5) -> List[Triple]:
    """Per-step coefficients for a rows x cols matrix (orientation does not matter)."""
    key = _key(rows, cols, steps)
    if key not in _cache:
        entry = load_table().get(key)
        _cache[key] = ([tuple(t) for t in entry["coefficients"]] if entry is not None
                       else fit_coefficients(rows, cols, steps))
    return list(_cache[key])


def write_table(path: str = TABLE_PATH, steps: int = 5) -> dict:
    entries = {}
    for rows, cols in TABLE_SHAPES:
        cf = fit_coefficients(rows, cols, steps)
        sigma = mp_singular_values(rows, cols)
        entries[_key(rows, cols, steps)] = {
            "coefficients": [list(t) for t in cf],
            "predicted_mse": predicted_mse(cf, sigma),
            "predicted_mse_tuned": predicted_mse([TUNED_ABC] * steps, sigma),
        }
        print(f"{rows}x{cols}: predicted MSE {entries[_key(rows, cols, steps)]['predicted_mse']:.3e} "
              f"(tuned triple {entries[_key(rows, cols, steps)]['predicted_mse_tuned']:.3e})", flush=True)
    doc = {
        "about": "Per-shape Newton-Schulz coefficients fitted by newton_schulz_matrix_amd/coeffs.py "
                 "(Marchenko-Pastur spectrum of a Gaussian matrix, Frobenius normalization, "
                 "intermediate values kept in [0, 1.3] on [0, 1]). Keys: n x m / T steps.",
        "entries": entries,
    }
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")
    return doc


def main() -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--write", action="store_true", help="refit every table shape and rewrite the table")
    ap.add_argument("--shape", type=int, nargs=2, metavar=("ROWS", "COLS"), help="fit one shape and print it")
    ap.add_argument("--steps", type=int, default=5)
    args = ap.parse_args()
    if args.write:
        write_table(steps=args.steps)
    elif args.shape:
        cf = fit_coefficients(args.shape[0], args.shape[1], args.steps)
        sigma = mp_singular_values(*args.shape)
        print(json.dumps({"coefficients": cf, "predicted_mse": predicted_mse(cf, sigma),
                          "predicted_mse_tuned": predicted_mse([TUNED_ABC] * args.steps, sigma)}))
    else:
        ap.print_help()


if __name__ == "__main__":
    main()
