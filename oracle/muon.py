"""One Muon optimizer step in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[Gram-NS], "Algorithm advantages: from standard Newton-Schulz to Gram
Newton-Schulz": Muon is steepest descent under the spectral norm; its update
(the displayed formula did not survive extraction) involves a momentum
coefficient mu, a learning rate eta and the polar factor of the momentum.
[NanoGPT-Muon], "Engineering reproduction checklist": momentum 0.95 with
Nesterov, five Newton-Schulz steps.

Reading (the plainest one the surviving text supports):

    M <- mu * M + G
    U  = G + mu * M        (Nesterov)   or   U = M   (plain momentum)
    W <- W - eta * NS_T(U)

with NS_T the Newton-Schulz iteration of ``ns.py`` (standard or Gram form)
standing in for polar(U).  No shape-dependent rescaling of eta: the pages
do not give one, so a caller folds any such factor into eta.
"""

from __future__ import annotations

from typing import Iterable

import numpy as np

from .ns import DEFAULT_EPS, TUNED_ABC, ns_gram, ns_standard


def momentum_update(m: np.ndarray, g: np.ndarray, mu: float,
                    nesterov: bool = True):
    """(new momentum, NS input): M' = mu M + G; U = G + mu M' or M'."""
    m_new = mu * np.asarray(m, dtype=np.float64) + np.asarray(g, dtype=np.float64)
    u = np.asarray(g, dtype=np.float64) + mu * m_new if nesterov else m_new
    return m_new, u


def muon_step(w: np.ndarray, g: np.ndarray, m: np.ndarray, lr: float,
              mu: float = 0.95, nesterov: bool = True, steps: int = 5,
              abc=TUNED_ABC, mode: str = "gram",
              restart: Iterable[int] = (4,), eps: float = DEFAULT_EPS):
    """Returns (W', M') for one step; inputs are not modified."""
    m_new, u = momentum_update(m, g, mu, nesterov)
    if mode == "standard":
        o = ns_standard(u, steps, abc, eps)
    elif mode == "gram":
        o = ns_gram(u, steps, abc, restart, eps)
    else:
        raise ValueError("mode must be 'standard' or 'gram'")
    return np.asarray(w, dtype=np.float64) - lr * o, m_new
