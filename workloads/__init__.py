"""Seeded synthetic inputs for Newton-Schulz orthogonalization.

This module only draws random matrices and rounds them to the storage dtype.
It holds none of the orthogonalization arithmetic, so that both the fp64
oracle and the HIP path can consume exactly the same values.

Every generator is deterministic in its seed.  Values are drawn on the host
with ``numpy.random.default_rng`` and rounded to the requested dtype with
round-to-nearest-even (torch's CPU cast).  The returned tensors live on the
CPU; callers move them to the device themselves.

Shapes follow the workloads the pages talk about:

* transformer weights of a 124M-parameter GPT-2 (d_model 768, MLP 3072)
  from the Muon / NanoGPT speed-run article;
* Llama-8B projections (4096 x 4096, 4096 x 14336 and its transpose);
* MoE expert matrices (Kimi K2 style experts, here 2048 x 1408);
* heavy-tailed (Student-t) gradients for the ROOT soft-threshold split.

None of these stands in for a dataset: the pages' workloads enter only
through their matrix shapes and value distributions.
"""

from __future__ import annotations

import math
from typing import Dict, List, Tuple

import numpy as np
import torch

_TORCH_DTYPES = {
    "bf16": torch.bfloat16,
    "fp16": torch.float16,
    "fp32": torch.float32,
    "fp64": torch.float64,
}


def torch_dtype(name: str) -> torch.dtype:
    """Map a short dtype name ("bf16", "fp16", "fp32") to a torch dtype."""
    return _TORCH_DTYPES[name]


def round_to(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Round a host array to ``dtype`` with round-to-nearest-even.

    The draw is first held in fp32 or fp64; torch's CPU cast rounds to
    nearest-even, which is the rounding the device kernels use too.
    """
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(_TORCH_DTYPES[dtype]).contiguous()


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def gaussian(shape: Tuple[int, ...], seed: int, dtype: str = "bf16",
             scale: float = 1.0) -> torch.Tensor:
    """i.i.d. N(0, scale^2) entries (fp32 draws), rounded to ``dtype``."""
    rng = _rng(seed, *shape)
    x = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return round_to(x, dtype)


def gaussian_lowrank(r: int, c: int, seed: int, dtype: str = "bf16",
                     scale: float = 0.02, rank: int = 8,
                     weight: float = 0.5) -> torch.Tensor:
    """``scale*G + weight*scale*P Q^T / sqrt(rank)``: a momentum-like matrix.

    G is r x c, P is r x rank and Q is c x rank, all i.i.d. N(0, 1).  The
    low-rank term has the same per-entry scale as the noise, times ``weight``.
    """
    rng = _rng(seed, r, c, rank)
    g = rng.standard_normal((r, c))
    p = rng.standard_normal((r, rank))
    q = rng.standard_normal((c, rank))
    x = scale * g + (weight * scale / math.sqrt(rank)) * (p @ q.T)
    return round_to(x, dtype)


def column_scaled(r: int, c: int, seed: int, dtype: str = "bf16",
                  lo: float = 1e-3, hi: float = 1.0) -> torch.Tensor:
    """N(0,1) entries times a per-column scale drawn log-uniform in [lo, hi].

    The column scales make the spectrum ill-conditioned, the way real
    update matrices are.  Columns are those of the stored (r x c) matrix.
    """
    rng = _rng(seed, r, c)
    g = rng.standard_normal((r, c), dtype=np.float32)
    s = np.exp(rng.uniform(math.log(lo), math.log(hi), size=c)).astype(np.float32)
    g *= s[None, :]
    return round_to(g, dtype)


def student_t(shape: Tuple[int, ...], seed: int, nu: float = 2.0,
              dtype: str = "bf16") -> torch.Tensor:
    """i.i.d. Student-t(nu) entries: heavy-tailed gradient stand-ins."""
    rng = _rng(seed, *shape)
    x = rng.standard_t(nu, size=shape).astype(np.float32)
    return round_to(x, dtype)


def designed_spectrum(r: int, c: int, s: np.ndarray, seed: int):
    """``M = U diag(s) V^T`` with U, V orthonormal from QR of Gaussians.

    Returns (M, U, V) in fp64.  ``len(s) == min(r, c)``.  Used for closed-form
    checks: the singular vectors are known, so the exact output of any odd
    polynomial iteration is known too.
    """
    k = min(r, c)
    rng = _rng(seed, r, c, 7)
    u, _ = np.linalg.qr(rng.standard_normal((r, k)))
    v, _ = np.linalg.qr(rng.standard_normal((c, k)))
    m = (u * np.asarray(s, dtype=np.float64)[None, :]) @ v.T
    return m, u, v


# ---------------------------------------------------------------------------
# The five named workloads.
# ---------------------------------------------------------------------------

def small_fp32(seed: int = 1) -> torch.Tensor:
    """One 256 x 1024 fp32 matrix with i.i.d. N(0, 1) entries."""
    return gaussian((256, 1024), seed, "fp32")


def nanogpt_set(seed: int = 2, layers: int = 12,
                dtype: str = "bf16") -> Dict[str, List[torch.Tensor]]:
    """The 2-D weights of a 12-layer d_model=768 GPT-2 (124M), bf16.

    Per layer: q, k, v, o (768 x 768), the MLP up projection (768 x 3072) and
    its down projection (3072 x 768).  Returned grouped by stored shape.
    """
    groups: Dict[str, List[torch.Tensor]] = {"768x768": [], "768x3072": [],
                                             "3072x768": []}
    for layer in range(layers):
        for j in range(4):
            groups["768x768"].append(
                gaussian_lowrank(768, 768, seed * 1000 + layer * 10 + j, dtype))
        groups["768x3072"].append(
            gaussian_lowrank(768, 3072, seed * 1000 + layer * 10 + 4, dtype))
        groups["3072x768"].append(
            gaussian_lowrank(3072, 768, seed * 1000 + layer * 10 + 5, dtype))
    return groups


LLAMA8B_SHAPES = ((4096, 4096), (4096, 14336), (14336, 4096))


def llama8b(shape: Tuple[int, int] = (4096, 14336), seed: int = 3,
            dtype: str = "bf16") -> torch.Tensor:
    """A Llama-8B-shaped bf16 matrix with log-uniform column scales."""
    return column_scaled(shape[0], shape[1], seed, dtype)


def moe_experts(experts: int = 128, r: int = 2048, c: int = 1408,
                seed: int = 4, dtype: str = "bf16") -> torch.Tensor:
    """``experts`` contiguous r x c N(0, 1) matrices, shape [E, r, c]."""
    return gaussian((experts, r, c), seed, dtype)


def heavy_tailed(r: int = 2048, c: int = 8192, seed: int = 5,
                 dtype: str = "bf16") -> torch.Tensor:
    """A 2048 x 8192 Student-t(2) gradient stand-in, bf16."""
    return student_t((r, c), seed, 2.0, dtype)
