"""Per-shape coefficients (ROOT's adaptive iteration) on the GPU.

The fitted per-step schedules go through the same kernels as the tuned
triple (per-step coefficient arrays).  Each case checks parity with the fp64
oracle run with the same schedule on the same rounded input, and the
orthogonalization MSE against the exact polar factor (ROOT page reading:
squared Frobenius error per singular value) against the tuned triple's.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import newton_schulz_matrix_amd as nsa
from newton_schulz_matrix_amd import coeffs

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _rel(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def _oracle(m64, mode, abc):
    if mode == "standard":
        return oracle.ns_standard(m64, 5, abc)
    return oracle.ns_gram(m64, 5, abc, restart=(4,))


@pytest.mark.parametrize("mode", ["gram", "standard"])
def test_page_example_2048x8192(mode):
    """[ROOT]'s example shape: the fitted schedule lowers the MSE by two orders of magnitude."""
    dev = _dev()
    m = workloads.gaussian((2048, 8192), seed=61, dtype="bf16")
    m64 = m.double().numpy()
    exact = oracle.polar_eigh(m64)
    cf = coeffs.root_coefficients(2048, 8192)
    mse = {}
    for name, abc in (("root", cf), ("tuned", nsa.TUNED_ABC)):
        x = m.to(dev)
        nsa.orthogonalize(x, abc=abc, mode=mode)
        torch.cuda.synchronize()
        out = x.double().cpu().numpy()
        ref = _oracle(m64, mode, abc)
        err = _rel(out, ref)
        mse[name] = oracle.orthogonalization_mse(out, m64, exact)
        mse_ref = oracle.orthogonalization_mse(ref, m64, exact)
        print(f"2048x8192 {mode} {name}: rel err {err:.3e}; MSE {mse[name]:.3e} (oracle {mse_ref:.3e})")
        assert err < 1e-2
    assert mse["root"] < 3.3e-4  # the page's adaptive figure
    assert mse["root"] < mse["tuned"] / 50


def test_moe_batch_with_shape_coefficients():
    """128 experts of 2048 x 1408 in one batched call with the 1408 x 2048 schedule."""
    dev = _dev()
    experts = workloads.moe_experts()
    cf = coeffs.root_coefficients(2048, 1408)
    x = experts.to(dev)
    nsa.orthogonalize_batched(x, abc=cf, mode="gram")
    torch.cuda.synchronize()
    out = x.cpu()
    for i in (0, 77, 127):
        m64 = experts[i].double().numpy()
        exact = oracle.polar_eigh(m64)
        got = out[i].double().numpy()
        ref = _oracle(m64, "gram", cf)
        err = _rel(got, ref)
        mse = oracle.orthogonalization_mse(got, m64, exact)
        mse_tuned = oracle.orthogonalization_mse(_oracle(m64, "gram", nsa.TUNED_ABC), m64, exact)
        print(f"moe expert {i}: rel err {err:.3e}; MSE {mse:.3e} (tuned triple, oracle: {mse_tuned:.3e})")
        assert err < 1e-2
        assert mse < mse_tuned / 50


def test_llama_mlp_shape_coefficients():
    """Gaussian 4096 x 14336 with its fitted schedule: the fp16 state, not the polynomial, then limits the MSE.

    (The schedule is fitted to a Gaussian matrix's spectrum; the column-scaled
    Llama workload has a much wider one and keeps the tuned triple.)
    """
    dev = _dev()
    m = workloads.gaussian((4096, 14336), seed=62, dtype="bf16")
    m64 = m.double().numpy()
    exact = oracle.polar_eigh(m64)
    cf = coeffs.root_coefficients(4096, 14336)
    x = m.to(dev)
    nsa.orthogonalize(x, abc=cf, mode="gram")
    torch.cuda.synchronize()
    out = x.double().cpu().numpy()
    mse = oracle.orthogonalization_mse(out, m64, exact)
    y = m.to(dev)
    nsa.orthogonalize(y, mode="gram")
    torch.cuda.synchronize()
    mse_tuned = oracle.orthogonalization_mse(y.double().cpu().numpy(), m64, exact)
    print(f"4096x14336 gram: MSE {mse:.3e} with the fitted schedule, {mse_tuned:.3e} with the tuned triple")
    assert mse < mse_tuned / 10
