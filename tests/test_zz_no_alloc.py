"""ns_orthogonalize_static: the allocation-free variant of
ns_orthogonalize_batched, called through the C ABI.

Its buffers live in the library's own device array, so it must give exactly
what the workspace entry point gives on the same input (the same kernels),
also on a second call that finds the first call's data in the array.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads
import newton_schulz_matrix_amd as nsa
from newton_schulz_matrix_amd import _binding as B
from parity_util import rel_err

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _static_call(x, mode, opt=None):
    batch, rows, cols = x.shape
    a, b, c = B._coefficients(B.TUNED_ABC, 5)
    return B.lib().ns_orthogonalize_static(
        ctypes.c_void_p(x.data_ptr()), batch, rows, cols, x.stride(1),
        x.stride(0), B.dtype_code(x.dtype), 5, a, b, c, B._MODE_CODE[mode],
        ctypes.byref(opt) if opt is not None else None,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_static_scratch_limit_is_checked_on_the_host():
    # A call whose workspace would exceed the array is refused before
    # anything is enqueued (the pointer is never dereferenced).
    limit = B.lib().ns_static_scratch_bytes()
    assert limit == 64 << 20
    a, b, c = B._coefficients(B.TUNED_ABC, 5)
    assert nsa.workspace_size(2048, 8192, 1, torch.bfloat16, "gram") > limit
    st = B.lib().ns_orthogonalize_static(
        ctypes.c_void_p(256), 1, 2048, 8192, 8192, 2048 * 8192, B.NS_BF16, 5,
        a, b, c, B.NS_GRAM, None, None)
    assert st == 3  # NS_ERR_WORKSPACE


def test_static_matches_workspace_entry_point_on_two_calls():
    dev = _dev()
    # The larger call first, then a smaller one with another dtype and form
    # (the array then holds the first call's data).
    cases = [(2, 1024, 2048, "bf16", "gram"), (3, 300, 700, "fp16", "standard")]
    for batch, rows, cols, dtype, mode in cases:
        tdt = workloads.torch_dtype(dtype)
        assert nsa.workspace_size(rows, cols, batch, tdt, mode) <= B.lib().ns_static_scratch_bytes()
        m = workloads.gaussian((batch, rows, cols), seed=rows + batch, dtype=dtype)
        ref = m.to(dev)
        nsa.orthogonalize_batched(ref, mode=mode)
        x = m.to(dev)
        st = torch.zeros(1, dtype=torch.int32, device=dev)
        opt = B.make_options(status=st)
        assert _static_call(x, mode, opt) == 0
        torch.cuda.synchronize()
        print(f"{batch}x{rows}x{cols} {dtype} {mode}: status {st.item()}", flush=True)
        assert st.item() == 0
        assert torch.equal(x, ref)
        err = rel_err(x[0].double().cpu().numpy(),
                      oracle.ns_standard(m[0].double().numpy()) if mode == "standard"
                      else oracle.ns_gram(m[0].double().numpy()))
        assert err < 1e-2
    # The Python face of the same entry point.
    m = workloads.gaussian((200, 300), seed=5, dtype="bf16")
    x, ref = m.to(dev), m.to(dev)
    nsa.orthogonalize(ref, mode="gram")
    B.orthogonalize_static(x, mode="gram")
    torch.cuda.synchronize()
    assert torch.equal(x, ref)
