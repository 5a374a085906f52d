"""Restarts on demand: the guarded Gram iteration (ns_options.guard_threshold).

The Gram-NS article ("Stability challenges and solutions") reports that the
naive Gram iteration is unstable in half precision and that a restart with
a fresh Gram matrix fixes it.  With the guard, the restart happens where the
state calls for it: after step k forms Q, a restart before step k + 1 is
scheduled on the device when max_i |Q_ii| * |a_{k+1}| exceeds the threshold.
The inputs below were chosen on the host's fp16 emulation of the iteration,
where the statistic passes 100 by 17 % (column scales down to 1e-5, before
step 4) or stays 18 % below it (a well-conditioned designed spectrum).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import newton_schulz_matrix_amd as nsa
from newton_schulz_matrix_amd import _binding as B
from parity_util import rel_err

pytestmark = pytest.mark.gpu

THETA = 100.0


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _ill(dtype):
    return workloads.column_scaled(384, 1000, seed=22, dtype=dtype, lo=1e-5)


def _well(dtype):
    m, _, _ = workloads.designed_spectrum(384, 1000, np.linspace(0.9, 1.0, 384), seed=61)
    return workloads.round_to(m, dtype)


def _run(m, mask, guard=0.0, batched=False):
    dev = _dev()
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    x = m.to(dev)
    fn = nsa.orthogonalize_batched if batched else nsa.orthogonalize
    fn(x, mode="gram", restart_mask=mask, guard=guard, status=st)
    torch.cuda.synchronize()
    return x, st.item()


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_guard_restarts_ill_conditioned_naive_gram(dtype):
    m = _ill(dtype)
    ref = oracle.ns_gram(m.double().numpy(), 5, oracle.TUNED_ABC, ())
    x0, w0 = _run(m, 0)
    x1, w1 = _run(m, 0, THETA)
    e0 = rel_err(x0.double().cpu().numpy(), ref)
    e1 = rel_err(x1.double().cpu().numpy(), ref)
    print(f"{dtype}: naive {e0:.3e}, guarded {e1:.3e}, status {w1:#x}")
    assert w0 == 0
    assert e0 > 1e-2
    assert e1 < 1e-2
    # One restart, before step 4 (where the fixed schedule restarts).
    assert w1 == B.STATUS_GUARD_RESTART | (1 << (15 + 4))
    assert nsa.status_code(w1) == 0
    # It is the fixed schedule's restart, bit for bit.
    x2, _ = _run(m, 1 << 4)
    assert torch.equal(x1, x2)


def test_guard_leaves_well_conditioned_input_naive():
    # No restart: the guarded call equals the naive one bit for bit (the
    # gated restart kernels ran and did nothing).
    m = _well("bf16")
    x0, _ = _run(m, 0)
    x1, w1 = _run(m, 0, THETA)
    assert w1 == 0
    assert torch.equal(x0, x1)
    ref = oracle.ns_gram(m.double().numpy(), 5, oracle.TUNED_ABC, ())
    assert rel_err(x1.double().cpu().numpy(), ref) < 1e-2


@pytest.mark.parametrize("mask", [0, 1 << 4, (1 << 2) | (1 << 4)])
def test_guard_extremes_equal_fixed_schedules(mask):
    # A threshold no statistic reaches gives the fixed schedule; a threshold
    # every statistic passes restarts before every step, which is the fixed
    # schedule with every bit set (both bit for bit: same kernels, buffers
    # chosen on the device).
    m = workloads.gaussian((300, 700), seed=63, dtype="bf16")
    fixed, _ = _run(m, mask)
    never, w = _run(m, mask, 1e30)
    assert w == 0 and torch.equal(fixed, never)
    every_mask = sum(1 << k for k in range(2, 6))
    every, _ = _run(m, every_mask)
    always, w = _run(m, mask, 1e-30)
    assert torch.equal(every, always)
    want = B.STATUS_GUARD_RESTART
    for k in range(2, 6):
        if not (mask >> k) & 1:
            want |= 1 << (15 + k)
    assert w == want


def test_guard_decides_per_matrix_in_a_batch():
    # Ill- and well-conditioned matrices in one batch: each member restarts
    # (or not) on its own and equals its single guarded call.
    mats = [_ill("bf16"), _well("bf16"), _ill("bf16") * 0.5, _well("bf16") * 3]
    batch = torch.stack(mats)
    xb, wb = _run(batch, 0, THETA, batched=True)
    assert wb == B.STATUS_GUARD_RESTART | (1 << (15 + 4))
    for i, m in enumerate(mats):
        xs, ws = _run(m, 0, THETA)
        assert torch.equal(xs, xb[i]), i
        assert (ws != 0) == (i % 2 == 0), (i, ws)


def test_guard_in_batched_persistent_and_pair_kernels():
    # 40 matrices of 512 x 1000 (persistent symmetric products, two-per-CU
    # updates) with a threshold that restarts before every step: equal to the
    # fixed every-step schedule.
    m = workloads.gaussian((40, 512, 1000), seed=64, dtype="bf16")
    every = sum(1 << k for k in range(2, 6))
    a, _ = _run(m, every, batched=True)
    b, w = _run(m, 0, 1e-30, batched=True)
    assert torch.equal(a, b)
    assert w & B.STATUS_GUARD_RESTART


def test_guard_ignored_by_standard_form():
    dev = _dev()
    m = workloads.gaussian((200, 300), seed=65, dtype="bf16")
    x, y = m.to(dev), m.to(dev)
    nsa.orthogonalize(x, mode="standard")
    nsa.orthogonalize(y, mode="standard", guard=1e-30)
    torch.cuda.synchronize()
    assert torch.equal(x, y)
