"""Every kernel build, run on the GPU and checked against the fp64 oracle.

The cases in coverage_cases.py reach every build that ns_plan_kernels can
report (tests/test_coverage.py checks that on the host).  Each runs in both
forms on seeded Gaussian input and is compared with the oracle member by
member: the relative Frobenius error (1e-2 for 16-bit input, 1e-4 for fp32)
and the largest 64 x 64 block error relative to the result's RMS (2e-2 for
16-bit, 2e-4 for fp32: twice the global bar; on the fp16 emulation of the
iteration on the host the worst block runs 1.2 to 1.5 times the global
error, while a wrong tile gives errors of the order of the entries).  The
batched calls carry a status word, which must stay clear, and sampled
members must equal single calls (other kernel builds, no status word) bit
for bit.  The builds that read extended arguments run too: each case
guarded (equal to the fixed schedule bit for bit at a threshold no
statistic reaches) and as a grouped call (equal to the plain call bit for
bit).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import newton_schulz_matrix_amd as nsa

from coverage_cases import CASES, DTYPES, MODES
from parity_util import block_err, rel_err

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp16": 1e-2, "fp32": 1e-4}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _oracle(m64, mode):
    if mode == "standard":
        return oracle.ns_standard(m64)
    return oracle.ns_gram(m64, restart=(4,))


def _input(batch, rows, cols, dtype, seed):
    if batch == 1:
        return workloads.column_scaled(rows, cols, seed=seed, dtype=dtype)
    return workloads.gaussian((batch, rows, cols), seed=seed, dtype=dtype)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_every_build_matches_oracle(case, mode):
    dev = _dev()
    batch, rows, cols, dtype, tile = case
    print(f"case {case} {mode}", flush=True)
    m = _input(batch, rows, cols, dtype, seed=rows + cols + batch)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    x = m.to(dev)
    if batch == 1:
        nsa.orthogonalize(x, mode=mode, tile=tile, status=st)
    else:
        nsa.orthogonalize_batched(x, mode=mode, tile=tile, status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    if batch == 1:
        members = [(None, x, m)]
    else:
        idx = (1,) if rows * cols > 4_000_000 else (0, batch // 2, batch - 1)
        members = [(i, x[i], m[i]) for i in idx]
    for i, got, src in members:
        ref = _oracle(src.double().numpy(), mode)
        out = got.double().cpu().numpy()
        err, blk = rel_err(out, ref), block_err(out, ref)
        print(f"  member {i}: rel err {err:.3e}, worst block {blk:.3e}", flush=True)
        assert err < TOL[dtype]
        assert blk < 2 * TOL[dtype]
        if i is not None:
            single = src.to(dev)
            nsa.orthogonalize(single, mode=mode, tile=tile)
            torch.cuda.synchronize()
            assert torch.equal(single, got), i


def _plain(m, dev, mode, tile):
    x = m.to(dev)
    fn = nsa.orthogonalize if m.dim() == 2 else nsa.orthogonalize_batched
    fn(x, mode=mode, tile=tile)
    return x


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_every_guarded_build_equals_fixed_schedule(case):
    # The guard's builds (extended arguments: device flags) at a threshold
    # no statistic reaches: the fixed schedule (restart before step 4) bit
    # for bit, with a clear status word.  The fixed schedule itself is
    # checked against the oracle above.
    dev = _dev()
    batch, rows, cols, dtype, tile = case
    print(f"guarded {case}", flush=True)
    m = _input(batch, rows, cols, dtype, seed=rows + cols + batch)
    fixed = _plain(m, dev, "gram", tile)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    x = m.to(dev)
    fn = nsa.orthogonalize if batch == 1 else nsa.orthogonalize_batched
    fn(x, mode="gram", tile=tile, guard=1e30, status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    assert torch.equal(x, fixed)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_every_grouped_build_equals_plain_call(case, mode):
    # The same matrices as a grouped call (each in its own allocation; the
    # final product reads the member table): equal to the batched or single
    # call bit for bit, with a clear status word.
    dev = _dev()
    batch, rows, cols, dtype, tile = case
    print(f"grouped {case} {mode}", flush=True)
    m = _input(batch, rows, cols, dtype, seed=rows + cols + batch)
    plain = _plain(m, dev, mode, tile)
    members = [m.to(dev)] if batch == 1 else [m[i].to(dev) for i in range(batch)]
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    nsa.orthogonalize_grouped(members, mode=mode, tile=tile, status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    if batch == 1:
        assert torch.equal(members[0], plain)
    else:
        for i in range(batch):
            assert torch.equal(members[i], plain[i]), i
