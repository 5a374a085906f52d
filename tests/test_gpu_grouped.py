"""Grouped calls: matrices of one shape up to orientation, each in its own
storage, with every stage launched once for all of them (the Gram-NS essay
on showapi.com, sections 2.3 and 4.1).  The NanoGPT-124M weight set runs as
two groups: the 48 square attention matrices, and the 12 wide 768 x 3072 with
the 12 tall 3072 x 768 MLP matrices.  Every member must equal the single
call on that matrix bit for bit, and the oracle within the 1e-2 bar.
"""

import pytest
import torch

import oracle
import workloads
import newton_schulz_matrix_amd as nsa
from parity_util import block_err, rel_err

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _oracle(m64, mode):
    return oracle.ns_standard(m64) if mode == "standard" else oracle.ns_gram(m64)


@pytest.mark.parametrize("mode", ["gram", "standard"])
def test_nanogpt_mlp_group_wide_and_tall(mode):
    dev = _dev()
    sets = workloads.nanogpt_set()
    mats = sets["768x3072"] + sets["3072x768"]
    assert len(mats) == 24
    xs = [m.to(dev) for m in mats]
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    nsa.orthogonalize_grouped(xs, mode=mode, status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    for i in range(len(mats)):
        single = mats[i].to(dev)
        nsa.orthogonalize(single, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(single, xs[i]), i
    for i in (0, 11, 12, 23):
        ref = _oracle(mats[i].double().numpy(), mode)
        out = xs[i].double().cpu().numpy()
        err, blk = rel_err(out, ref), block_err(out, ref)
        print(f"member {i} {tuple(mats[i].shape)} {mode}: rel err {err:.3e}, worst block {blk:.3e}")
        assert err < 1e-2 and blk < 2e-2


def test_grouped_square_attention_group():
    dev = _dev()
    mats = workloads.nanogpt_set()["768x768"]
    assert len(mats) == 48
    xs = [m.to(dev) for m in mats]
    nsa.orthogonalize_grouped(xs, mode="gram")
    stacked = torch.stack(mats).to(dev)
    nsa.orthogonalize_batched(stacked, mode="gram")
    torch.cuda.synchronize()
    for i in range(48):
        assert torch.equal(xs[i], stacked[i]), i


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_grouped_strided_members_and_ragged_shape(dtype):
    # Members with padded rows (ld > stored width), wide and tall, ragged
    # against every tile edge; several batch forms (with 40 members the
    # 16-bit products take the persistent and two-per-CU kernels).
    dev = _dev()
    count = 40
    mats, xs = [], []
    for i in range(count):
        tall = i % 3 == 1
        shape = (700, 300) if tall else (300, 700)
        m = workloads.gaussian(shape, seed=80 + i, dtype=dtype)
        mats.append(m)
        pad = 8 * (i % 4)
        buf = torch.zeros(shape[0], shape[1] + pad, dtype=m.dtype, device=dev)
        buf[:, :shape[1]] = m.to(dev)
        xs.append(buf[:, :shape[1]])
    nsa.orthogonalize_grouped(xs, mode="gram")
    torch.cuda.synchronize()
    tol = 1e-4 if dtype == "fp32" else 1e-2
    for i in (0, 1, 2, 17, 39):
        single = mats[i].to(dev)
        nsa.orthogonalize(single, mode="gram")
        torch.cuda.synchronize()
        assert torch.equal(single, xs[i]), i
        err = rel_err(xs[i].double().cpu().numpy(), _oracle(mats[i].double().numpy(), "gram"))
        assert err < tol, (i, err)


def test_grouped_member_table_in_several_chunks():
    # More members than one launch's argument block carries (128): the
    # member table is written by three launches (128 + 128 + 44 entries).
    # Every member, wide or tall, in its own allocation, must equal the
    # batched call on the same matrices bit for bit (the tall ones
    # transposed into the wide orientation first, which is exact).
    dev = _dev()
    count = 300
    wide = [workloads.gaussian((48, 80), seed=900 + i, dtype="bf16") for i in range(count)]
    xs = [(w.t().contiguous() if i % 5 == 2 else w.clone()).to(dev) for i, w in enumerate(wide)]
    print(f"grouped table chunks: {count} members", flush=True)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    nsa.orthogonalize_grouped(xs, mode="gram", status=st)
    stacked = torch.stack(wide).to(dev)
    nsa.orthogonalize_batched(stacked, mode="gram")
    torch.cuda.synchronize()
    assert st.item() == 0
    for i in range(count):
        got = xs[i].t() if i % 5 == 2 else xs[i]
        assert torch.equal(got, stacked[i]), i
    for i in (0, 127, 128, 257, 299):
        ref = _oracle(wide[i].double().numpy(), "gram")
        assert rel_err(stacked[i].double().cpu().numpy(), ref) < 1e-2, i
