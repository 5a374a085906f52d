"""Parity at the full workload sizes, in the configuration bench.py times.

Llama-8B shapes are compared whole against the fp64 oracle.  Batches (MoE
experts, the NanoGPT weight set) are launched whole; sampled members are
compared against the oracle one by one and against single-matrix calls.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import newton_schulz_matrix_amd as nsa
from parity_util import block_err

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _rel(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def _oracle(m64, mode):
    if mode == "standard":
        return oracle.ns_standard(m64)
    return oracle.ns_gram(m64, restart=(4,))


@pytest.mark.parametrize("shape,mode", [((4096, 14336), "gram"),
                                        ((4096, 14336), "standard"),
                                        ((14336, 4096), "gram"),
                                        ((4096, 4096), "standard")])
def test_llama8b_full_size(shape, mode):
    dev = _dev()
    m = workloads.llama8b(shape)
    x = m.to(dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    nsa.orthogonalize(x, mode=mode, status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    out = x.double().cpu().numpy()
    del x
    ref = _oracle(m.double().numpy(), mode)
    err, blk = _rel(out, ref), block_err(out, ref)
    print(f"llama8b {shape} {mode}: rel err {err:.3e}, worst 64x64 block {blk:.3e}")
    assert err < 1e-2
    assert blk < 2e-2
    # The pages' monitoring rule: singular values of the result sit near 1
    # (the tuned triple's band), here on the top of the spectrum.
    sv = np.linalg.svd(out[:512] if shape[0] <= shape[1] else out[:, :512],
                       compute_uv=False)
    assert sv.max() < 1.3


def test_moe_expert_batch_sampled():
    dev = _dev()
    m = workloads.moe_experts(128, 2048, 1408)
    x = m.to(dev)
    nsa.orthogonalize_batched(x, mode="gram")
    torch.cuda.synchronize()
    for e in (0, 63, 127):
        out = x[e].double().cpu().numpy()
        ref = _oracle(m[e].double().numpy(), "gram")
        err, blk = _rel(out, ref), block_err(out, ref)
        print(f"expert {e}: rel err {err:.3e}, worst block {blk:.3e}")
        assert err < 1e-2
        assert blk < 2e-2
        single = m[e].to(dev)
        nsa.orthogonalize(single, mode="gram")
        assert torch.equal(single, x[e])


def test_moe_expert_batch_transposed_sampled():
    dev = _dev()
    m = workloads.moe_experts(128, 1408, 2048)
    x = m.to(dev)
    nsa.orthogonalize_batched(x, mode="gram")
    torch.cuda.synchronize()
    for e in (5, 100):
        out = x[e].double().cpu().numpy()
        ref = _oracle(m[e].double().numpy(), "gram")
        err, blk = _rel(out, ref), block_err(out, ref)
        print(f"expert {e} (1408x2048): rel err {err:.3e}, worst block {blk:.3e}")
        assert err < 1e-2
        assert blk < 2e-2


def test_nanogpt_weight_set():
    dev = _dev()
    groups = workloads.nanogpt_set()
    for shape, mats in groups.items():
        stack = torch.stack(mats)
        for mode in ("standard", "gram"):
            x = stack.to(dev)
            nsa.orthogonalize_batched(x, mode=mode)
            torch.cuda.synchronize()
            for i in (0, len(mats) - 1):
                out = x[i].double().cpu().numpy()
                ref = _oracle(mats[i].double().numpy(), mode)
                err, blk = _rel(out, ref), block_err(out, ref)
                print(f"nanogpt {shape} #{i} {mode}: rel err {err:.3e}, worst block {blk:.3e}")
                assert err < 1e-2
                assert blk < 2e-2


def test_nanogpt_groups_on_concurrent_streams():
    # The three weight groups as the bench runs them: one batched call per
    # group, each on its own stream with its own workspace, launched back to
    # back so their kernels overlap.  The library keeps no state between
    # calls, so the results equal one-at-a-time calls bit for bit.
    dev = _dev()
    groups = [torch.stack(m) for m in workloads.nanogpt_set().values()]
    serial = [g.to(dev) for g in groups]
    for x in serial:
        nsa.orthogonalize_batched(x, mode="gram")
    torch.cuda.synchronize()
    conc = [g.to(dev) for g in groups]
    streams = [torch.cuda.Stream() for _ in conc]
    main = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(main)
    for x, s in zip(conc, streams):
        with torch.cuda.stream(s):
            nsa.orthogonalize_batched(x, mode="gram")
    for s in streams:
        main.wait_stream(s)
    torch.cuda.synchronize()
    for a, b in zip(serial, conc):
        assert torch.equal(a, b)


def test_root_split_then_orthogonalize():
    dev = _dev()
    m = workloads.heavy_tailed()
    m64 = m.double().numpy()
    b_ref, _, lam = oracle.soft_threshold_split(m64)
    # B is stored in the input dtype (round to nearest even).
    b_ref16 = workloads.round_to(b_ref, "bf16").double().numpy()
    lam_out = torch.zeros(1, dtype=torch.float32, device=dev)
    b, o = nsa.soft_threshold_split(m.to(dev), lambda_out=lam_out)
    torch.cuda.synchronize()
    assert lam_out.item() == pytest.approx(lam, rel=1e-7)
    assert np.array_equal(b.double().cpu().numpy(), b_ref16)
    exact = oracle.polar_eigh(b_ref16)
    for mode in ("gram", "standard"):
        x = b.clone()
        nsa.orthogonalize(x, mode=mode)
        torch.cuda.synchronize()
        out = x.double().cpu().numpy()
        ref = _oracle(b_ref16, mode)
        err = _rel(out, ref)
        mse_gpu = oracle.orthogonalization_mse(out, b_ref16, exact)
        mse_ref = oracle.orthogonalization_mse(ref, b_ref16, exact)
        print(f"root split + {mode}: rel err {err:.3e}, MSE vs polar "
              f"{mse_gpu:.4f} (oracle {mse_ref:.4f})")
        assert err < 1e-2
        assert abs(mse_gpu - mse_ref) < 0.1 * mse_ref


@pytest.mark.parametrize("tall", [False, True])
def test_matrix_above_2gib_block_embedding(tall):
    # A 16384 x 65536 bf16 matrix (2 GiB; its internal X buffers are 2 GiB
    # too) that is zero except a ragged 200 x 300 Gaussian block A at the far
    # corner.  M = P A Q^T with P, Q column selections, so the result is A's
    # orthogonalization at the same place and exact zeros elsewhere: the
    # whole path runs with offsets past 2^31 bytes, checked against the
    # oracle on A.
    dev = _dev()
    rows, cols = (65536, 16384) if tall else (16384, 65536)
    br, bc = 200, 300
    r0, c0 = rows - br - 7, cols - bc - 5
    a = workloads.gaussian((br, bc), seed=91, dtype="bf16")
    x = torch.zeros(rows, cols, dtype=torch.bfloat16, device=dev)
    x[r0:r0 + br, c0:c0 + bc] = a.to(dev)
    nsa.orthogonalize(x, mode="gram")
    torch.cuda.synchronize()
    block = x[r0:r0 + br, c0:c0 + bc].double().cpu().numpy()
    err = _rel(block, _oracle(a.double().numpy(), "gram"))
    print(f"{rows}x{cols} block at ({r0}, {c0}): rel err {err:.3e}")
    assert err < 1e-2
    x[r0:r0 + br, c0:c0 + bc] = 0
    assert torch.count_nonzero(x).item() == 0


@pytest.mark.parametrize("mode", ["gram", "standard"])
def test_largest_batch(mode):
    # 65535 members, the largest batch a call takes (one grid dimension of
    # the per-matrix kernels): 17 x 40 bf16 Gaussian matrices, one 128 tile
    # each, so every product launch has 65535 tiles (two work-groups per
    # CU, persistent, non-temporal stores).  Sampled members, first and last
    # included, equal single calls bit for bit and the oracle within the bar.
    dev = _dev()
    batch = 65535
    m = workloads.gaussian((batch, 17, 40), seed=95, dtype="bf16")
    print(f"largest batch: {batch} x 17 x 40 {mode}", flush=True)
    x = m.to(dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    nsa.orthogonalize_batched(x, mode=mode, status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    for i in (0, 1, 4096, 32767, batch - 2, batch - 1):
        single = m[i].to(dev)
        nsa.orthogonalize(single, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(single, x[i]), i
        err = _rel(x[i].double().cpu().numpy(), _oracle(m[i].double().numpy(), mode))
        assert err < 1e-2, (i, err)
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_split_past_2_31_elements_closed_form(dtype):
    # 2^31 + 13 elements (4 or 8 GiB) of a periodic pattern whose lower
    # median of |M| follows from counting one period: v_i = (i mod 7) - 3,
    # times 101 where i mod 1000 == 0 (the outliers).  lambda = 3 x median
    # (in fp32), B = clip(M, -lambda, lambda) and O = M - B then follow
    # elementwise.  Runs the select (one pass over 16-bit keys, three radix
    # passes for fp32) and the split with indices past 2^31.
    dev = _dev()
    numel = (1 << 31) + 13
    period = 7000
    print(f"split of {numel} elements, {dtype}", flush=True)

    def value(i):
        v = (i % 7) - 3
        return v * 101 if i % 1000 == 0 else v

    counts = {}
    full, rest = divmod(numel, period)
    for i in range(period):
        a = abs(value(i))
        counts[a] = counts.get(a, 0) + full + (1 if i < rest else 0)
    assert sum(counts.values()) == numel
    want, acc = (numel + 1) // 2, 0
    for a in sorted(counts):
        acc += counts[a]
        if acc >= want:
            median = a
            break
    lam = float(torch.tensor(3.0 * median, dtype=torch.float32))
    chunk = 1 << 28
    m = torch.empty(numel, dtype=dtype, device=dev)
    for s in range(0, numel, chunk):
        idx = torch.arange(s, min(s + chunk, numel), device=dev, dtype=torch.int64)
        m[s:s + idx.numel()] = ((idx % 7 - 3) * torch.where(idx % 1000 == 0, 101, 1)).to(dtype)
    del idx
    lam_out = torch.zeros(1, dtype=torch.float32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    b, o = nsa.soft_threshold_split(m, lambda_out=lam_out, status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    assert lam_out.item() == lam
    nonzero_o = 0
    for s in range(0, numel, chunk):
        ms, bs, os_ = m[s:s + chunk], b[s:s + chunk], o[s:s + chunk]
        assert torch.equal(bs, ms.clamp(-lam, lam)), s
        assert torch.equal(os_, (ms.float() - bs.float()).to(dtype)), s
        nonzero_o += int(torch.count_nonzero(os_).item())
    assert nonzero_o == sum(c for a, c in counts.items() if a > lam)
    del m, b, o
    torch.cuda.empty_cache()
