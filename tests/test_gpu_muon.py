"""Parity of the device Muon step with the fp64 oracle.

One step is M <- mu M + G, U = G + mu M (Nesterov) or M, W <- W - lr NS(U).
The oracle runs it in fp64 on the same stored inputs.  Bars: the new W (or
the applied change W' - W) within 1e-2 relative Frobenius error for 16-bit
storage and 1e-4 for fp32; the fp32 momentum within 1e-6 (fp32 rounding of
a two-term sum).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
import newton_schulz_matrix_amd as nsa

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _rel(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


def _restarts(mask):
    return tuple(k for k in range(1, 33) if (mask >> k) & 1)


def _inputs(shape, dtype, seed, w_scale):
    w = workloads.gaussian(shape, seed, dtype, scale=w_scale)
    g = workloads.gaussian(shape, seed + 1, dtype)
    m = workloads.gaussian(shape, seed + 2, "fp32", scale=0.5)
    return w, g, m


@pytest.mark.parametrize("shape", [(256, 640), (640, 256), (300, 300)])
@pytest.mark.parametrize("mode", ["gram", "standard"])
@pytest.mark.parametrize("nesterov", [True, False])
def test_muon_step_bf16_matches_oracle(shape, mode, nesterov):
    dev = _dev()
    # W = 0: the new W is -lr NS(U), so the comparison is not dominated by
    # the bf16 rounding of a large W.
    w, g, m = _inputs(shape, "bf16", 50, 0.0)
    lr, mu = 0.02, 0.95
    w_ref, m_ref = oracle.muon_step(w.double().numpy(), g.double().numpy(),
                                    m.double().numpy(), lr, mu, nesterov,
                                    mode=mode, restart=(4,))
    wd, gd, md = w.to(dev), g.to(dev), m.to(dev)
    nsa.muon_step(wd, gd, md, lr, mu, nesterov, mode=mode)
    torch.cuda.synchronize()
    err_w = _rel(wd.double().cpu().numpy(), w_ref)
    err_m = _rel(md.double().cpu().numpy(), m_ref)
    print(f"{shape} {mode} nesterov={nesterov}: W {err_w:.3e}, M {err_m:.3e}")
    assert err_w < 1e-2
    assert err_m < 1e-6
    assert torch.equal(gd.cpu(), g)


@pytest.mark.parametrize("mode", ["gram", "standard"])
def test_muon_step_fp32_applied_change(mode):
    dev = _dev()
    w, g, m = _inputs((256, 1024), "fp32", 60, 0.01)
    lr = 0.05
    w_ref, _ = oracle.muon_step(w.double().numpy(), g.double().numpy(),
                                m.double().numpy(), lr, 0.95, True, mode=mode)
    wd = w.to(dev)
    nsa.muon_step(wd, g.to(dev), m.to(dev), lr, 0.95, True, mode=mode)
    torch.cuda.synchronize()
    w0 = w.double().numpy()
    err = _rel(wd.double().cpu().numpy() - w0, w_ref - w0)
    print(f"fp32 {mode}: applied change rel err {err:.3e}")
    assert err < 1e-4


def test_muon_step_zero_lr_leaves_w_and_updates_m():
    dev = _dev()
    w, g, m = _inputs((200, 520), "bf16", 70, 1.0)
    wd, md = w.to(dev), m.to(dev)
    nsa.muon_step(wd, g.to(dev), md, 0.0, 0.9, True)
    torch.cuda.synchronize()
    assert torch.equal(wd.cpu(), w)
    expect = 0.9 * m.double().numpy() + g.double().numpy()
    assert _rel(md.double().cpu().numpy(), expect) < 1e-6


def test_muon_step_batched_equals_single_and_strided():
    dev = _dev()
    e, rows, cols = 4, 192, 448
    w, g, m = _inputs((e, rows, cols), "bf16", 80, 0.5)
    wb, gb, mb = w.to(dev), g.to(dev), m.to(dev)
    nsa.muon_step(wb, gb, mb, 0.03, 0.95, True, mode="gram")
    torch.cuda.synchronize()
    for i in range(e):
        ws, ms = w[i].to(dev), m[i].to(dev)
        nsa.muon_step(ws, g[i].to(dev), ms, 0.03, 0.95, True, mode="gram")
        torch.cuda.synchronize()
        assert torch.equal(ws, wb[i]), i
        assert torch.equal(ms, mb[i]), i
    # Rows with a leading dimension larger than cols (views of wider buffers).
    pad = 24
    big_w = torch.zeros(rows, cols + pad, dtype=torch.bfloat16, device=dev)
    big_g = torch.zeros_like(big_w)
    big_m = torch.zeros(rows, cols + pad, dtype=torch.float32, device=dev)
    big_w[:, :cols] = w[0].to(dev)
    big_g[:, :cols] = g[0].to(dev)
    big_m[:, :cols] = m[0].to(dev)
    vw, vg, vm = big_w[:, :cols], big_g[:, :cols], big_m[:, :cols]
    nsa.muon_step(vw, vg, vm, 0.03, 0.95, True, mode="gram")
    torch.cuda.synchronize()
    assert torch.equal(vw, wb[0]) and torch.equal(vm, mb[0])
    assert torch.count_nonzero(big_w[:, cols:]) == 0


def test_muon_step_llama_mlp_full_size():
    dev = _dev()
    g = workloads.llama8b((4096, 14336))
    w = torch.zeros_like(g)
    m = torch.zeros(g.shape, dtype=torch.float32)
    w_ref, m_ref = oracle.muon_step(w.double().numpy(), g.double().numpy(),
                                    m.double().numpy(), 0.02, 0.95, True,
                                    mode="gram", restart=(4,))
    wd, md = w.to(dev), m.to(dev)
    nsa.muon_step(wd, g.to(dev), md, 0.02, 0.95, True, mode="gram")
    torch.cuda.synchronize()
    err = _rel(wd.double().cpu().numpy(), w_ref)
    print(f"4096x14336 Muon step: W rel err {err:.3e}")
    assert err < 1e-2
    assert _rel(md.double().cpu().numpy(), m_ref) < 1e-6
