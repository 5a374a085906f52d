"""The n x n matrices of the Gram form are stored exactly symmetric.

The symmetric products compute the upper tiles only: an off-diagonal tile is
written twice (itself and its mirror) and a diagonal tile takes every element
from its upper triangle.  The products' outputs stay in the caller's
workspace after a call, so the tests read them back from there: the last
four buffers of the workspace are the n x n matrices (R, Z' and the two Q / V
buffers), each n_pad x n_pad fp16 per matrix of the batch.  Exact symmetry is
a property of the stores, not of the arithmetic, so it is checked bit for bit
(rounding-level asymmetry would pass every parity test).
"""

import pytest
import torch

import workloads
import newton_schulz_matrix_amd as nsa

pytestmark = pytest.mark.gpu

ALIGN = 256


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _align(x):
    return (x + ALIGN - 1) // ALIGN * ALIGN


def _nn_buffers(x, tile, steps=5, restart_mask=1 << 4):
    """Orthogonalize x ([E, r, c] or [r, c], bf16) in Gram form with a forced
    tile edge; return the four n x n buffers as [4, E, n_pad, n_pad] fp16."""
    batched = x.dim() == 3
    e, r, c = (x.shape if batched else (1,) + tuple(x.shape))
    n = min(r, c)
    n_pad = (n + tile - 1) // tile * tile
    need = nsa.workspace_size(r, c, e, x.dtype, "gram", restart_mask=restart_mask, tile=tile)
    ws = torch.full((need + 256,), 0xFF, dtype=torch.uint8, device=x.device)
    base = (-ws.data_ptr()) % 256  # the binding aligns the buffer start to 256 bytes
    if batched:
        nsa.orthogonalize_batched(x, steps=steps, mode="gram", restart_mask=restart_mask, workspace=ws, tile=tile)
    else:
        nsa.orthogonalize(x, steps=steps, mode="gram", restart_mask=restart_mask, workspace=ws, tile=tile)
    torch.cuda.synchronize()
    nn_bytes = _align(e * n_pad * n_pad * 2)
    bufs = []
    for i in range(4):
        off = base + need - (4 - i) * nn_bytes
        raw = ws[off:off + e * n_pad * n_pad * 2]
        bufs.append(raw.view(torch.float16).view(e, n_pad, n_pad))
    return torch.stack(bufs), n, n_pad


@pytest.mark.parametrize("shape,tile", [((500, 1200), 192), ((1300, 512), 128), ((400, 900), 256)])
def test_single_matrix_nn_buffers_exactly_symmetric(shape, tile):
    dev = _dev()
    x = workloads.gaussian(shape, seed=81, dtype="bf16").to(dev)
    bufs, n, n_pad = _nn_buffers(x, tile)
    for i in range(4):
        b = bufs[i, 0]
        assert torch.isfinite(b).all()
        assert torch.equal(b, b.T), f"buffer {i} not symmetric"
        # Rows and columns past n are zero (the next products rely on it).
        assert not b[n:, :].any() and not b[:, n:].any()


@pytest.mark.parametrize("batch", [60, 100])
def test_batched_nn_buffers_exactly_symmetric(batch):
    # 384 x 512 on 128 tiles: 6 triangle tiles per matrix, 6 k-tiles.
    # 60 matrices (360 tiles) take the persistent kernels; 100 (600 tiles)
    # the ones built for two work-groups per compute unit.
    dev = _dev()
    x = workloads.gaussian((batch, 384, 512), seed=82, dtype="bf16").to(dev)
    bufs, n, n_pad = _nn_buffers(x, 128)
    assert torch.isfinite(bufs).all()
    assert torch.equal(bufs, bufs.transpose(-1, -2))


@pytest.mark.parametrize("tile", [128, 192])
def test_fresh_q_is_z_plus_a_on_the_real_diagonal(tile):
    """One Gram step: Z' = b R + c R^2 and, from the same epilogue, Q = a I + Z'
    with its diagonal rounded once from fp32 (real rows only)."""
    dev = _dev()
    r, c = 300, 700
    a = nsa.TUNED_ABC[0]
    x = workloads.gaussian((r, c), seed=83, dtype="bf16").to(dev)
    bufs, n, n_pad = _nn_buffers(x, tile, steps=1, restart_mask=0)
    z, q = bufs[1, 0].float(), bufs[2, 0].float()
    off = ~torch.eye(n_pad, dtype=torch.bool, device=dev)
    assert torch.equal(q[off], z[off])
    dz, dq = torch.diagonal(z), torch.diagonal(q)
    # Real rows: a + Z'_ii, rounded once to fp16 from the fp32 value (so
    # within one fp16 rounding of a + (fp16) Z'_ii); padding rows stay 0.
    ulp = (torch.abs(a + dz[:n]) + torch.abs(dz[:n])) * 2.0 ** -10
    assert (torch.abs(dq[:n] - (a + dz[:n])) <= ulp).all()
    assert not dq[n:].any() and not dz[n:].any()
