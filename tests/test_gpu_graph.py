"""Calls captured into a HIP graph replay to the eager result, bit for bit.

The library makes no allocation, copy, memset or synchronization on the
caller's stream (buffers are cleared by fill kernels), so a call can be
captured with torch.cuda.graph and replayed.  Each test captures one call
with static inputs and workspace, then replays it several times with eager
calls of the library and synchronizations between the replays, and compares
every replay with an eager call on the same input: bitwise, with a clear
status word.  Covered: single and batched calls, chained Muon steps, the
soft-threshold split, a grouped call and the allocation-free entry point.
"""

import pytest
import torch

import workloads
import newton_schulz_matrix_amd as nsa

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _capture(fn):
    """Warm fn up on a side stream, then capture it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _ws(nbytes, dev):
    return torch.empty(nbytes + 4096, dtype=torch.uint8, device=dev)


@pytest.mark.parametrize("shape,dtype,mode", [
    ((1024, 4096), "bf16", "gram"),
    ((4096, 1024), "bf16", "standard"),
    ((256, 1024), "fp32", "gram"),
    ((40, 512, 1000), "bf16", "gram"),
    ((40, 512, 1000), "fp16", "standard"),
])
def test_orthogonalize_replays_equal_eager(shape, dtype, mode):
    dev = _dev()
    print(f"graph {shape} {dtype} {mode}", flush=True)
    batched = len(shape) == 3
    x0 = (workloads.gaussian(shape, seed=31, dtype=dtype) if batched
          else workloads.column_scaled(shape[0], shape[1], seed=31, dtype=dtype)).to(dev)
    tdt = x0.dtype
    rows, cols = shape[-2], shape[-1]
    batch = shape[0] if batched else 1
    call = nsa.orthogonalize_batched if batched else nsa.orthogonalize
    need = nsa.workspace_size(rows, cols, batch, tdt, mode)
    # Eager reference, with its own workspace.
    ref = x0.clone()
    call(ref, mode=mode, workspace=_ws(need, dev))
    # Captured call on static buffers.
    xs = x0.clone()
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = _ws(need, dev)
    g = _capture(lambda: call(xs, mode=mode, workspace=ws, status=st))
    other = x0.clone()
    ws_other = _ws(need, dev)
    for i in range(REPLAYS):
        xs.copy_(x0)
        st.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == 0, i
        assert torch.equal(xs, ref), i
        # Eager library work between the replays.
        other.copy_(x0)
        call(other, mode=mode, workspace=ws_other)
        torch.cuda.synchronize()
        assert torch.equal(other, ref), i


def test_muon_step_replays_equal_eager():
    dev = _dev()
    rows, cols = 768, 3072
    w0 = workloads.gaussian((rows, cols), seed=32, dtype="bf16").to(dev)
    grads = [workloads.gaussian((rows, cols), seed=40 + i, dtype="bf16").to(dev) for i in range(REPLAYS)]
    need = nsa.muon_workspace_size(rows, cols, 1, torch.bfloat16, "gram")
    # Eager: REPLAYS steps from the same state.
    w_ref, m_ref = w0.clone(), torch.zeros(rows, cols, dtype=torch.float32, device=dev)
    ws_ref = _ws(need, dev)
    eager = []
    for gr in grads:
        nsa.muon_step(w_ref, gr, m_ref, lr=0.02, workspace=ws_ref)
        torch.cuda.synchronize()
        eager.append((w_ref.clone(), m_ref.clone()))
    # Captured step on static buffers; warm-up and capture run on scratch
    # state, then the state is reset.
    w, m = w0.clone(), torch.zeros(rows, cols, dtype=torch.float32, device=dev)
    g_in = grads[0].clone()
    ws = _ws(need, dev)
    g = _capture(lambda: nsa.muon_step(w, g_in, m, lr=0.02, workspace=ws))
    w.copy_(w0)
    m.zero_()
    for i, gr in enumerate(grads):
        g_in.copy_(gr)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(w, eager[i][0]), i
        assert torch.equal(m, eager[i][1]), i


def test_soft_threshold_split_replays_equal_eager():
    dev = _dev()
    m0 = workloads.heavy_tailed(1024, 4096, seed=33).to(dev)
    b_ref, o_ref = nsa.soft_threshold_split(m0.clone())
    torch.cuda.synchronize()
    ms = m0.clone()
    out_b = torch.empty_like(ms)
    lam = torch.zeros(1, dtype=torch.float32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    result = {}

    def step():
        result["b"], result["o"] = nsa.soft_threshold_split(ms, out_b=out_b, lambda_out=lam, status=st)

    g = _capture(step)
    for i in range(REPLAYS):
        ms.copy_(m0)
        st.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == 0, i
        assert torch.equal(out_b, b_ref), i
        assert torch.equal(result["o"], o_ref), i
        b2, _ = nsa.soft_threshold_split(m0.clone())
        torch.cuda.synchronize()
        assert torch.equal(b2, b_ref), i


def test_grouped_call_replays_equal_eager():
    # The member table goes to the device as a kernel argument, so a
    # captured grouped call replays with the members it was captured with.
    dev = _dev()
    mats = [workloads.gaussian((96, 320), seed=60 + i, dtype="bf16") for i in range(5)]
    host = [m.t().contiguous() if i % 2 else m for i, m in enumerate(mats)]
    ref = [h.to(dev) for h in host]
    nsa.orthogonalize_grouped(ref, mode="gram")
    torch.cuda.synchronize()
    xs = [h.to(dev) for h in host]
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    need = nsa.grouped_workspace_size(96, 320, len(xs), torch.bfloat16, "gram")
    ws = _ws(need, dev)
    g = _capture(lambda: nsa.orthogonalize_grouped(xs, mode="gram", workspace=ws, status=st))
    for i in range(REPLAYS):
        for x, h in zip(xs, host):
            x.copy_(h.to(dev))
        st.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert int(st.item()) == 0, i
        for j, (x, r) in enumerate(zip(xs, ref)):
            assert torch.equal(x, r), (i, j)
        other = [h.to(dev) for h in host]
        nsa.orthogonalize_grouped(other, mode="gram")
        torch.cuda.synchronize()
        assert all(torch.equal(o, r) for o, r in zip(other, ref)), i


def test_static_call_replays_equal_eager():
    # The allocation-free entry point works in the library's own device
    # scratch; eager calls between the replays use the same scratch.
    dev = _dev()
    x0 = workloads.column_scaled(512, 1536, seed=61, dtype="bf16").to(dev)
    ref = x0.clone()
    nsa.orthogonalize_static(ref, mode="gram")
    torch.cuda.synchronize()
    xs = x0.clone()
    g = _capture(lambda: nsa.orthogonalize_static(xs, mode="gram"))
    for i in range(REPLAYS):
        xs.copy_(x0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xs, ref), i
        other = x0.clone()
        nsa.orthogonalize_static(other, mode="gram")
        torch.cuda.synchronize()
        assert torch.equal(other, ref), i
