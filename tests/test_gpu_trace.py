"""The launch trace (ns_trace) on the GPU: which launches it records, the
algorithmic work it reports for them, and event times that fit inside the
call's own time."""

import pytest
import torch

import bench
import workloads
import newton_schulz_matrix_amd as nsa
from newton_schulz_matrix_amd._binding import KERNEL_KINDS

pytestmark = pytest.mark.gpu


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


# Gram form, 5 steps, restart before step 4: the first X X^T, then b R + c R^2
# (which also gives Q at a fresh start) and the two products of R's update
# for steps 1 and 2 with Q's product in step 2, b R + c R^2 and Q's product in
# step 3, the restart (Q X and a new X X^T), steps 4 and 5 like 1 and 3, and
# the final Q X.
GRAM_SEQUENCE = (["norm", "stage", "gram"] + ["sym"] * 3 + ["sym"] * 4 + ["sym"] * 2
                 + ["update", "gram"] + ["sym"] * 3 + ["sym"] * 2 + ["update"])
STANDARD_SEQUENCE = ["norm", "stage"] + ["gram", "sym", "update"] * 5


@pytest.mark.parametrize("mode,expected", [("gram", GRAM_SEQUENCE), ("standard", STANDARD_SEQUENCE)])
def test_trace_records_every_launch(mode, expected):
    dev = _dev()
    r, c = 512, 2048
    x = workloads.gaussian((r, c), seed=71, dtype="bf16").to(dev)
    nsa.orthogonalize(x.clone(), mode=mode)  # load the kernels' code first
    ev = bench.Events(2 * 64)
    tr = bench.make_trace(ev, 64, 0xFFFFFFFF)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    nsa.orthogonalize(x, mode=mode, trace=tr)
    stop.record()
    torch.cuda.synchronize()
    kinds = [KERNEL_KINDS[tr.kinds[i]] for i in range(tr.count)]
    assert kinds == expected
    times = [ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(tr.count)]
    print(mode, [f"{k}:{t * 1e3:.1f}us" for k, t in zip(kinds, times)])
    assert all(t > 0 for t in times)
    assert sum(times) <= start.elapsed_time(stop)
    n, m = r, c
    for i, k in enumerate(kinds):
        if k == "gram":
            assert tr.flops[i] == n * n * m
        elif k == "sym":
            assert tr.flops[i] == n * n * n
        elif k == "update":
            assert tr.flops[i] == 2 * n * n * m
        else:
            assert tr.flops[i] == 0 and tr.bytes[i] >= n * m * 2
    ev.close()


def test_trace_kind_mask_and_capacity():
    dev = _dev()
    x = workloads.gaussian((256, 1024), seed=72, dtype="bf16").to(dev)
    ev = bench.Events(2 * 64)
    only_sym = bench.make_trace(ev, 64, 1 << KERNEL_KINDS.index("sym"))
    nsa.orthogonalize(x, mode="gram", trace=only_sym)
    torch.cuda.synchronize()
    assert only_sym.count == 14
    assert all(KERNEL_KINDS[only_sym.kinds[i]] == "sym" for i in range(only_sym.count))
    # Launches past capacity run but are not recorded.
    y = workloads.gaussian((256, 1024), seed=72, dtype="bf16").to(dev)
    short = bench.make_trace(ev, 5, 0xFFFFFFFF)
    nsa.orthogonalize(y, mode="gram", trace=short)
    torch.cuda.synchronize()
    assert short.count == 5
    assert torch.equal(x, y)
    ev.close()
