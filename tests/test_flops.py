"""The FLOP counter used in throughput reports, against the pages' claims."""

import json
import os

import pytest

from newton_schulz_matrix_amd.flops import gram_flops, ns_flops, standard_flops

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _claims():
    with open(os.path.join(GOLDEN, "cost_claims.json")) as f:
        return json.load(f)


def test_gram_reduction_in_the_pages_range():
    lo, hi = _claims()["flop_reduction"]["range"]
    n = 1024
    m = 4 * n                                    # alpha = 4
    std = standard_flops(n, m)
    one_restart = gram_flops(n, m, restarts=(3,))
    naive = gram_flops(n, m, restarts=())
    r1 = 1 - one_restart / std
    r0 = 1 - naive / std
    # Stabilized (one restart) and naive Gram bracket the printed range.
    assert lo - 0.01 < r1 < r0 < hi
    assert r1 < lo + 0.02 and r0 > hi - 0.04
    # No saving on square matrices for the restarted form.
    assert gram_flops(n, n, restarts=(3,)) >= standard_flops(n, n)


@pytest.mark.parametrize("case", _claims()["muon_overhead"]["cases"])
def test_muon_overhead_bound(case):
    # Training costs about 6 * params * tokens FLOPs; for a square m x m
    # weight the dense NS cost per step is 6 m^3, so the overhead is T m / B.
    m, b, t = case["m"], case["batch_tokens"], case["steps"]
    ratio = standard_flops(m, m, t, symmetric=False) / (6.0 * m * m * b)
    assert ratio == pytest.approx(t * m / b, rel=1e-12)
    if "about" in case:
        assert abs(ratio - case["about"]) < 0.0005
    if "below" in case:
        assert ratio < case["below"]


def test_overhead_bound_holds_for_rectangles():
    for n, m in [(768, 3072), (4096, 14336), (1408, 2048)]:
        dense = standard_flops(n, m, 5, symmetric=False)
        assert dense / (6.0 * n * m) <= 5 * min(n, m)


def test_counter_by_enumeration():
    # Walk the product sequence of the Gram form one call at a time.
    n, m, t = 7, 19, 5
    sym_nn, sym_nm, dense_nm = n ** 3, n * n * m, 2 * n * n * m
    expect = (sym_nm                                   # R = X X^T
              + sym_nn + 0 + 2 * sym_nn                # step 1
              + sym_nn + sym_nn                        # step 2 (restart next)
              + dense_nm + sym_nm                      # restart before 3
              + sym_nn + 0 + 2 * sym_nn                # step 3
              + sym_nn + sym_nn + 2 * sym_nn           # step 4
              + sym_nn + sym_nn                        # step 5
              + dense_nm)                              # output
    assert gram_flops(n, m, t, (3,)) == expect
    assert ns_flops(m, n, t, "gram", 1 << 3) == expect
    assert ns_flops(n, m, t, "standard") == t * (sym_nm + sym_nn + dense_nm)


def test_bench_issued_work_counts_whole_tiles():
    # The bench's supplementary roofline counts the MFMA work a symmetric
    # launch issues: every upper-triangle tile in full, contraction rounded
    # up to the k-tile (64 elements for 16-bit operands, 32 for fp32).
    import sys
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    # 4096 on 192 tiles: 22 blocks (the last 64 wide), 253 tiles.
    assert bench.issued_flops("sym", 1, 4096, 14336, 192, "fp16") == 253 * 192 ** 2 * 4096 * 2
    assert bench.issued_flops("gram", 1, 14336, 4096, 192, "fp16") == 253 * 192 ** 2 * 14336 * 2
    # 2048 on 128 tiles: 136 tiles; the expert batch: 66 tiles per matrix.
    assert bench.issued_flops("sym", 1, 2048, 8192, 128, "fp16") == 136 * 128 ** 2 * 2048 * 2
    assert bench.issued_flops("sym", 128, 2048, 1408, 128, "fp16") == 128 * 66 * 128 ** 2 * 1408 * 2
    # fp32: 256 on 64 tiles, contraction in 32-element k-tiles; ragged n.
    assert bench.issued_flops("sym", 1, 256, 1024, 64, "fp32") == 10 * 64 ** 2 * 256 * 2
    assert bench.issued_flops("sym", 1, 100, 300, 64, "fp32") == 3 * 64 ** 2 * 128 * 2
    # Symmetric products only; the issued count is never below the
    # algorithmic one (n^3 for an n x n product).
    assert bench.issued_flops("update", 1, 4096, 14336, 192, "fp16") is None
    for n in (1, 100, 1000, 4096):
        assert bench.issued_flops("sym", 1, n, 2 * n, 128, "fp16") >= n ** 3
