"""The GPU coverage cases reach every kernel build the library launches.

Host only: ns_plan_kernels (and ns_plan_kernels_grouped) report which builds
a call would launch without touching a device.  A sweep over shapes (ragged
and tile-aligned, tall and wide, 1 to 14336), batch sizes, I/O dtypes, both
forms, every tile edge, restart masks, the guard and grouped calls collects
every reachable build; the cases that tests/test_gpu_coverage.py runs on the
GPU (each plain in both forms, guarded in the Gram form, and grouped in both
forms) must reach all of them.
"""

import itertools
import os

import pytest

from newton_schulz_matrix_amd import _binding as B
import newton_schulz_matrix_amd as nsa

from coverage_cases import CASES, DTYPES, MODES

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libnsortho.so not built")

SIZES = [1, 17, 100, 128, 200, 300, 384, 512, 640, 700, 768, 1000, 1024,
         1300, 1408, 2048, 3072, 4096, 8192, 14336]
BATCHES = [1, 2, 5, 12, 24, 40, 48, 60, 128]


def _plan(batch, rows, cols, dtype, mode, tile, mask=1 << 4, guard=0.0, grouped=False):
    try:
        return nsa.plan_kernels(rows, cols, batch, DTYPES[dtype], mode, 5,
                                mask, None, tile, guard=guard, grouped=grouped)
    except nsa.NSError:
        return []


def reachable():
    seen = set()
    for n, m in itertools.combinations_with_replacement(SIZES, 2):
        for batch, dtype, tile in itertools.product(BATCHES, DTYPES, (0, 128, 192, 256)):
            for rows, cols in ((n, m), (m, n)):
                seen.update(_plan(batch, rows, cols, dtype, "standard", tile))
                for mask in (1 << 4, 0, (1 << 2) | (1 << 4)):
                    seen.update(_plan(batch, rows, cols, dtype, "gram", tile, mask))
                seen.update(_plan(batch, rows, cols, dtype, "gram", tile, guard=100.0))
            # A grouped call's plan does not depend on its members' orientation.
            for mode in MODES:
                seen.update(_plan(batch, n, m, dtype, mode, tile, grouped=True))
    return seen


def case_plans(case):
    """Every plan the GPU coverage tests run for one case."""
    batch, rows, cols, dtype, tile = case
    plans = [_plan(batch, rows, cols, dtype, mode, tile) for mode in MODES]
    plans.append(_plan(batch, rows, cols, dtype, "gram", tile, guard=100.0))
    plans += [_plan(batch, rows, cols, dtype, mode, tile, grouped=True) for mode in MODES]
    return plans


def test_cases_reach_every_build():
    covered = set()
    for case in CASES:
        for ks in case_plans(case):
            assert ks, case
            covered.update(ks)
    every = reachable()
    missing = sorted(every - covered)
    assert not missing, missing
    # Every build has a name of the documented form.
    for k in every:
        assert k.split("<")[0] in ("sumsq", "stage", "xxt", "nn", "upd", "out"), k
    assert len(every) >= 60
