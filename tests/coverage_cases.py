"""Calls that, between them, launch every kernel build the library can reach.

Each case is (batch, rows, cols, dtype, tile) and is run in both forms by
tests/test_gpu_coverage.py.  tests/test_coverage.py checks on the host (with
ns_plan_kernels, no device) that these cases reach every build that a sweep
over shapes, batches, dtypes, forms, tile edges and restart masks reaches.
"""

import torch

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}

CASES = [
    # 512 x 1000 on 128 tiles: 10 upper-triangle and 32 update tiles per
    # matrix.  40 matrices: persistent symmetric products (400 tiles) and,
    # for 16-bit, two-per-CU updates (1280 tiles); fp32 updates persistent.
    (40, 512, 1000, "bf16", 0),
    (40, 512, 1000, "fp16", 0),
    (40, 512, 1000, "fp32", 0),
    # 60 matrices: 600 upper tiles, the two-per-CU persistent grid.
    (60, 512, 1000, "bf16", 0),
    (60, 512, 1000, "fp16", 0),
    # 12 matrices: 120 upper tiles (one work-group each), 384 update tiles
    # (persistent).
    (12, 512, 1000, "bf16", 0),
    (12, 512, 1000, "fp16", 0),
    (12, 512, 1000, "fp32", 0),
    # 192 tiles: 360 upper tiles and 1080 update tiles, both persistent.
    (60, 512, 1000, "bf16", 192),
    (60, 512, 1000, "fp16", 192),
    # Long contractions with at least 512 tiles of 128: the two-per-CU
    # kernels with one work-group per tile (650 upper tiles, 50 and 52
    # k-tiles).
    (2, 3200, 3300, "bf16", 128),
    # The same kernels writing more than 256 MiB per launch take their builds
    # with non-temporal stores: 16 x 3200 x 3300 (328 MB per n x n product),
    # and the MoE batch (128 x 1408 x 1408: 507 MB per n x n product,
    # persistent) for both 16-bit I/O types.
    (16, 3200, 3300, "bf16", 128),
    (128, 2048, 1408, "bf16", 0),
    (128, 1408, 2048, "fp16", 0),
    # One work-group per tile at every edge, both 16-bit I/O types (ragged
    # in both directions; tall, so the result is transposed back).
    (1, 1300, 700, "bf16", 128),
    (1, 1300, 700, "bf16", 192),
    (1, 1300, 700, "bf16", 256),
    (1, 1300, 700, "fp16", 128),
    (1, 1300, 700, "fp16", 192),
    (1, 1300, 700, "fp16", 256),
    (1, 640, 512, "fp32", 0),
    (1, 640, 512, "fp32", 128),
    (1, 1300, 700, "fp32", 64),
    # fp32 single matrices take 64 tiles while the n x n products would not
    # fill the chip with 128 tiles; 1024 x 4224 has 1056 update tiles of 64
    # (persistent), and forced to 128, 264 update tiles of 32 k-tiles
    # (persistent too).
    (1, 1024, 4224, "fp32", 0),
    (1, 1024, 4224, "fp32", 128),
]

MODES = ("standard", "gram")
