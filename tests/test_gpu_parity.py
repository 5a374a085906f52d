"""Parity of the HIP path with the fp64 oracle, element by element.

Every case runs the library through its C ABI (via the ctypes binding) on
seeded inputs and compares with the oracle on the same rounded values.  The
bar is the relative Frobenius error ||gpu - oracle||_F / ||oracle||_F:
1e-2 for 16-bit input and 1e-4 for fp32 input (the oracle is fp64; the
device products accumulate in fp32 and store 16-bit or fp32 intermediates).
Integer work (the median select and the clip decisions) is compared exactly.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
import newton_schulz_matrix_amd as nsa

pytestmark = pytest.mark.gpu

TUNED = oracle.TUNED_ABC
TOL = {torch.bfloat16: 1e-2, torch.float16: 1e-2, torch.float32: 1e-4}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def _rel(x, ref):
    d = np.linalg.norm(x - ref)
    n = np.linalg.norm(ref)
    return float(d / n) if n > 0 else float(d)


def _restarts(mask):
    return tuple(k for k in range(1, 33) if (mask >> k) & 1)


def _oracle(m64, mode, steps=5, abc=TUNED, mask=1 << 4, eps=1e-7):
    if mode == "standard":
        return oracle.ns_standard(m64, steps, abc, eps)
    return oracle.ns_gram(m64, steps, abc, _restarts(mask), eps)


def _run(m_cpu, mode, steps=5, abc=TUNED, mask=1 << 4, internal=None,
         ld_pad=0, tile=0):
    dev = _dev()
    rows, cols = m_cpu.shape
    if ld_pad:
        big = torch.zeros(rows, cols + ld_pad, dtype=m_cpu.dtype)
        big[:, :cols] = m_cpu
        x = big.to(dev)[:, :cols]
    else:
        x = m_cpu.to(dev)
    nsa.orthogonalize(x, steps=steps, abc=abc, mode=mode, restart_mask=mask,
                      internal=internal, tile=tile)
    torch.cuda.synchronize()
    return x.double().cpu().numpy()


# ---------------------------------------------------------------------------
# Small and ragged shapes, both forms, every dtype.
# ---------------------------------------------------------------------------

SHAPES = [(256, 1024), (200, 300), (300, 200), (128, 128), (1, 17), (17, 1),
          (130, 700), (640, 512)]


@pytest.mark.parametrize("mode", ["standard", "gram"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16,
                                   torch.float32])
@pytest.mark.parametrize("shape", SHAPES)
def test_parity_small(shape, dtype, mode):
    name = {torch.bfloat16: "bf16", torch.float16: "fp16",
            torch.float32: "fp32"}[dtype]
    m = workloads.gaussian(shape, seed=sum(shape), dtype=name)
    ref = _oracle(m.double().numpy(), mode)
    out = _run(m, mode)
    err = _rel(out, ref)
    print(f"{shape} {name} {mode}: rel err {err:.3e}")
    assert err < TOL[dtype]


def test_parity_config1_fp32_both_forms():
    m = workloads.small_fp32()
    m64 = m.double().numpy()
    for mode in ("standard", "gram"):
        err = _rel(_run(m, mode), _oracle(m64, mode))
        print(f"256x1024 fp32 {mode}: {err:.3e}")
        assert err < 1e-4


def test_parity_gram_restart_schedules():
    # Ill-conditioned input (column scales down to 1e-3).  The Gram-NS article
    # ("Stability challenges and solutions") reports that the naive Gram
    # iteration is unstable in half precision and that restarting fixes it:
    # with fp16 products every restarted schedule meets the 1e-2 bar and the
    # naive one is the worst of the four.
    m = workloads.column_scaled(384, 1000, seed=21, dtype="bf16")
    m64 = m.double().numpy()
    errs = {}
    masks = (0, 1 << 3, 1 << 4, (1 << 2) | (1 << 4))
    for mask in masks:
        ref = _oracle(m64, "gram", mask=mask)
        errs[mask] = _rel(_run(m, "gram", mask=mask), ref)
    print(", ".join(f"mask {k:#x}: {v:.3e}" for k, v in errs.items()))
    restarted = [errs[k] for k in masks[1:]]
    assert errs[0] > max(restarted)
    assert errs[0] < 5e-2
    assert max(restarted) < 1e-2


def test_parity_per_step_coefficients_and_steps():
    m = workloads.gaussian((192, 448), seed=23, dtype="fp32")
    sched = [TUNED, oracle.CLASSIC_ABC, TUNED, (1.5, -0.5, 0.0),
             oracle.CLASSIC_ABC, oracle.CLASSIC_ABC, TUNED]
    m64 = m.double().numpy()
    for mode in ("standard", "gram"):
        err = _rel(_run(m, mode, steps=7, abc=sched, mask=(1 << 3) | (1 << 6)),
                   _oracle(m64, mode, steps=7, abc=sched,
                           mask=(1 << 3) | (1 << 6)))
        assert err < 1e-4, (mode, err)
    for steps in (1, 2, 3):
        err = _rel(_run(m, "gram", steps=steps),
                   _oracle(m64, "gram", steps=steps))
        assert err < 1e-4, (steps, err)


def test_parity_strided_rows():
    m = workloads.gaussian((150, 260), seed=24, dtype="bf16")
    ref = _oracle(m.double().numpy(), "standard")
    assert _rel(_run(m, "standard", ld_pad=37), ref) < 1e-2
    mt = workloads.gaussian((260, 150), seed=25, dtype="bf16")
    ref = _oracle(mt.double().numpy(), "gram")
    assert _rel(_run(mt, "gram", ld_pad=8), ref) < 1e-2


def test_zero_matrix_gives_zero():
    dev = _dev()
    for mode in ("standard", "gram"):
        x = torch.zeros(64, 96, dtype=torch.bfloat16, device=dev)
        nsa.orthogonalize(x, mode=mode)
        assert torch.count_nonzero(x).item() == 0


@pytest.mark.parametrize("mode", ["standard", "gram"])
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_nonfinite_status_word(mode, bad):
    # A clean call leaves the word clear.  A NaN or Inf in the input makes
    # the norm non-finite (NS_STATUS_AT_INPUT); it then spreads through
    # every product, so the n x n epilogues (R, Z', Q, V / A, b A + c A^2)
    # report NS_STATUS_AT_STATE and the final one NS_STATUS_AT_OUTPUT, each
    # with the code NS_ERR_NONFINITE in the low byte.
    from newton_schulz_matrix_amd import _binding as B
    dev = _dev()
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    x = workloads.gaussian((64, 96), seed=26).to(dev)
    nsa.orthogonalize(x, mode=mode, status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    x = workloads.gaussian((64, 96), seed=26).to(dev)
    x[3, 5] = bad
    nsa.orthogonalize(x, mode=mode, status=st)
    torch.cuda.synchronize()
    word = st.item()
    assert nsa.status_code(word) == B.NS_ERR_NONFINITE
    for bit in (B.STATUS_AT_INPUT, B.STATUS_AT_STATE, B.STATUS_AT_OUTPUT):
        assert word & bit, hex(word)
    assert not word & (B.STATUS_AT_SPLIT | B.STATUS_GUARD_RESTART)
    if mode == "standard":
        assert word & B.STATUS_AT_ITERATE
    # Without a status word the same call runs the same kernels unchecked.
    y = workloads.gaussian((64, 96), seed=26).to(dev)
    y[3, 5] = bad
    nsa.orthogonalize(y, mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(torch.isnan(x), torch.isnan(y))


def test_binding_rejects_mismatched_buffers():
    # Checked in Python before any call into the library.
    dev = _dev()
    m = torch.zeros(64, 96, dtype=torch.bfloat16, device=dev)
    for out_b in (torch.zeros(64, 96, dtype=torch.float16, device=dev),
                  torch.zeros(64, 95, dtype=torch.bfloat16, device=dev),
                  torch.zeros(96, 128, dtype=torch.bfloat16, device=dev)[:, :64].t(),
                  torch.zeros(64, 96, dtype=torch.bfloat16)):
        with pytest.raises(ValueError):
            nsa.soft_threshold_split(m, out_b=out_b)
    with pytest.raises(ValueError):
        nsa.orthogonalize(m, workspace=torch.zeros(1 << 20, dtype=torch.uint8))


def test_exact_symmetry_and_orientation():
    # The tall result is the transpose of the wide result, bit for bit.
    dev = _dev()
    m = workloads.gaussian((180, 420), seed=27, dtype="fp16")
    for mode in ("standard", "gram"):
        a = m.to(dev)
        b = m.t().contiguous().to(dev)
        nsa.orthogonalize(a, mode=mode)
        nsa.orthogonalize(b, mode=mode)
        assert torch.equal(a, b.t())


# ---------------------------------------------------------------------------
# Larger single matrices with 256-wide tiles and ragged edges.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(2048, 4096), (2600, 2304), (1792, 5000)])
@pytest.mark.parametrize("mode", ["standard", "gram"])
def test_parity_large_ragged(shape, mode):
    m = workloads.column_scaled(shape[0], shape[1], seed=31, dtype="bf16")
    err = _rel(_run(m, mode), _oracle(m.double().numpy(), mode))
    print(f"{shape} {mode}: rel err {err:.3e}")
    assert err < 1e-2


# ---------------------------------------------------------------------------
# Every tile edge, forced: several tiles and a ragged tail in each direction.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("tile", [128, 192, 256])
@pytest.mark.parametrize("shape", [(700, 1300), (1300, 700), (384, 384)])
@pytest.mark.parametrize("mode", ["standard", "gram"])
def test_parity_forced_tile(tile, shape, mode):
    m = workloads.column_scaled(shape[0], shape[1], seed=41, dtype="bf16")
    err = _rel(_run(m, mode, tile=tile), _oracle(m.double().numpy(), mode))
    print(f"{shape} {mode} tile {tile}: rel err {err:.3e}")
    assert err < 1e-2


@pytest.mark.parametrize("tile", [128, 192, 256])
@pytest.mark.parametrize("mode", ["standard", "gram"])
def test_forced_tile_fp16_input(tile, mode):
    m = workloads.gaussian((520, 900), seed=42, dtype="fp16")
    err = _rel(_run(m, mode, tile=tile), _oracle(m.double().numpy(), mode))
    print(f"fp16 in, tile {tile}, {mode}: rel err {err:.3e}")
    assert err < 1e-2


# ---------------------------------------------------------------------------
# Batched launcher.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(200, 136), (136, 200), (256, 512)])
@pytest.mark.parametrize("mode", ["gram", "standard"])
def test_batched_matches_oracle_and_single_calls(shape, mode):
    dev = _dev()
    e = 5
    m = workloads.gaussian((e,) + shape, seed=28, dtype="bf16")
    x = m.to(dev)
    nsa.orthogonalize_batched(x, mode=mode)
    torch.cuda.synchronize()
    for i in range(e):
        single = m[i].to(dev)
        nsa.orthogonalize(single, mode=mode)
        assert torch.equal(single, x[i]), i
        err = _rel(x[i].double().cpu().numpy(),
                   _oracle(m[i].double().numpy(), mode))
        assert err < 1e-2, (i, err)


@pytest.mark.parametrize("mode", ["gram", "standard"])
@pytest.mark.parametrize("e", [40, 60])
def test_batched_persistent_grid_matches_single_calls(mode, e):
    # e matrices of 512 x 1000 on 128 tiles: 10 upper-triangle tiles and 32
    # update tiles per matrix.  With 40, the symmetric products (400 tiles)
    # run as a persistent grid looping over tiles of different matrices on
    # the one-work-group-per-CU kernels and the updates (1280 tiles) on the
    # two-work-groups-per-CU kernels; with 60, the symmetric products (600
    # tiles) take the two-per-CU persistent grid too.  Single calls use one
    # work-group per tile and the one-per-CU kernels.  Results must agree
    # bit for bit.
    dev = _dev()
    m = workloads.gaussian((e, 512, 1000), seed=29, dtype="bf16")
    x = m.to(dev)
    nsa.orthogonalize_batched(x, mode=mode, tile=128)
    torch.cuda.synchronize()
    for i in (0, 17, e - 1):
        single = m[i].to(dev)
        nsa.orthogonalize(single, mode=mode, tile=128)
        torch.cuda.synchronize()
        assert torch.equal(single, x[i]), i
        err = _rel(x[i].double().cpu().numpy(),
                   _oracle(m[i].double().numpy(), mode))
        assert err < 1e-2, (i, err)


# ---------------------------------------------------------------------------
# Soft-threshold split.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("numel_shape", [(1, 1), (3, 5), (64, 96), (333, 77),
                                         (512, 2048)])
def test_soft_threshold_matches_oracle(dtype, numel_shape):
    dev = _dev()
    m = workloads.student_t(numel_shape, seed=29, dtype=dtype)
    m64 = m.double().numpy()
    lam_out = torch.zeros(1, dtype=torch.float32, device=dev)
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    b, o = nsa.soft_threshold_split(m.to(dev), lambda_out=lam_out, status=st)
    torch.cuda.synchronize()
    assert st.item() == 0
    lam = lam_out.item()
    # The median is an order statistic of the stored values (exact), and
    # lambda is 3 * median rounded once to fp32.
    med = oracle.lower_median_abs(m64)
    assert lam == float(np.float32(3.0 * med))
    b = b.double().cpu().numpy()
    o = o.double().cpu().numpy()
    # Every clip decision, exactly: the oracle's split with the device's
    # lambda, B rounded to the storage type, equals the device's B.
    b_ref, o_ref, _ = oracle.soft_threshold_split(m64, lam=lam)
    b_ref16 = workloads.round_to(b_ref, dtype).double().numpy()
    assert np.array_equal(b, b_ref16)
    # O = M - B within one storage ulp of the exact outlier.
    ulp = {"bf16": 2.0 ** -7, "fp16": 2.0 ** -10, "fp32": 2.0 ** -23}[dtype]
    assert np.all(np.abs(o - o_ref) <= ulp * (np.abs(o_ref) + lam))


def test_soft_threshold_status_word():
    from newton_schulz_matrix_amd import _binding as B
    dev = _dev()
    m = workloads.student_t((64, 96), seed=33, dtype="bf16").to(dev)
    m[1, 2] = float("nan")
    st = torch.zeros(1, dtype=torch.int32, device=dev)
    b, _ = nsa.soft_threshold_split(m, status=st)
    torch.cuda.synchronize()
    assert st.item() == B.NS_ERR_NONFINITE | B.STATUS_AT_SPLIT
    assert torch.isnan(b[1, 2]) and torch.isfinite(b).sum() == b.numel() - 1


def test_soft_threshold_explicit_lambda_and_in_place():
    dev = _dev()
    m = workloads.student_t((100, 100), seed=30, dtype="bf16")
    x = m.to(dev)
    b, o = nsa.soft_threshold_split(x, lam=1.0, out_b=x)
    torch.cuda.synchronize()
    ref_b, ref_o, _ = oracle.soft_threshold_split(m.double().numpy(), lam=1.0)
    assert np.array_equal(x.double().cpu().numpy(), ref_b)
    assert np.abs(o.double().cpu().numpy() - ref_o).max() <= 2 ** -7 * (
        np.abs(ref_o).max() + 1)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_soft_threshold_unaligned_and_ragged(dtype):
    # A contiguous view that starts 3 elements into its buffer (not 16-byte
    # aligned) and has a ragged length takes the element-by-element paths;
    # the same values in an aligned buffer take the 16-byte ones.  The split
    # is elementwise and the median exact, so both agree bit for bit, and
    # with the oracle as in the test above.
    dev = _dev()
    numel = 100_003
    m = workloads.student_t((numel,), seed=31, dtype=dtype)
    torch_dtype = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    buf = torch.zeros(numel + 3, dtype=torch_dtype, device=dev)
    buf[3:] = m.to(dev)
    view = buf[3:]
    assert view.is_contiguous() and view.data_ptr() % 16 != 0
    lam_u = torch.zeros(1, dtype=torch.float32, device=dev)
    lam_a = torch.zeros(1, dtype=torch.float32, device=dev)
    b_u, o_u = nsa.soft_threshold_split(view, lambda_out=lam_u)
    aligned = m.to(dev)
    assert aligned.data_ptr() % 16 == 0
    b_a, o_a = nsa.soft_threshold_split(aligned, lambda_out=lam_a)
    torch.cuda.synchronize()
    assert lam_u.item() == lam_a.item()
    assert torch.equal(b_u, b_a) and torch.equal(o_u, o_a)
    m64 = m.double().numpy()
    assert lam_a.item() == pytest.approx(3.0 * oracle.lower_median_abs(m64), rel=1e-7)
    b_ref, _, lam_ref = oracle.soft_threshold_split(m64)
    clipped = np.abs(m64) > lam_ref
    assert np.array_equal(b_a.double().cpu().numpy()[~clipped], m64[~clipped])
    # Without the outlier output (O null) the robust part is the same.
    b_n, o_n = nsa.soft_threshold_split(aligned.clone(), outliers=False)
    torch.cuda.synchronize()
    assert o_n is None and torch.equal(b_n, b_a)


@pytest.mark.parametrize("mode", ["standard", "gram"])
@pytest.mark.parametrize("tall", [False, True])
def test_zero_rows_and_columns_stay_exactly_zero(mode, tall):
    # Rank-deficient by construction: zero rows and columns of X give zero
    # rows and columns of X X^T and of every n x n matrix built from it, so
    # the result keeps them exactly zero (p(0) = 0 needs no special case).
    # The rest is the orthogonalization of the nonzero submatrix.
    dev = _dev()
    m = workloads.gaussian((300, 700), seed=71, dtype="bf16").clone()
    zr, zc = [5, 77, 299], [0, 350, 699]
    m[zr, :] = 0
    m[:, zc] = 0
    if tall:
        m = m.t().contiguous()
    x = m.to(dev)
    nsa.orthogonalize(x, mode=mode)
    torch.cuda.synchronize()
    out = x.t() if tall else x
    assert torch.count_nonzero(out[zr, :]).item() == 0
    assert torch.count_nonzero(out[:, zc]).item() == 0
    ref = _oracle(m.double().numpy(), mode)
    assert _rel(x.double().cpu().numpy(), ref) < 1e-2


@pytest.mark.parametrize("mode", ["standard", "gram"])
@pytest.mark.parametrize("rank", [8, 40])
def test_low_rank_input_signal_and_null_parts(mode, rank):
    # M = A B^T of rank r, rounded to bf16.  On M's top-r right singular
    # subspace the result matches the oracle within the 1e-2 bar.  Off it,
    # both results hold only rounding noise that the iteration amplifies (up
    # to the product of the a_k, about 486, near zero): the oracle's from the
    # bf16 input, the device's from that plus its fp16 state, whose unit
    # roundoff (2^-11) is a quarter of bf16's (2^-9).  So the difference off
    # the subspace stays below half the oracle's own part there.
    dev = _dev()
    rng = np.random.default_rng(72 + rank)
    a, b = rng.standard_normal((300, rank)), rng.standard_normal((700, rank))
    m = workloads.round_to((a @ b.T).astype(np.float32), "bf16")
    m64 = m.double().numpy()
    x = m.to(dev)
    nsa.orthogonalize(x, mode=mode)
    torch.cuda.synchronize()
    out = x.double().cpu().numpy()
    ref = _oracle(m64, mode)
    vt = np.linalg.svd(m64, full_matrices=False)[2][:rank]
    sig = lambda y: y @ vt.T @ vt
    e_sig = np.linalg.norm(sig(out - ref)) / np.linalg.norm(sig(ref))
    null_err = np.linalg.norm((out - ref) - sig(out - ref))
    null_ref = np.linalg.norm(ref - sig(ref))
    print(f"rank {rank} {mode}: signal rel err {e_sig:.3e}, off-subspace "
          f"difference {null_err:.3e} against the oracle's {null_ref:.3e}")
    assert e_sig < 1e-2
    assert null_err < 0.5 * null_ref
