"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each test names what fixes the expected value: a textbook routine
(numpy's LAPACK SVD), a closed form, an invariant of the iteration, or a
number printed on the pages (fixtures under tests/golden/, each with its
citation).
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import (CLASSIC_ABC, TUNED_ABC, frobenius_stage, gram_iterate,
                    jacobi_svd, lower_median_abs,
                    momentum_update, muon_step, ns_gram, ns_standard,
                    orthogonalization_mse, polar_eigh, polar_jacobi,
                    scalar_map, soft_threshold_split)
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rel(x, y):
    return float(np.linalg.norm(x - y) / np.linalg.norm(y))


# ---------------------------------------------------------------------------
# The coefficient fixture is what the oracle's constants must be.
# ---------------------------------------------------------------------------

def test_coefficients_match_fixture():
    g = _golden("coefficients.json")
    assert tuple(g["tuned_abc"]) == TUNED_ABC
    assert tuple(g["classic_abc"]) == CLASSIC_ABC
    assert g["steps"] == 5


# ---------------------------------------------------------------------------
# Jacobi SVD and the polar factor, against LAPACK and the definitions.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(9, 5), (16, 16), (30, 7)])
def test_jacobi_svd_against_lapack(shape):
    rng = np.random.default_rng(11)
    a = rng.standard_normal(shape)
    u, s, v = jacobi_svd(a)
    ref = np.linalg.svd(a, compute_uv=False)
    np.testing.assert_allclose(np.sort(s)[::-1], ref, rtol=1e-12, atol=0)
    np.testing.assert_allclose(u.T @ u, np.eye(shape[1]), atol=1e-12)
    np.testing.assert_allclose(v.T @ v, np.eye(shape[1]), atol=1e-12)
    np.testing.assert_allclose((u * s) @ v.T, a, atol=1e-12)


def test_polar_factors_agree_and_are_isometries():
    rng = np.random.default_rng(12)
    for shape in [(12, 20), (20, 12), (15, 15)]:
        a = rng.standard_normal(shape)
        pj = polar_jacobi(a)
        pe = polar_eigh(a)
        uu, _, vvt = np.linalg.svd(a, full_matrices=False)
        np.testing.assert_allclose(pj, uu @ vvt, atol=1e-12)
        np.testing.assert_allclose(pe, pj, atol=1e-10)
        k = min(shape)
        g = pj @ pj.T if shape[0] <= shape[1] else pj.T @ pj
        np.testing.assert_allclose(g, np.eye(k), atol=1e-12)


# ---------------------------------------------------------------------------
# P1: the classic triple run long enough converges to U V^T.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(4, 7), (8, 16), (16, 16), (7, 3)])
def test_classic_iteration_converges_to_polar(shape):
    rng = np.random.default_rng(sum(shape))
    a = rng.standard_normal(shape)
    exact = polar_jacobi(a)
    out_s = ns_standard(a, steps=40, abc=CLASSIC_ABC)
    out_g = ns_gram(a, steps=40, abc=CLASSIC_ABC, restart=(10, 20, 30))
    assert np.max(np.abs(out_s - exact)) < 1e-10
    assert np.max(np.abs(out_g - exact)) < 1e-10


# ---------------------------------------------------------------------------
# P4: designed spectrum, closed form U diag(p^T(s/||s||)) V^T.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(48, 130), (130, 48), (64, 64)])
@pytest.mark.parametrize("form", ["standard", "gram", "gram_naive"])
def test_designed_spectrum_closed_form(shape, form):
    k = min(shape)
    s = np.geomspace(1.0, 1e-3, k)
    m, u, v = workloads.designed_spectrum(shape[0], shape[1], s, seed=5)
    expect = (u * scalar_map(s / np.linalg.norm(s))[None, :]) @ v.T
    if form == "standard":
        out = ns_standard(m, eps=0.0)
    elif form == "gram":
        out = ns_gram(m, restart=(3,), eps=0.0)
    else:
        out = ns_gram(m, restart=(), eps=0.0)
    assert _rel(out, expect) < 1e-12


def test_designed_spectrum_per_step_coefficients():
    s = np.linspace(1.0, 0.01, 40)
    m, u, v = workloads.designed_spectrum(40, 90, s, seed=6)
    sched = [TUNED_ABC, CLASSIC_ABC, TUNED_ABC, (1.5, -0.5, 0.0),
             CLASSIC_ABC]
    expect = (u * scalar_map(s / np.linalg.norm(s), sched)[None, :]) @ v.T
    for out in (ns_standard(m, abc=sched, eps=0.0),
                ns_gram(m, abc=sched, restart=(2, 4), eps=0.0)):
        assert _rel(out, expect) < 1e-12


def test_rank_deficient_keeps_zero_singular_values():
    s = np.array([1.0, 0.5, 0.2, 0.0, 0.0, 0.0])
    m, u, v = workloads.designed_spectrum(6, 20, s, seed=7)
    expect = (u * scalar_map(s / np.linalg.norm(s))[None, :]) @ v.T
    assert _rel(ns_standard(m, eps=0.0), expect) < 1e-12
    assert _rel(ns_gram(m, eps=0.0), expect) < 1e-12


# ---------------------------------------------------------------------------
# P2: the Gram form equals the standard form in fp64.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("restart", [(), (3,), (2, 4), (2, 3, 4, 5)])
def test_gram_equals_standard(restart):
    m = workloads.column_scaled(96, 300, seed=8, dtype="fp64").numpy()
    ref = ns_standard(m)
    out = ns_gram(m, restart=restart)
    assert _rel(out, ref) < 1e-12


def test_gram_equals_standard_tall_bf16_input():
    m = workloads.gaussian((200, 64), seed=9, dtype="bf16").double().numpy()
    assert _rel(ns_gram(m), ns_standard(m)) < 1e-12


# ---------------------------------------------------------------------------
# The failure of naive Gram iterations ([Gram-NS], "Stability challenges and
# solutions"): a Gram matrix that lost positive semi-definiteness.  Its
# smallest eigenvalue is replaced by mu < 0 (same eigenvector u); every matrix
# of the recurrence is then a polynomial in that R, so along u the iteration
# is the scalar recurrence  w_k = a + b mu_k + c mu_k^2,  mu_{k+1} = mu_k w_k^2,
# with Q multiplied by w_k.  For mu < 0 every term of w_k is positive and
# mu_k runs off to minus infinity.
# ---------------------------------------------------------------------------

def _negative_gram(mu):
    m = workloads.gaussian((48, 160), seed=21, dtype="fp64").numpy()
    x, _ = frobenius_stage(m)
    r = x @ x.T
    lam, vec = np.linalg.eigh(r)
    u = vec[:, 0]
    return x, r + (mu - lam[0]) * np.outer(u, u), u


def test_naive_gram_from_a_negative_eigenvalue_follows_the_scalar_recurrence():
    mu0 = -1e-3
    x, r_bad, u = _negative_gram(mu0)
    sched = [TUNED_ABC] * 5
    out = gram_iterate(x, r_bad, sched, restart=())
    q_u, mu = 1.0, mu0
    for a, b, c in sched:
        w = a + b * mu + c * mu * mu
        q_u, mu = q_u * w, mu * w * w
    assert q_u > 1e9
    # Along u the result is q_u times X's component; elsewhere R is
    # untouched, so the rest equals the ordinary naive iteration.
    assert abs(float(u @ out @ (x.T @ u)) / float(u @ x @ x.T @ u) - q_u) < 1e-9 * q_u
    good = gram_iterate(x, x @ x.T, sched, restart=())
    proj = np.eye(len(u)) - np.outer(u, u)
    # fp64 rounding of the products leaks about eps * q_u of the huge
    # component along u into the others.
    assert _rel(proj @ out, proj @ good) < 1e-15 * q_u
    assert np.linalg.norm(out, 2) > 1e3


def test_restart_discards_the_negative_eigenvalue():
    x, r_bad, _ = _negative_gram(-1e-3)
    sched = [TUNED_ABC] * 5
    # A restart before step 2 recomputes R from X after one step: the
    # result is back in the band of the ordinary iteration.
    out = gram_iterate(x, r_bad, sched, restart=(2,))
    s = np.linalg.svd(out, compute_uv=False)
    assert np.all(np.isfinite(s)) and s.max() < 1.3
    ref = np.linalg.svd(gram_iterate(x, x @ x.T, sched, restart=(2,)), compute_uv=False)
    assert s.max() <= ref.max() + 1e-6


# ---------------------------------------------------------------------------
# P3: the tuned triple leaves singular values in roughly [0.7, 1.3].
# ---------------------------------------------------------------------------

def test_tuned_band():
    band = _golden("coefficients.json")["tuned_target_band"]
    # Scalar map on a dense grid of normalized singular values.
    x = np.geomspace(3e-3, 1.0, 20001)
    y = scalar_map(x)
    assert y.min() > 0.68 and y.max() < 1.21
    assert band[0] - 0.02 < y.min() and y.max() < band[1]
    # The matrix iteration does the same to a designed spectrum.
    s = np.concatenate([[1.0], np.geomspace(0.05, 4e-3, 79)])
    s = s / np.linalg.norm(s)
    assert s.min() > 3e-3
    m, _, _ = workloads.designed_spectrum(80, 200, s, seed=10)
    sv = np.linalg.svd(ns_standard(m, eps=0.0), compute_uv=False)
    assert sv.min() > 0.68 and sv.max() < 1.21
    # The classic triple (p(1) = 1, max of p on [0, 1] is 1.0018) moves the
    # small values up more slowly.
    yc = scalar_map(x, CLASSIC_ABC)
    assert np.all(yc <= 1.0019) and yc.min() < y.min()


# ---------------------------------------------------------------------------
# Invariants: orientation, sign, scale, orthogonal equivariance, zero.
# ---------------------------------------------------------------------------

def test_invariants():
    rng = np.random.default_rng(13)
    m = rng.standard_normal((24, 60))
    out = ns_standard(m)
    np.testing.assert_allclose(ns_standard(m.T), out.T, atol=1e-13)
    np.testing.assert_allclose(ns_standard(-m), -out, atol=1e-13)
    np.testing.assert_allclose(ns_standard(7.5 * m, eps=0.0),
                               ns_standard(m, eps=0.0), atol=1e-12)
    qa, _ = np.linalg.qr(rng.standard_normal((24, 24)))
    qb, _ = np.linalg.qr(rng.standard_normal((60, 60)))
    np.testing.assert_allclose(ns_standard(qa @ m @ qb, eps=0.0),
                               qa @ ns_standard(m, eps=0.0) @ qb, atol=1e-12)
    np.testing.assert_allclose(ns_gram(qa @ m @ qb, eps=0.0),
                               qa @ ns_gram(m, eps=0.0) @ qb, atol=1e-12)


def test_zero_and_single_row():
    z = np.zeros((5, 9))
    assert np.all(ns_standard(z) == 0) and np.all(ns_gram(z) == 0)
    row = np.arange(1.0, 11.0)[None, :]
    expect = scalar_map(1.0) * row / np.linalg.norm(row)
    np.testing.assert_allclose(ns_standard(row, eps=0.0), expect, atol=1e-14)
    np.testing.assert_allclose(ns_gram(row, eps=0.0), expect, atol=1e-14)


# ---------------------------------------------------------------------------
# P5: the ROOT page's printed MSE for 2048 x 2048.
# ---------------------------------------------------------------------------

def test_root_page_mse_2048():
    g = _golden("root_mse.json")
    r, c = g["shape"]
    m = np.random.default_rng(0).standard_normal((r, c))
    mse = orthogonalization_mse(ns_standard(m), m)
    assert abs(mse - g["mse"]) < g["tolerance_abs"], mse
    # The per-entry mean is not what the page reports.
    assert orthogonalization_mse(ns_standard(m), m) / c < 1e-3 * g["mse"]


# ---------------------------------------------------------------------------
# P6: soft-threshold split.
# ---------------------------------------------------------------------------

def test_lower_median_brute_force():
    rng = np.random.default_rng(14)
    for n in (1, 2, 7, 100, 101):
        x = rng.standard_normal(n)
        vals = sorted(abs(float(t)) for t in x)
        assert lower_median_abs(x) == vals[(n + 1) // 2 - 1]


def test_soft_threshold_closed_form_and_optimality():
    rng = np.random.default_rng(15)
    m = rng.standard_t(2.0, size=(64, 96))
    b, o, lam = soft_threshold_split(m)
    assert lam == 3.0 * lower_median_abs(m)
    np.testing.assert_allclose(b + o, m, rtol=0, atol=1e-14 * np.abs(m).max())
    assert np.all(np.abs(b) <= lam) and np.all(b[np.abs(m) <= lam] ==
                                               m[np.abs(m) <= lam])
    assert np.all(np.abs(b[np.abs(m) > lam]) == lam)
    # Subgradient optimality of O for 1/2 ||M - O||^2 + lam ||O||_1.
    nz = o != 0
    np.testing.assert_allclose((m - o)[nz], lam * np.sign(o[nz]), atol=1e-14)
    assert np.all(np.abs(m[~nz]) <= lam)
    # Explicit lambda is honoured; lambda above max|M| leaves O = 0.
    b2, o2, lam2 = soft_threshold_split(m, lam=np.abs(m).max() + 1)
    assert np.all(o2 == 0) and np.array_equal(b2, m)


def test_soft_threshold_student_t_statistics():
    # For t(2): P(|T| <= x) = x / sqrt(2 + x^2), so median |T| = sqrt(2/3),
    # lambda = 3 sqrt(2/3) = sqrt(6) and P(|T| > lambda) = 1 - sqrt(3)/2.
    m = workloads.heavy_tailed().double().numpy()
    b, o, lam = soft_threshold_split(m)
    assert abs(lam - math.sqrt(6.0)) < 0.01 * math.sqrt(6.0)
    frac = float(np.mean(o != 0))
    assert abs(frac - (1.0 - math.sqrt(3.0) / 2.0)) < 2e-3


# ---------------------------------------------------------------------------
# Muon step: momentum recurrence and the whole update in closed form.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nesterov", [True, False])
def test_momentum_constant_gradient_geometric_series(nesterov):
    # With M_0 = 0 and a constant gradient G, M_t = G (1 - mu^t) / (1 - mu):
    # the sum of a geometric series, independent of the recurrence's code.
    rng = np.random.default_rng(0)
    g = rng.standard_normal((5, 7))
    mu = 0.95
    m = np.zeros_like(g)
    for t in range(1, 13):
        m, u = momentum_update(m, g, mu, nesterov)
        geo = (1.0 - mu ** t) / (1.0 - mu)
        assert np.allclose(m, geo * g, rtol=1e-13, atol=0)
        expect_u = g * (1.0 + mu * geo) if nesterov else geo * g
        assert np.allclose(u, expect_u, rtol=1e-13, atol=0)


@pytest.mark.parametrize("mode", ["standard", "gram"])
@pytest.mark.parametrize("nesterov", [True, False])
def test_muon_step_designed_spectrum(mode, nesterov):
    # G = U diag(s) V^T and M = c G: the step's NS input is a multiple of G,
    # Frobenius normalization removes the multiple, so
    # W' = W - lr U diag(p^T(s / ||s||)) V^T exactly (eps = 0).
    s = np.geomspace(1.0, 2e-3, 24)
    g, u, v = workloads.designed_spectrum(24, 60, s, seed=11)
    rng = np.random.default_rng(1)
    w = rng.standard_normal(g.shape)
    m0 = 0.3 * g
    lr = 0.02
    w1, m1 = muon_step(w, g, m0, lr, 0.95, nesterov, mode=mode, eps=0.0)
    expect_o = (u * scalar_map(s / np.linalg.norm(s))[None, :]) @ v.T
    assert _rel(w - w1, lr * expect_o) < 1e-12
    assert np.allclose(m1, 0.95 * m0 + g, rtol=1e-14, atol=1e-15)


def test_muon_step_zero_lr_and_inputs_untouched():
    rng = np.random.default_rng(2)
    w = rng.standard_normal((8, 20))
    g = rng.standard_normal((8, 20))
    m = rng.standard_normal((8, 20))
    copies = (w.copy(), g.copy(), m.copy())
    w1, m1 = muon_step(w, g, m, 0.0)
    assert np.array_equal(w1, w)
    for a, b in zip((w, g, m), copies):
        assert np.array_equal(a, b)
