"""Pins of the fp64 oracle against mathematics that does not go through it.

Each pin takes a different route to the same number (an SVD closed form, exact
rational arithmetic, a scalar recursion, a library polar decomposition, an
invariant of the method), so that a plausible slip in the oracle (a dropped
term, a wrong sign, a transposed operand, eps in the wrong place, a missing
transpose back) fails at least one of them.  The planted-mistake tests at the
end check exactly that.
"""

from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import ns_oracle
from oracle.ns_oracle import DEFAULT_COEFFS, EPS, newton_schulz, newton_schulz_batched

COEFF_SETS = [DEFAULT_COEFFS, (1.5, -0.5, 0.0), (2.0, -1.5, 0.5), (0.7, 0.3, -0.2)]


def scalar_poly_iter(s, coeffs, steps):
    """p^k(s) with p(x) = a x + b x^3 + c x^5 (works on floats, arrays, Fractions)."""
    a, b, c = coeffs
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s


def svd_closed_form(x, steps, coeffs, eps=EPS):
    """NS acts on singular values only: X = U S Vᵀ maps to U p^k(S/(||X||_F+eps)) Vᵀ.

    Each step is an odd matrix polynomial of X: with A = U S² Uᵀ,
    b A + c A² = U (b S² + c S⁴) Uᵀ and so aX + B X = U (aS + bS³ + cS⁵) Vᵀ.
    """
    x = np.asarray(x, dtype=np.float64)
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    s0 = s / (np.linalg.norm(s) + eps)  # ||X||_F = sqrt(sum s²)
    return (u * scalar_poly_iter(s0, coeffs, steps)) @ vt


def rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


@pytest.mark.parametrize("shape", [(8, 12), (12, 8), (64, 96), (96, 64), (16, 16), (1, 7), (7, 1)])
@pytest.mark.parametrize("coeffs", COEFF_SETS)
@pytest.mark.parametrize("steps", [0, 1, 5])
def test_svd_closed_form(shape, coeffs, steps):
    rng = np.random.default_rng(sum(shape) * 31 + steps)
    x = rng.standard_normal(shape)
    y = newton_schulz(x, steps, coeffs)
    assert y.shape == x.shape
    assert rel(y, svd_closed_form(x, steps, coeffs)) <= 1e-12


def test_svd_closed_form_batch_of_three():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 20, 33)) * np.array([1e-3, 1.0, 30.0])[:, None, None]
    y = newton_schulz_batched(x)
    for i in range(3):
        assert rel(y[i], svd_closed_form(x[i], 5, DEFAULT_COEFFS)) <= 1e-12


# ---------------------------------------------------------------- exact rational

def _frac(v):
    return Fraction(v).limit_denominator(10 ** 12) if isinstance(v, float) else Fraction(v)


def _mm(p, q):
    return [[sum(p[i][k] * q[k][j] for k in range(len(q))) for j in range(len(q[0]))]
            for i in range(len(p))]


def _exact_ns(x_int, norm_int, steps, coeffs):
    """Brute-force NS of a small integer matrix with integer Frobenius norm, in
    exact rational arithmetic (eps = 1e-7 exactly)."""
    a, b, c = (Fraction(str(v)) for v in coeffs)
    eps = Fraction(1, 10 ** 7)
    X = [[Fraction(v) / (norm_int + eps) for v in row] for row in x_int]
    tall = len(X) > len(X[0])
    if tall:
        X = [list(r) for r in zip(*X)]
    for _ in range(steps):
        Xt = [list(r) for r in zip(*X)]
        A = _mm(X, Xt)
        AA = _mm(A, A)
        B = [[b * A[i][j] + c * AA[i][j] for j in range(len(A))] for i in range(len(A))]
        BX = _mm(B, X)
        X = [[a * X[i][j] + BX[i][j] for j in range(len(X[0]))] for i in range(len(X))]
    if tall:
        X = [list(r) for r in zip(*X)]
    return np.array([[float(v) for v in row] for row in X])


@pytest.mark.parametrize("x_int,norm", [
    ([[3, 4]], 5),
    ([[3], [4]], 5),
    ([[2, 1], [2, 4]], 5),
    ([[1, 2, 2], [2, -2, 1], [2, 1, -2], [0, 0, 3]], 6),
    ([[2, 0, 1], [0, 2, 0], [4, 0, 0]], 5),
    ([[4, 0, 2], [0, 2, 1]], 5),
    ([[1, 0, 2, 2], [0, 4, 0, 0]], 5),
])
def test_exact_rational_bruteforce(x_int, norm):
    sq = sum(v * v for row in x_int for v in row)
    r = int(round(np.sqrt(sq)))
    assert r * r == sq == norm * norm, "each case has an integer Frobenius norm"
    exact = _exact_ns(x_int, r, 5, DEFAULT_COEFFS)
    got = newton_schulz(np.array(x_int, dtype=np.float64))
    assert np.max(np.abs(got - exact)) <= 1e-14 * max(1.0, np.max(np.abs(exact)))


def test_rank_one_value():
    # [[3, 4]] has the single singular value 5; normalised it is 5/(5+eps), and
    # the output is p^5 of that times the unit direction [0.6, 0.8].
    eps = Fraction(1, 10 ** 7)
    coeffs = tuple(Fraction(str(v)) for v in DEFAULT_COEFFS)
    sigma = scalar_poly_iter(Fraction(5) / (5 + eps), coeffs, 5)
    got = newton_schulz(np.array([[3.0, 4.0]]))
    want = np.array([[0.6, 0.8]]) * float(sigma)
    assert np.max(np.abs(got - want)) <= 1e-14
    assert abs(float(sigma) - 0.69643643004713) < 1e-13


# ---------------------------------------------------------------- special cases

@pytest.mark.parametrize("m,s", [(256, 1.0), (64, 3.0), (8, 1e-2)])
def test_scaled_identity(m, s):
    x = s * np.eye(m)
    sigma0 = s / (s * np.sqrt(m) + EPS)
    want = scalar_poly_iter(sigma0, DEFAULT_COEFFS, 5)
    y = newton_schulz(x)
    assert np.allclose(y, want * np.eye(m), rtol=1e-13, atol=1e-15)
    if m == 256 and s == 1.0:
        # eps-free value of p^5(1/16)
        assert abs(scalar_poly_iter(1 / 16, DEFAULT_COEFFS, 5) - 1.0705244477) < 1e-9


def test_rectangular_diagonal_maps_elementwise():
    d = np.array([3.0, -1.0, 0.5, 2.0])
    x = np.zeros((4, 7))
    x[np.arange(4), np.arange(4)] = d
    y = newton_schulz(x)
    s0 = np.abs(d) / (np.linalg.norm(d) + EPS)
    want = np.zeros_like(x)
    want[np.arange(4), np.arange(4)] = np.sign(d) * scalar_poly_iter(s0, DEFAULT_COEFFS, 5)
    assert np.max(np.abs(y - want)) <= 1e-15


def test_zero_steps_and_identity_coeffs_give_normalised_input():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((9, 14))
    n = x / (np.sqrt((x * x).sum()) + EPS)
    assert np.array_equal(newton_schulz(x, steps=0), n)
    assert rel(newton_schulz(x, steps=5, coeffs=(1.0, 0.0, 0.0)), n) <= 1e-15


def test_zero_matrix_gives_zero():
    y = newton_schulz(np.zeros((5, 9)))
    assert np.all(y == 0)


# ---------------------------------------------------------------- polar factor

@pytest.mark.parametrize("shape", [(12, 8), (8, 12), (10, 10)])
def test_cubic_coefficients_converge_to_polar_factor(shape):
    # (a, b, c) = (1.5, -0.5, 0) is the cubic Newton–Schulz iteration, which
    # converges to the orthogonal polar factor for singular values in (0, √3).
    rng = np.random.default_rng(11)
    m, n = shape
    q1, _ = np.linalg.qr(rng.standard_normal((m, m)))
    q2, _ = np.linalg.qr(rng.standard_normal((n, n)))
    k = min(m, n)
    s = np.linspace(0.3, 1.0, k)
    x = q1[:, :k] @ np.diag(s) @ q2[:, :k].T
    y = newton_schulz(x, steps=60, coeffs=(1.5, -0.5, 0.0))
    if m >= n:
        want = scipy.linalg.polar(x)[0]
    else:
        want = scipy.linalg.polar(x.T)[0].T
    assert np.max(np.abs(y - want)) <= 1e-10


# ---------------------------------------------------------------- invariants

def test_gram_is_symmetric():
    rng = np.random.default_rng(2)
    x = ns_oracle.frobenius_normalize(rng.standard_normal((40, 70)))
    a = x @ x.T
    assert np.linalg.norm(a - a.T) <= 1e-15 * np.linalg.norm(a)


def test_tall_is_transpose_of_wide():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((30, 50))
    assert np.array_equal(newton_schulz(x.T), newton_schulz(x).T)


def test_batch_slices_are_independent():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 16, 24)) * np.array([1, 10, 1e-2, 3])[:, None, None]
    y = newton_schulz_batched(x)
    for i in range(4):
        assert np.array_equal(y[i], newton_schulz(x[i]))
    sub = newton_schulz_batched(x, slices=[2, 0])
    assert np.array_equal(sub[0], y[2]) and np.array_equal(sub[1], y[0])


@pytest.mark.parametrize("s", [1e-3, 1e3])
def test_scale_invariance(s):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((20, 32))
    assert rel(newton_schulz(s * x, eps=0.0), newton_schulz(x, eps=0.0)) <= 1e-12
    # with eps, the change is bounded by the relative size of eps
    assert rel(newton_schulz(s * x), newton_schulz(x)) <= 1e-4


def test_orthogonal_equivariance():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((16, 24))
    q, _ = np.linalg.qr(rng.standard_normal((16, 16)))
    r, _ = np.linalg.qr(rng.standard_normal((24, 24)))
    assert rel(newton_schulz(q @ x @ r), q @ newton_schulz(x) @ r) <= 1e-12


def test_singular_value_band():
    # p(x) = a x + b x³ + c x⁵ has critical points where p'(x) = 0, i.e.
    # x² = (-3b ± sqrt(9b² - 20ac)) / (10c).  Between them p has a local max
    # and a local min; once every singular value is in the band they bound,
    # later steps keep it there.
    a, b, c = DEFAULT_COEFFS
    disc = np.sqrt(9 * b * b - 20 * a * c)
    xs = np.sqrt(np.array([(-3 * b - disc) / (10 * c), (-3 * b + disc) / (10 * c)]))
    p = lambda v: a * v + b * v ** 3 + c * v ** 5
    hi, lo = p(xs[0]), p(xs[1])
    assert abs(hi - 1.202369) < 1e-5 and abs(lo - 0.681831) < 1e-5
    rng = np.random.default_rng(8)
    x = rng.standard_normal((32, 256))  # well conditioned: normalised σ >= ~0.05
    s_in = np.linalg.svd(x / np.linalg.norm(x), compute_uv=False)
    assert s_in.min() > 0.003
    s_out = np.linalg.svd(newton_schulz(x), compute_uv=False)
    assert s_out.min() >= lo - 1e-9 and s_out.max() <= hi + 1e-9


# ---------------------------------------------------------------- planted mistakes

MUTANTS = {
    "drop_bA": lambda X, a, b, c: a * X + (c * ((X @ X.T) @ (X @ X.T))) @ X,
    "drop_cAA": lambda X, a, b, c: a * X + (b * (X @ X.T)) @ X,
    "sign_a": lambda X, a, b, c: -a * X + (b * (X @ X.T) + c * ((X @ X.T) @ (X @ X.T))) @ X,
    "XB_for_BX": lambda X, a, b, c: a * X + X @ (b * (X.T @ X) + c * ((X.T @ X) @ (X.T @ X))).T
    if X.shape[0] == X.shape[1] else a * X + (b * (X @ X.T)) @ X,
    "swap_b_c": lambda X, a, b, c: a * X + (c * (X @ X.T) + b * ((X @ X.T) @ (X @ X.T))) @ X,
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistakes_are_caught(name, monkeypatch):
    monkeypatch.setattr(ns_oracle, "ns_iteration", MUTANTS[name])
    rng = np.random.default_rng(9)
    caught = False
    for shape in [(10, 10), (8, 12)]:
        x = rng.standard_normal(shape)
        # XB_for_BX differs from BX only when X is not normal: use a square
        # non-symmetric X (generic Gaussian) for it
        with np.errstate(all="ignore"):
            y = ns_oracle.newton_schulz(x)
            if not np.all(np.isfinite(y)) or not rel(y, svd_closed_form(x, 5, DEFAULT_COEFFS)) <= 1e-6:
                caught = True
    assert caught, f"mutant {name} not caught by the closed form"


def test_planted_eps_inside_sqrt_is_caught(monkeypatch):
    def bad(x, eps=EPS):
        x = np.asarray(x, dtype=np.float64)
        return x / np.sqrt(np.sum(x * x) + eps)
    monkeypatch.setattr(ns_oracle, "frobenius_normalize", bad)
    got = ns_oracle.newton_schulz(np.array([[3.0, 4.0]]))
    eps = Fraction(1, 10 ** 7)
    coeffs = tuple(Fraction(str(v)) for v in DEFAULT_COEFFS)
    want = float(scalar_poly_iter(Fraction(5) / (5 + eps), coeffs, 5)) * np.array([[0.6, 0.8]])
    assert np.max(np.abs(got - want)) > 1e-12


def test_planted_missing_transpose_back_is_caught(monkeypatch):
    def bad(x, steps=5, coeffs=DEFAULT_COEFFS, eps=EPS):
        X = np.array(x, dtype=np.float64)
        if X.shape[0] > X.shape[1]:
            X = X.T
        X = ns_oracle.frobenius_normalize(X, eps)
        for _ in range(steps):
            X = ns_oracle.ns_iteration(X, *coeffs)
        return X
    rng = np.random.default_rng(10)
    x = rng.standard_normal((12, 8))
    y = bad(x)
    assert y.shape != x.shape or rel(y, svd_closed_form(x, 5, DEFAULT_COEFFS)) > 1e-6


def test_flops_formula():
    # 4096² square: 5 * (4 m² n + 2 m³) with m = n = 4096
    assert oracle.dense_equivalent_flops(1, 4096, 4096) == 5 * 6 * 4096 ** 3
    assert oracle.dense_equivalent_flops(128, 1536, 2048) == 128 * 5 * (4 * 1536 ** 2 * 2048 + 2 * 1536 ** 3)
    assert oracle.dense_equivalent_flops(1, 14336, 4096) == oracle.dense_equivalent_flops(1, 4096, 14336)


# ---------------------------------------------------------------- step helpers

@pytest.mark.parametrize("shape", [(12, 20), (20, 12), (16, 16)])
def test_step_helpers_compose_to_one_iteration(shape):
    # the per-step helpers (used as references for single kernels) regroup
    # exactly the iteration: aX + (bA + cAA)X = (aI + bA + cAA)X, and for a
    # tall X the same step on Xᵀ, transposed back.
    rng = np.random.default_rng(12)
    x = ns_oracle.frobenius_normalize(rng.standard_normal(shape))
    a, b, c = DEFAULT_COEFFS
    C = ns_oracle.poly_matrix(ns_oracle.gram_matrix(x), a, b, c)
    got = ns_oracle.apply_update(x, C)
    want = ns_oracle.ns_iteration(x.T, a, b, c).T if shape[0] > shape[1] else ns_oracle.ns_iteration(x, a, b, c)
    assert rel(got, want) <= 1e-14
    assert ns_oracle.gram_matrix(x).shape == (min(shape), min(shape))
