"""Pins of the oracle's SVDQuant weight preparation (oracle/svd_prep.py): matrices
whose singular values and vectors are fixed by construction, the closed forms
of the balanced split, and the residual identity.  CPU only."""
import numpy as np
import pytest

import oracle
from oracle import svd_prep


def _planted(rng, N, K, sigma):
    """W = U diag(sigma) V^T with orthonormal U [N, n], V [K, n] (QR of Gaussian
    matrices); exact in double, returned in double (not rounded)."""
    n = len(sigma)
    u, _ = np.linalg.qr(rng.standard_normal((N, n)))
    v, _ = np.linalg.qr(rng.standard_normal((K, n)))
    return (u * sigma[None, :]) @ v.T, u, v


def test_rank_one_closed_form():
    # W = 5 a b^T with unit a, b; its entries (0, +-1.5, +-2) are exact in
    # bf16: sigma = 5, l2 = +-sqrt(5) a, l1 = +-sqrt(5) b^T (one common sign)
    a = np.array([0.5, -0.5, 0.5, 0.5])
    b = np.array([0.0, 0.6, 0.8])
    w = 5.0 * np.outer(a, b)
    wb = oracle.f64_to_bf16(w)
    assert np.array_equal(oracle.bf16_to_f64(wb), w)
    sigma, u, vt = svd_prep.truncated_svd(wb, 1)
    l2, l1 = svd_prep.balanced_factors(sigma, u, vt)
    assert abs(sigma[0] - 5.0) < 1e-12
    sgn = np.sign(l2[0, 0]) * np.sign(a[0])
    assert np.allclose(l2[:, 0], sgn * np.sqrt(5.0) * a, atol=1e-12)
    assert np.allclose(l1[0], sgn * np.sqrt(5.0) * b, atol=1e-12)


def test_planted_spectrum_is_recovered():
    """Singular values fixed by construction: the oracle returns them, and its
    rank-r part is the constructed U_r S_r V_r^T (a transposed or sign-flipped
    factor would not reproduce it)."""
    rng = np.random.default_rng(0)
    N, K, r = 60, 40, 5
    sigma = 2.0 ** -np.arange(12, dtype=np.float64) * 4.0
    w, u, v = _planted(rng, N, K, sigma)
    wb = oracle.f64_to_bf16(w)
    w_q = oracle.bf16_to_f64(wb)     # the bf16 rounding moves sigma by < ||W - W_q||_2
    sig, uu, vt = svd_prep.truncated_svd(wb, r)
    slack = np.linalg.norm(w - w_q, 2)
    assert np.all(np.abs(sig - sigma[:r]) <= slack + 1e-12)
    l2, l1 = svd_prep.balanced_factors(sig, uu, vt)
    ref = (u[:, :r] * sigma[:r]) @ v[:, :r].T
    assert np.linalg.norm(l2 @ l1 - ref) <= 8 * slack * np.sqrt(r) + 1e-12


def test_balanced_split_norms_and_orthogonality():
    rng = np.random.default_rng(1)
    wb = oracle.f64_to_bf16(rng.standard_normal((48, 32)) * 0.1)
    sig, u, vt = svd_prep.truncated_svd(wb, 8)
    l2, l1 = svd_prep.balanced_factors(sig, u, vt)
    # each component splits its singular value evenly between the two factors
    assert np.allclose(np.linalg.norm(l2, axis=0), np.sqrt(sig), rtol=1e-12)
    assert np.allclose(np.linalg.norm(l1, axis=1), np.sqrt(sig), rtol=1e-12)
    assert np.allclose(l2.T @ l2, np.diag(sig), atol=1e-12)
    assert np.allclose(l1 @ l1.T, np.diag(sig), atol=1e-12)
    assert np.all(np.diff(sig) <= 0)


def test_eckart_young_residual_energy():
    """Closed form: for W = U diag(sigma) V^T the best rank-r error has squared
    Frobenius norm sum_{i > r} sigma_i^2; the oracle's unrounded split attains it."""
    rng = np.random.default_rng(2)
    sigma = np.linspace(3.0, 0.1, 20)
    w, _, _ = _planted(rng, 50, 30, sigma)
    wb = oracle.f64_to_bf16(w)
    w_q = oracle.bf16_to_f64(wb)
    for r in (1, 4, 10):
        sig, u, vt = svd_prep.truncated_svd(wb, r)
        l2, l1 = svd_prep.balanced_factors(sig, u, vt)
        tail = np.sum(np.linalg.svd(w_q, compute_uv=False)[r:] ** 2)
        assert abs(np.sum((w_q - l2 @ l1) ** 2) - tail) <= 1e-10 * np.sum(w_q ** 2)
        # and the constructed tail within the bf16 rounding of W
        assert abs(np.sqrt(tail) - np.sqrt(np.sum(sigma[r:] ** 2))) <= np.linalg.norm(w - w_q) + 1e-12


def test_residual_identity():
    """R is W minus the product of the stored bf16 factors, rounded once."""
    rng = np.random.default_rng(3)
    sigma = 2.0 ** -np.arange(8, dtype=np.float64)
    w, _, _ = _planted(rng, 24, 16, sigma)
    wb = oracle.f64_to_bf16(w)
    sig, l1b, l2b, rb = svd_prep.svdq_prepare(wb, 3)
    exact = oracle.bf16_to_f64(wb) - oracle.bf16_to_f64(l2b) @ oracle.bf16_to_f64(l1b)
    assert np.array_equal(rb, oracle.f64_to_bf16(exact))
    # |R| bounded by the tail plus the factor rounding
    assert np.linalg.norm(oracle.bf16_to_f64(rb)) <= np.sqrt(np.sum(sigma[3:] ** 2)) + 0.02 * np.sum(sigma[:3])


@pytest.mark.parametrize("r", [1, 16, 32])
def test_zero_matrix(r):
    sig, l1b, l2b, rb = svd_prep.svdq_prepare(np.zeros((64, 32), np.uint16), min(r, 32))
    assert np.all(sig == 0) and not l1b.any() and not l2b.any() and not rb.any()


def test_low_rank_and_residual_definitions():
    # hand-computed: l2 . l1 of these bf16-exact factors, and W = l2 . l1 + E
    # with every entry of W exact in bf16, so the residual must be E exactly
    # (a swapped operand, a sign or a transposition changes it)
    l2 = oracle.f64_to_bf16(np.array([[1.0, 0.5], [-2.0, 0.25], [0.0, 4.0]]))
    l1 = oracle.f64_to_bf16(np.array([[0.5, -1.0, 2.0, 0.0], [8.0, 0.125, -0.5, 1.0]]))
    p = np.array([[4.5, -0.9375, 1.75, 0.5],
                  [1.0, 2.03125, -4.125, 0.25],
                  [32.0, 0.5, -2.0, 4.0]])
    assert np.array_equal(svd_prep.low_rank(l2, l1), p)
    e = np.array([[0.5, 0.0, 0.0, -0.5], [0.0, 0.25, 0.0, 0.0], [1.0, 0.0, 0.0, 0.5]])
    w = oracle.f64_to_bf16(p + e)
    assert np.array_equal(oracle.bf16_to_f64(w), p + e)          # W is exact in bf16
    assert np.array_equal(oracle.bf16_to_f64(svd_prep.residual(w, l2, l1)), e)
    assert not svd_prep.residual(oracle.f64_to_bf16(p), l2, l1).any()


# ---------------------------------------------------------------------------
# The subspace iteration of the oracle (svd_prep.rsi, the method the GPU
# preparation computes) against the method's deterministic error bounds
# (Halko, Martinsson and Tropp 2011, Theorems 9.1 and 9.2 and the construction
# behind them), on planted spectra and a test matrix drawn as the GPU tests
# draw it.  The bounds come from the exact SVD and the test matrix alone.

def _omega(s, K, seed):
    import workloads
    return workloads.normal_bf16(np.random.default_rng(seed), (s, K), 1.0)


def _planted_bits(seed, N, K, sigma):
    w, _, _ = _planted(np.random.default_rng(seed), N, K, sigma)
    return oracle.f64_to_bf16(w)


SPECTRUM = 4.0 * 2.0 ** (-np.arange(128) / 4.0)


@pytest.mark.parametrize("r,s,iters", [(16, 32, 2), (32, 48, 2), (8, 32, 0), (48, 64, 1), (64, 64, 2), (4, 16, 1)])
def test_rsi_within_its_deterministic_bounds(r, s, iters):
    wb = _planted_bits(r + 100 * iters, 512, 384, SPECTRUM)
    om = _omega(s, 384, r + 7)
    sg, u, vt = svd_prep.rsi(wb, om, r, iters)
    b = svd_prep.rsi_bounds(wb, om, r, iters)
    lo, hi, spec, fro, opt = b["lo"], b["hi"], b["spec"], b["fro"], b["opt"]
    eps = 1e-12 * hi[0]
    assert np.all(sg >= lo - eps) and np.all(sg <= hi + eps)
    w = oracle.bf16_to_f64(wb)
    a = (u * sg[None, :]) @ vt
    assert np.linalg.norm(w - a, 2) <= spec + eps
    e = float(np.sum((w - a) ** 2))
    assert opt * (1 - 1e-12) - eps <= e <= fro * (1 + 1e-12) + eps   # Eckart-Young below, the bound above


def test_rsi_bounds_are_tight_enough_to_see_a_dropped_power_iteration():
    # the same test matrix without the two power iterations leaves the window
    # of the iterated method (a mistake the bounds must catch)
    wb = _planted_bits(232, 512, 384, SPECTRUM)
    om = _omega(48, 384, 39)
    b = svd_prep.rsi_bounds(wb, om, 32, 2)
    lo, hi = b["lo"], b["hi"]
    sg0, _, _ = svd_prep.rsi(wb, om, 32, 0)
    assert np.any(sg0 < lo)
    assert np.max(1 - lo / hi) < 1e-2


def test_rsi_exact_when_the_subspace_holds_the_range():
    # W = A B of rank 6 with small integer factors (entries exact in bf16),
    # s = 16 >= 6: F = 0 at the split k = 6, the window closes and the
    # iteration returns the exact SVD (no power iteration needed)
    rng = np.random.default_rng(5)
    w = rng.integers(-3, 4, (64, 6)).astype(np.float64) @ rng.integers(-3, 4, (6, 48)).astype(np.float64)
    wb = oracle.f64_to_bf16(w)
    assert np.array_equal(oracle.bf16_to_f64(wb), w) and np.linalg.matrix_rank(w) == 6
    om = _omega(16, 48, 1)
    b = svd_prep.rsi_bounds(wb, om, 6, 0)
    lo, hi = b["lo"], b["hi"]
    ref = np.linalg.svd(w, compute_uv=False)[:6]
    assert np.allclose(lo, hi, rtol=1e-10) and np.allclose(hi, ref, rtol=1e-12)
    sg, u, vt = svd_prep.rsi(wb, om, 6, 0)
    assert np.allclose(sg, ref, rtol=1e-10)
    assert np.linalg.norm(w - (u * sg[None, :]) @ vt) <= 1e-10 * np.linalg.norm(w)
