"""CPU oracle of the SVDQuant weight preparation -- TEST INFRASTRUCTURE.

Only the tests (and the benchmark's CPU-baseline leg) may import this module;
the product library never calls it.

OneTrainer PR #1034 "SVDQuant" and the wiki's SVDQuant entry: the weight is
split into a bf16 low-rank pair (of rank 16 to 32) plus a residual that is
quantized like any W8A8 weight.  The pages name the method only by its paper;
the split computed here is the plainest one that agrees with them:

  * the low-rank part is the rank-r truncated SVD of W, W_r = U_r S_r V_r^T
    (Eckart-Young: the best rank-r approximation in the Frobenius norm);
  * it is stored in the nn.Linear layout of the forward pass, balanced:
    l2 = U_r S_r^(1/2)  [N, r]  (up-projection),
    l1 = S_r^(1/2) V_r^T [r, K] (down-projection), both rounded to bf16;
  * the residual is R = bf16(W - l2 . l1), formed from the stored (bf16)
    factors in double, so that W ~ l2 . l1 + R holds for what is stored.

Arithmetic in float64; the SVD is numpy's LAPACK routine (a library step).
The GPU computes the truncated SVD by randomized subspace iteration; `rsi`
is that iteration in double on the same test matrix, and `rsi_bounds` the
method's deterministic error bounds for a given W and test matrix (the
windows its result must lie in).  bf16 values travel as uint16 bit patterns.
"""
import numpy as np

from . import bf16_to_f64, f64_to_bf16


def truncated_svd(w_bits, r):
    """Rank-r truncated SVD of the bf16 matrix W [N, K] in double.
    Returns (sigma [r], u [N, r], vt [r, K]); singular values descending."""
    w = bf16_to_f64(np.asarray(w_bits, np.uint16))
    u, s, vt = np.linalg.svd(w, full_matrices=False)
    return s[:r].copy(), u[:, :r].copy(), vt[:r].copy()


def balanced_factors(sigma, u, vt):
    """l2 = U S^(1/2), l1 = S^(1/2) V^T in double (before the bf16 rounding)."""
    root = np.sqrt(sigma)
    return u * root[None, :], vt * root[:, None]


def svdq_prepare(w_bits, r):
    """The whole preparation: returns (sigma f64 [r], l1 bf16 [r, K], l2 bf16 [N, r], residual bf16 [N, K])."""
    sigma, u, vt = truncated_svd(w_bits, r)
    l2, l1 = balanced_factors(sigma, u, vt)
    l2_bits, l1_bits = f64_to_bf16(l2), f64_to_bf16(l1)
    return sigma, l1_bits, l2_bits, residual(w_bits, l2_bits, l1_bits)


def residual(w_bits, l2_bits, l1_bits):
    """R = bf16(W - l2 . l1) from bf16 W [N, K], l2 [N, r], l1 [r, K], in double."""
    w = bf16_to_f64(np.asarray(w_bits, np.uint16))
    l2 = bf16_to_f64(np.asarray(l2_bits, np.uint16))
    l1 = bf16_to_f64(np.asarray(l1_bits, np.uint16))
    return f64_to_bf16(w - l2 @ l1)


def low_rank(l2_bits, l1_bits):
    """l2 . l1 in double from the stored bf16 factors."""
    return bf16_to_f64(np.asarray(l2_bits, np.uint16)) @ bf16_to_f64(np.asarray(l1_bits, np.uint16))


# ---------------------------------------------------------------------------
# The randomized subspace iteration itself, and what its theory fixes.
#
# Halko, Martinsson and Tropp, "Finding structure with randomness", SIAM
# Review 53 (2011): randomized subspace iteration (their Algorithm 4.4) on a
# test matrix G = Omega^T [K, s]:  Q = orth(W G); q times: Q = orth(W orth(W^T Q)).
# In exact arithmetic range(Q) = range((W W^T)^q W G); the approximation is
# the rank-r truncation of Q Q^T W.  The bounds below are deterministic given
# W and Omega (no expectation): they hold for every draw.


def rsi(w_bits, omega_bits, r, iters):
    """The subspace iteration in double on the caller's test matrix
    omega bf16 [s, K]: returns (sigma [r], u [N, r], vt [r, K]) of the rank-r
    truncation of Q Q^T W.  orth() is numpy's Householder QR (a library
    step); any orthonormal basis of the same range gives the same result."""
    w = bf16_to_f64(np.asarray(w_bits, np.uint16))
    g = bf16_to_f64(np.asarray(omega_bits, np.uint16)).T
    q, _ = np.linalg.qr(w @ g)
    for _ in range(iters):
        z, _ = np.linalg.qr(w.T @ q)
        q, _ = np.linalg.qr(w @ z)
    ub, s, vt = np.linalg.svd(q.T @ w, full_matrices=False)
    return s[:r].copy(), (q @ ub)[:, :r].copy(), vt[:r].copy()


def _rsi_terms(w_bits, omega_bits, iters):
    """Terms of the bounds for every split k = 1 .. min(s, rank): with the
    exact SVD W = U S V^T, G1 = V_k^T G [k, s], G2 = V_rest^T G and
    H_k = S_rest^(2q+1) G2 G1^+, the tangent of the captured subspace is
    F_k = H_k S_k^-(2q+1): range(Q) contains the columns of U_k + U_rest F_k.
    Returns (sigma of W, {k: (||F_k||_2, ||H_k||_2)}) over the splits where
    sigma_k > 0 and G1 has full row rank."""
    w = bf16_to_f64(np.asarray(w_bits, np.uint16))
    g = bf16_to_f64(np.asarray(omega_bits, np.uint16)).T
    _, sv, vt = np.linalg.svd(w, full_matrices=False)
    p = 2 * iters + 1
    terms = {}
    for k in range(1, min(g.shape[1], len(sv)) + 1):
        g1 = vt[:k] @ g
        if sv[k - 1] <= 0 or np.linalg.matrix_rank(g1) < k:
            continue
        h = (sv[k:] ** p)[:, None] * ((vt[k:] @ g) @ np.linalg.pinv(g1))
        if h.size == 0:
            terms[k] = (0.0, 0.0)
            continue
        terms[k] = (np.linalg.norm(h / (sv[:k] ** p)[None, :], 2), np.linalg.norm(h, 2))
    return sv, terms


def rsi_bounds(w_bits, omega_bits, r, iters):
    """Deterministic bounds on what the subspace iteration returns, from the
    exact SVD of W and the test matrix alone (Halko, Martinsson and Tropp
    2011, the construction of their Theorem 9.1 with the powers of their
    Section 9.2, and Theorem 9.2):

      sigma window, j = 1 .. r:
        lo_j = sigma_j / sqrt(1 + min_{k >= j} ||F_k||^2)  <=  sigma^_j  <=  sigma_j.
        Upper side: sigma^_j are the singular values of Q^T W, a projection
        of W (interlacing).  Lower side: range(Q) contains Z = U_k + U_rest F_k,
        so for j <= k, sigma^_j >= sigma_j(P_Z W V_k) = sigma_j(P_Z U_k S_k)
        >= sigma_min(P_Z U_k) sigma_j, and P_Z U_k = Z (I + F^T F)^-1 has
        sigma_min = 1 / sqrt(1 + ||F_k||^2).
      spectral residual of the rank-r result A_r:
        ||W - A_r||_2 <= sigma_{r+1} + min_{k >= r} (sigma_{k+1}^(2p) + ||H_k||^2)^(1/(2p)),
        p = 2q + 1: Theorem 9.1 for (W W^T)^q W bounds ||(I - P_Q) W||_2
        through Theorem 9.2, and the truncation to rank r adds at most
        sigma_{r+1}(P_Q W) <= sigma_{r+1}.
      Frobenius residual: W - A_r splits into (I - P_Q) W and P_Q W - A_r,
        orthogonal to each other, so ||W - A_r||_F^2 = ||W||_F^2 - sum_{j<=r} sigma^_j^2
        <= ||W||_F^2 - sum_{j<=r} lo_j^2; the optimum (Eckart-Young) is
        ||W||_F^2 - sum_{j<=r} sigma_j^2.

    Returns a dict: lo [r], hi [r] (= sigma_1..r of W), spec, fro (bound on
    the squared Frobenius residual), opt (its optimum)."""
    sv, terms = _rsi_terms(w_bits, omega_bits, iters)
    p = 2 * iters + 1
    hi = sv[:r].copy()
    lo = np.zeros(r)
    for j in range(1, r + 1):
        fs = [t[0] for k, t in terms.items() if k >= j]
        if fs:
            lo[j - 1] = hi[j - 1] / np.sqrt(1.0 + min(fs) ** 2)
    sig_r1 = float(sv[r]) if r < len(sv) else 0.0
    spec = np.inf
    for k, (_, hn) in terms.items():
        if k >= r:
            sk1 = float(sv[k]) if k < len(sv) else 0.0
            spec = min(spec, sig_r1 + (sk1 ** (2 * p) + hn * hn) ** (1.0 / (2 * p)))
    total = float(np.sum(sv ** 2))
    return {"lo": lo, "hi": hi, "spec": spec, "fro": total - float(np.sum(lo ** 2)),
            "opt": total - float(np.sum(hi ** 2))}
