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
bf16 values travel as uint16 bit patterns.
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
