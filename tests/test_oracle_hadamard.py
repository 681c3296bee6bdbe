"""Pins of the oracle's Hadamard rotation: the Sylvester matrix built by
Kronecker products (numpy, independent of the fast transform), involution,
norm preservation, and the invariance of the linear product.  CPU only."""
import numpy as np
import pytest

import oracle


def _sylvester(b):
    h = np.array([[1.0]])
    while h.shape[0] < b:
        h = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), h)
    return h


@pytest.mark.parametrize("K,b", [(16, 16), (48, 16), (96, 32), (1024, 1024), (3072, 1024), (4096, 1024),
                                 (12288, 1024), (80, 16), (200, 8)])
def test_block_size(K, b):
    assert oracle.hadamard_block(K) == b


@pytest.mark.parametrize("K", [16, 64, 96, 1024, 3072])
def test_matches_sylvester_matrix(K):
    """Integer inputs small enough that every f32 sum is exact: the fast
    transform equals x . blockdiag(H_b) / sqrt(b) computed in double."""
    rng = np.random.default_rng(K)
    M = 5
    x = rng.integers(-64, 65, (M, K)).astype(np.float64)
    xb = oracle.f64_to_bf16(x)
    b = oracle.hadamard_block(K)
    h = _sylvester(b) / np.sqrt(b)
    ref = np.concatenate([x[:, j:j + b] @ h for j in range(0, K, b)], axis=1)
    got = oracle.hadamard_rows_f32(xb).astype(np.float64)
    # exact sums; only the final multiply by f32(1/sqrt(b)) rounds
    assert np.allclose(got, ref, rtol=2 ** -22, atol=1e-12)  # atol: double rounding of h in the reference
    if b in (16, 64, 256, 1024):      # 1/sqrt(b) is a power of two: exact
        assert np.array_equal(got, ref)


def test_unit_vectors_give_hadamard_rows():
    K = 64
    b = oracle.hadamard_block(K)
    eye = oracle.f64_to_bf16(np.eye(K))
    got = oracle.hadamard_rows_f32(eye).astype(np.float64)
    assert np.array_equal(got, _sylvester(b) / 8.0)     # H_64 / sqrt(64), symmetric


def test_involution_and_norm():
    """H_b / sqrt(b) is symmetric and orthogonal: applying it twice returns the
    input (exactly, for small integers and b = 1024); norms are preserved."""
    rng = np.random.default_rng(1)
    x = rng.integers(-100, 101, (3, 3072)).astype(np.float64)
    once = oracle.hadamard_rows_f32(oracle.f64_to_bf16(x)).astype(np.float64)
    assert np.allclose(np.linalg.norm(once, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)
    # values of `once` are multiples of 1/32 below 2^12: exact in bf16 only if
    # short; compare the double transform of `once` instead
    b = 1024
    h = _sylvester(b) / np.sqrt(b)
    twice = np.concatenate([once[:, j:j + b] @ h for j in range(0, 3072, b)], axis=1)
    assert np.allclose(twice, x, atol=1e-9)


def test_rotated_linear_is_invariant():
    """(X H)(W H)^T = X W^T: the rotated, quantized linear approximates the
    unrotated product within the quantization error of both operands."""
    rng = np.random.default_rng(2)
    M, N, K = 16, 24, 2048
    x = rng.standard_normal((M, K))
    x[:, rng.choice(K, 4, replace=False)] *= 30.0          # outlier channels
    w = rng.standard_normal((N, K)) * 0.02
    xb, wb = oracle.f64_to_bf16(x), oracle.f64_to_bf16(w)
    ref = oracle.bf16_to_f64(xb) @ oracle.bf16_to_f64(wb).T
    xq, sx = oracle.quant_act_rowwise_hadamard(oracle.INT8, xb)
    wr = oracle.hadamard_rotate_bf16(wb)
    wq, _, sw = oracle.quant_weight_tensorwise(oracle.INT8, wr)
    y = oracle.bf16_to_f64(oracle.linear(oracle.INT8, xq, sx, wq, sw))
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    # without rotation the outliers inflate the activation scales
    xq0, sx0 = oracle.quant_act_rowwise(oracle.INT8, xb)
    wq0, _, sw0 = oracle.quant_weight_tensorwise(oracle.INT8, wb)
    y0 = oracle.bf16_to_f64(oracle.linear(oracle.INT8, xq0, sx0, wq0, sw0))
    rel0 = np.linalg.norm(y0 - ref) / np.linalg.norm(ref)
    assert rel < 0.02 and rel < rel0


def test_hadamard_quant_scale_rule():
    rng = np.random.default_rng(3)
    x = oracle.f64_to_bf16(rng.standard_normal((4, 96)))
    for qt, qmax in ((oracle.INT8, 127.0), (oracle.FP8_E4M3, 448.0)):
        q, s = oracle.quant_act_rowwise_hadamard(qt, x)
        v = oracle.hadamard_rows_f32(x)
        amax = np.abs(v).max(axis=1)
        assert np.array_equal(s, (amax / np.float32(qmax)).astype(np.float32))
