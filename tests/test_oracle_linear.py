"""Pins of the oracle's 8-bit products: brute force and numpy integer matmul,
a hand-worked linear, exact fp8 special cases, the SVDQuant reductions and the
backward identity.  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from helpers import bf16_to_f64

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(vals):
    return workloads.f32_to_bf16_bits(np.asarray(vals, np.float32))


def _padded(rows, width):
    out = np.zeros((len(rows), width), np.float32)
    for i, r in enumerate(rows):
        out[i, :len(r)] = r
    return out


def test_gemm_i32_brute_force_and_numpy():
    rng = np.random.default_rng(0)
    for (M, N, K) in [(1, 1, 1), (3, 5, 7), (17, 9, 64), (33, 40, 130)]:
        a = rng.integers(-128, 128, (M, K), dtype=np.int8)
        b = rng.integers(-128, 128, (N, K), dtype=np.int8)
        acc = oracle.gemm_i32(a, b)
        ref = a.astype(np.int64) @ b.astype(np.int64).T
        assert np.array_equal(acc, ref)
        if M * N * K <= 300:
            for m in range(M):
                for n in range(N):
                    s = 0
                    for k in range(K):
                        s += int(a[m, k]) * int(b[n, k])
                    assert acc[m, n] == s


def test_gemm_i32_extremes():
    K = 3072
    a = np.full((2, K), -128, np.int8)
    b = np.full((2, K), -128, np.int8)
    b[1] = 127
    acc = oracle.gemm_i32(a, b)
    assert acc[0, 0] == K * 128 * 128 and acc[0, 1] == -K * 128 * 127


def test_linear_worked_example():
    with open(os.path.join(GOLD, "linear_int8_tiny.json")) as f:
        g = json.load(f)
    K = g["K"]
    x = _bf16(_padded(g["x_rows"], K))
    w = _bf16(_padded(g["w_rows"], K))
    xq, sx = oracle.quant_act_rowwise(oracle.INT8, x)
    wq, _, sw = oracle.quant_weight_tensorwise(oracle.INT8, w)
    assert sx.tolist() == g["x_scale"] and sw == np.float32(g["w_scale"])
    assert np.array_equal(xq.view(np.int8), _padded(g["x_codes"], K).astype(np.int8))
    assert np.array_equal(wq.view(np.int8), _padded(g["w_codes"], K).astype(np.int8))
    assert oracle.gemm_i32(xq.view(np.int8), wq.view(np.int8)).tolist() == g["acc"]
    y = oracle.linear(oracle.INT8, xq, sx, wq, sw, _bf16(g["bias"]))
    assert workloads.bf16_bits_to_f32(y).tolist() == g["y"]
    # without bias: the same products, bias term absent
    y0 = oracle.linear(oracle.INT8, xq, sx, wq, sw, None)
    acc = np.array(g["acc"], np.float64)
    want = acc * np.array(g["x_scale"])[:, None] * g["w_scale"]
    assert np.array_equal(workloads.bf16_bits_to_f32(y0), workloads.bf16_bits_to_f32(_bf16(want)))


def test_linear_matches_numpy_f64_chain():
    # non-square shapes catch a transposed operand or swapped scale vector
    rng = np.random.default_rng(1)
    for qt in (oracle.INT8, oracle.FP8_E4M3):
        x = workloads.activations_bf16(rng, 24, 96, outliers=2)
        w = workloads.normal_bf16(rng, (40, 96), 0.02)
        b = workloads.normal_bf16(rng, (40,), 0.02)
        xq, sx = oracle.quant_act_rowwise(qt, x)
        wq, _, sw = oracle.quant_weight_tensorwise(qt, w)
        y = oracle.linear(qt, xq, sx, wq, sw, b)
        if qt == oracle.INT8:
            xd, wd = xq.view(np.int8).astype(np.float64), wq.view(np.int8).astype(np.float64)
        else:
            xd, wd = oracle.e4m3_to_f64(xq), oracle.e4m3_to_f64(wq)
        ref = (xd @ wd.T) * sx.astype(np.float64)[:, None] * np.float64(sw) \
            + workloads.bf16_bits_to_f32(b).astype(np.float64)[None, :]
        # float64 matmul sums in another order; compare after rounding to bf16
        # allowing the two sides to straddle a bf16 rounding boundary (1 ulp)
        got = workloads.bf16_bits_to_f32(y).astype(np.float64)
        assert (np.abs(got - ref) <= np.abs(ref) * 2**-8 + 1e-30).all()


def test_linear_error_bound_against_unquantized():
    # |y - x.w| <= sum_k (|x_k| sw/2 + |w_k| sx/2 + sx sw / 4) + half a bf16 ulp
    rng = np.random.default_rng(2)
    x = workloads.activations_bf16(rng, 16, 256, outliers=3)
    w = workloads.normal_bf16(rng, (32, 256), 0.02)
    xq, sx = oracle.quant_act_rowwise(oracle.INT8, x)
    wq, _, sw = oracle.quant_weight_tensorwise(oracle.INT8, w)
    y = workloads.bf16_bits_to_f32(oracle.linear(oracle.INT8, xq, sx, wq, sw)).astype(np.float64)
    xf = workloads.bf16_bits_to_f32(x).astype(np.float64)
    wf = workloads.bf16_bits_to_f32(w).astype(np.float64)
    exact = xf @ wf.T
    sxd, swd = sx.astype(np.float64)[:, None], np.float64(sw)
    bound = (np.abs(xf).sum(1)[:, None] * swd / 2 + np.abs(wf).sum(1)[None, :] * sxd / 2
             + 256 * sxd * swd / 4) + np.abs(exact) * 2**-8
    assert (np.abs(y - exact) <= bound).all()


def test_fp8_linear_exact_on_small_integer_codes():
    # With codes from {0, +-1, +-2, +-4} every partial sum is a small integer, so
    # the exact sum is the numpy integer product.
    rng = np.random.default_rng(3)
    vals = np.array([0, 1, -1, 2, -2, 4, -4], np.float32)
    xc = oracle.f32_to_e4m3(rng.choice(vals, (8, 256)))
    wc = oracle.f32_to_e4m3(rng.choice(vals, (12, 256)))
    sx = np.ones(8, np.float32)
    y = oracle.linear(oracle.FP8_E4M3, xc, sx, wc, np.float32(1.0))
    ref = oracle.e4m3_to_f64(xc) @ oracle.e4m3_to_f64(wc).T
    assert np.array_equal(workloads.bf16_bits_to_f32(y).astype(np.float64),
                          workloads.bf16_bits_to_f32(_bf16(ref)).astype(np.float64))


@pytest.mark.parametrize("qt", [oracle.INT8, oracle.FP8_E4M3])
def test_backward_dx_identity_and_numpy(qt):
    rng = np.random.default_rng(4)
    M, N, K = 16, 48, 40
    w = workloads.normal_bf16(rng, (N, K), 0.02)
    dy = workloads.normal_bf16(rng, (M, N), 1e-3)
    wq, wqt, sw = oracle.quant_weight_tensorwise(qt, w, transposed=True)
    dyq, sdy = oracle.quant_act_rowwise(qt, dy)
    dx = oracle.linear_backward_dx(qt, dyq, sdy, wq, sw)
    # identity: dX equals the forward linear applied to (dYq, Wq^T)
    assert np.array_equal(dx, oracle.linear(qt, dyq, sdy, wqt, sw))
    dec = (lambda c: c.view(np.int8).astype(np.float64)) if qt == oracle.INT8 else oracle.e4m3_to_f64
    ref = (dec(dyq) @ dec(wq)) * sdy.astype(np.float64)[:, None] * np.float64(sw)
    got = workloads.bf16_bits_to_f32(dx).astype(np.float64)
    assert (np.abs(got - ref) <= np.abs(ref) * 2**-8 + 1e-30).all()


def test_svdq_reduces_to_linear_when_low_rank_is_zero():
    rng = np.random.default_rng(5)
    M, K, N, r = 8, 64, 24, 4
    x = workloads.activations_bf16(rng, M, K, outliers=1)
    res = workloads.normal_bf16(rng, (N, K), 0.02)
    b = workloads.normal_bf16(rng, (N,), 0.02)
    rq, _, sr = oracle.quant_weight_tensorwise(oracle.INT8, res)
    l1 = np.zeros((r, K), np.uint16)
    l2 = workloads.normal_bf16(rng, (N, r), 0.1)
    y, xq, sx = oracle.svdq_linear(oracle.INT8, x, rq, sr, l1, l2, b)
    xq2, sx2 = oracle.quant_act_rowwise(oracle.INT8, x)
    assert np.array_equal(xq, xq2) and np.array_equal(sx, sx2)
    assert np.array_equal(y, oracle.linear(oracle.INT8, xq2, sx2, rq, sr, b))


def test_svdq_reduces_to_low_rank_chain_when_residual_is_zero():
    rng = np.random.default_rng(6)
    M, K, N, r = 8, 64, 24, 4
    x = workloads.activations_bf16(rng, M, K, outliers=1)
    rq = np.zeros((N, K), np.int8)
    l1 = workloads.normal_bf16(rng, (r, K), 0.1)
    l2 = workloads.normal_bf16(rng, (N, r), 0.1)
    b = workloads.normal_bf16(rng, (N,), 0.02)
    y, _, _ = oracle.svdq_linear(oracle.INT8, x, rq, np.float32(0.01), l1, l2, b)
    f = lambda a: workloads.bf16_bits_to_f32(a).astype(np.float64)
    ref = (f(x) @ f(l1).T) @ f(l2).T + f(b)[None, :]
    got = f(y)
    assert (np.abs(got - ref) <= np.abs(ref) * 2**-8 + 1e-30).all()


def test_svdq_brute_force_tiny():
    rng = np.random.default_rng(7)
    M, K, N, r = 3, 32, 5, 2
    x = workloads.activations_bf16(rng, M, K, outliers=1)
    res = workloads.normal_bf16(rng, (N, K), 0.02)
    rq, _, sr = oracle.quant_weight_tensorwise(oracle.INT8, res)
    l1 = workloads.normal_bf16(rng, (r, K), 0.1)
    l2 = workloads.normal_bf16(rng, (N, r), 0.1)
    y, xq, sx = oracle.svdq_linear(oracle.INT8, x, rq, sr, l1, l2, None)
    f = lambda a: workloads.bf16_bits_to_f32(a).astype(np.float64)
    xf, l1f, l2f = f(x), f(l1), f(l2)
    for m in range(M):
        for n in range(N):
            acc = sum(int(xq.view(np.int8)[m, k]) * int(rq.view(np.int8)[n, k]) for k in range(K))
            low = sum(sum(xf[m, k] * l1f[j, k] for k in range(K)) * l2f[n, j] for j in range(r))
            v = acc * float(sx[m]) * float(sr) + low
            assert abs(f(y[m:m + 1, n:n + 1])[0, 0] - v) <= abs(v) * 2**-8


def test_svdq_u_needs_more_than_one_bf16():
    """Why U = X . L1^T reaches the bf16 MFMA as two halves: on 16 rows of the
    SVDQuant workload (X with outlier channels, L1 and L2 N(0, 0.1), r = 32),
    the linear with U rounded to one bf16 puts outputs outside the bf16 bound
    |d| <= 2^-7 |ref| + 1e-3 against the oracle (U unrounded), while
    hi = bf16(U), lo = bf16(U - hi) keeps every output inside it.  The
    residual part, the bias and the final rounding are the oracle's own."""
    d = workloads.svdq()
    x = d["x"][:16]
    rq, _, sr = oracle.quant_weight_tensorwise(oracle.INT8, d["r"])
    y_ref, xq, sx = oracle.svdq_linear(oracle.INT8, x, rq, sr, d["l1"], d["l2"], d["bias"])
    acc = oracle.gemm_i32(xq.view(np.int8), np.asarray(rq).view(np.int8)).astype(np.float64)
    base = acc * sx.astype(np.float64)[:, None] * float(np.float32(sr)) + bf16_to_f64(d["bias"])[None, :]
    u = bf16_to_f64(x) @ bf16_to_f64(d["l1"]).T
    l2 = bf16_to_f64(d["l2"])
    ref = bf16_to_f64(y_ref)

    def outside(u_used):
        y = bf16_to_f64(oracle.f64_to_bf16(base + u_used @ l2.T))
        return int((np.abs(y - ref) > 2.0 ** -7 * np.abs(ref) + 1e-3).sum())

    hi = bf16_to_f64(oracle.f64_to_bf16(u))
    lo = bf16_to_f64(oracle.f64_to_bf16(u - hi))
    assert outside(u) == 0          # the recomposition matches the oracle
    assert outside(hi) > 1000       # one bf16: 18882 of 196608 outputs on this data
    assert outside(hi + lo) == 0

