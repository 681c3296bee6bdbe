"""svdq_linear_noalloc (u in the library's fixed per-GPU scratch) against
svdq_linear (u in a caller workspace) through the C ABI: identical codes,
scales and outputs on consecutive calls, the later ones smaller and on the
other code paths, so that a call finding the previous call's u in the
scratch would show it.  Runs alone in a fresh process or after the other
GPU tests."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import assert_bf16_close, assert_equal, bf16_dev, bf16_host, bytes_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_quantized_linear_quant_amd as w8
    return w8


def _inputs(rng, M, K, N, r, qt, w8):
    x = workloads.activations_bf16(rng, M, K, outliers=2)
    l1 = workloads.normal_bf16(rng, (r, K), 0.1)
    l2 = workloads.normal_bf16(rng, (N, r), 0.1)
    res = workloads.normal_bf16(rng, (N, K), 0.02)
    b = workloads.normal_bf16(rng, (N,), 0.02)
    rq, _, sr = w8.w8a8_quant_weight_tensorwise(bf16_dev(res), qtype=qt)
    return x, bf16_dev(x), rq, sr, bf16_dev(l1), bf16_dev(l2), bf16_dev(b), (l1, l2, res, b)


# (M, K, N, r, qtype): fused act-quant + down path with LDS-staged factors,
# then smaller calls on the generic-rank and two-kernel (K > 4096) paths
CALLS = [(1000, 1024, 520, 32, oracle.INT8), (37, 96, 130, 5, oracle.INT8), (20, 4160, 64, 24, oracle.FP8_E4M3),
         (3, 64, 48, 16, oracle.FP8_E4M3)]


def test_noalloc_matches_workspace_entry_point(w8):
    rng = np.random.default_rng(2026)
    for i, (M, K, N, r, qt) in enumerate(CALLS):
        print(f"[no-alloc] call {i}: M={M} K={K} N={N} r={r} qt={qt}", flush=True)
        x, xd, rq, sr, l1d, l2d, bd, host = _inputs(rng, M, K, N, r, qt, w8)
        y0, xq0, sx0 = w8.svdq_linear(xd, rq, sr, l1d, l2d, bd)
        y1 = torch.empty_like(y0)
        xq1 = torch.empty_like(xq0)
        sx1 = torch.empty_like(sx0)
        w8.svdq_linear_noalloc(xd, rq, sr, l1d, l2d, bd, out=y1, xq_out=xq1, x_scale_out=sx1)
        torch.cuda.synchronize()
        assert_equal(bytes_host(xq1), bytes_host(xq0), f"call {i} codes")
        assert_equal(sx1.cpu().numpy().view(np.uint32), sx0.cpu().numpy().view(np.uint32), f"call {i} scales")
        # the same kernels on the same inputs: the bf16 outputs agree bit for
        # bit, which is within the bf16 bound of the parity tests
        assert_bf16_close(bf16_host(y1), bf16_host(y0), f"call {i} y")
        assert_equal(bf16_host(y1), bf16_host(y0), f"call {i} y bits")
    # the last call against the oracle as well
    l1, l2, res, b = host
    orq, _, osr = oracle.quant_weight_tensorwise(qt, res)
    ref_y, ref_xq, ref_sx = oracle.svdq_linear(qt, x, orq, osr, l1, l2, b)
    assert_equal(bytes_host(xq1), ref_xq, "oracle codes")
    assert_bf16_close(bf16_host(y1), ref_y, "oracle y")


def test_noalloc_rejects_beyond_its_scratch(w8):
    M = w8.SVDQ_NOALLOC_SCRATCH_BYTES // (2 * 2 * 32) + 1
    K, N, r = 64, 64, 32
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    rq = torch.zeros((N, K), dtype=torch.int8, device="cuda")
    sr = torch.ones(1, dtype=torch.float32, device="cuda")
    l1 = torch.zeros((r, K), dtype=torch.bfloat16, device="cuda")
    l2 = torch.zeros((N, r), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(w8.W8A8Error, match="SCRATCH_LIMIT"):
        w8.svdq_linear_noalloc(x, rq, sr, l1, l2)
    # one row fewer fits exactly
    y, _, _ = w8.svdq_linear_noalloc(x[: M - 1], rq, sr, l1, l2)
    torch.cuda.synchronize()
    assert not bf16_host(y).any()
