"""GPU parity: every C-ABI entry point against the CPU oracle on the same seeded
inputs.  Codes, scales, int32 accumulators and Q8_0 bytes must match bit for
bit; bf16 outputs within |d| <= 2^-7 |ref| + 1e-3.  Full-size workloads are
compared on sampled rows (and, for e4m3 products, sampled columns) that the
oracle computes one by one, taken at every tile boundary plus random rows."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import (assert_bf16_close, assert_equal, assert_frobenius, bf16_dev, bf16_host, bytes_host, codes_dev,
                     f32_dev, sample_rows)

pytestmark = pytest.mark.gpu

W8 = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global W8
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_quantized_linear_quant_amd as w8
    W8 = w8
    yield


def _say(msg):
    print(f"[parity] {msg}", flush=True)


INT8, FP8 = oracle.INT8, oracle.FP8_E4M3


# ------------------------------------------------------------ act quant
def _act_quant_check(x_bits, qt, ldq=None, rows=None, what=""):
    M, K = x_bits.shape
    if K % 8:
        # rows must start on 16-byte boundaries: a [:, :K] view of padded rows
        xp = np.zeros((M, K + (-K) % 8), np.uint16)
        xp[:, :K] = x_bits
        xd = bf16_dev(xp)[:, :K]
    else:
        xd = bf16_dev(x_bits)
    xq, sx = W8.w8a8_quant_act_rowwise(xd, qtype=qt, ldq=ldq)
    torch.cuda.synchronize()
    got_q, got_s = bytes_host(xq), sx.cpu().numpy()
    sel = np.arange(M) if rows is None else rows
    ref_q, ref_s = oracle.quant_act_rowwise(qt, x_bits[sel], ldq=got_q.shape[1])
    assert_equal(got_s[sel].view(np.uint32), ref_s.view(np.uint32), what + " scales")
    assert_equal(got_q[sel], ref_q, what + " codes")


@pytest.mark.parametrize("qt", [INT8, FP8])
def test_act_quant_tiny(qt):
    _say(f"act_quant tiny qt={qt}")
    _act_quant_check(workloads.tiny()["x"], qt, what="tiny")


def _edge_rows(K):
    rows = np.zeros((12, K), np.float32)
    rows[1, :8] = [127, 0.5, 1.5, 2.5, -2.5, -0.5, 126.5, -127]           # int8 ties
    rows[2, :8] = [448, 1.0625, 1.1875, -1.0625, 2**-10, 1.5 * 2**-9, -0.0, 0.0]  # e4m3 ties
    rows[3, 5] = -3e38                                                    # huge single value
    rows[4, :] = 1e-38                                                    # bf16 subnormal-ish
    rows[5, 7] = 9e-11                                                    # below the scale floor
    rows[6, :] = -1.0                                                     # all equal
    rows[7, ::3] = 7.0                                                    # ties of the absmax
    rows[7, 1::3] = -7.0
    rng = np.random.default_rng(3)
    rows[8] = rng.standard_normal(K) * 1e3
    rows[9] = rng.standard_normal(K)
    rows[9, rng.choice(K, 3, replace=False)] *= 50
    rows[10] = -0.0
    rows[11] = rng.uniform(-1, 1, K) * 2.0 ** rng.integers(-30, 30, K)
    return workloads.f32_to_bf16_bits(rows)


@pytest.mark.parametrize("qt", [INT8, FP8])
@pytest.mark.parametrize("K,ldq", [(64, None), (37, 48), (200, 256), (3072, None), (12288, None), (20000, None)])
def test_act_quant_edges(qt, K, ldq):
    _say(f"act_quant edges qt={qt} K={K} ldq={ldq}")
    _act_quant_check(_edge_rows(K), qt, ldq=ldq, what=f"edges K={K}")


@pytest.mark.parametrize("qt,qmax", [(INT8, 127.0), (FP8, 448.0)])
def test_act_quant_every_bf16_value(qt, qmax):
    # one row per scale 2^e: [qmax * 2^e, every bf16 value v with |v| <= qmax * 2^e]
    _say(f"act_quant every bf16 value qt={qt}")
    allv = workloads.bf16_bits_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    # Powers of two give exact reciprocals; the absmax values qmax (1 + k/128) 2^e
    # (rounded to bf16) give scales whose reciprocal is inexact, where the
    # kernels' corrected quotient has to reproduce the IEEE division.
    rows = []
    lims = [qmax * 2.0 ** e for e in (-20, -3, 0, 5)]
    lims += [qmax * (1 + k / 128) * 2.0 ** e for k, e in ((1, 0), (37, -3), (85, 2), (127, -9), (51, 7))]
    for lim in lims:
        lim = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(np.array([lim], np.float32)))[0]
        v = allv[np.isfinite(allv) & (np.abs(allv) <= lim)]
        rows.append(np.concatenate([[lim], v]))
    K = max(len(r) for r in rows)
    K += (-K) % 8
    x = np.zeros((len(rows), K), np.float32)
    for i, r in enumerate(rows):
        x[i, :len(r)] = r
    _act_quant_check(workloads.f32_to_bf16_bits(x), qt, what="all bf16")


def test_act_quant_ragged_rows():
    _say("act_quant ragged M")
    for M in (1, 3, 5, 130):
        _act_quant_check(workloads.random_rows(M, M, 96), INT8, what=f"M={M}")


def test_act_quant_dit_full_int8():
    _say("act_quant dit X [4608,3072] int8")
    _act_quant_check(workloads.dit()["x"], INT8, what="dit")


def test_act_quant_fp8_step():
    _say("act_quant fp8 step X and dY (sampled rows)")
    d = workloads.fp8_step()
    _act_quant_check(d["x"], FP8, rows=sample_rows(d["x"].shape[0], 256), what="fp8 X")
    _act_quant_check(d["dy"], FP8, rows=sample_rows(d["dy"].shape[0], 96, seed=1), what="fp8 dY")


# ------------------------------------------------------------ weight quant
@pytest.mark.parametrize("qt", [INT8, FP8])
@pytest.mark.parametrize("N,K", [(256, 256), (48, 40), (3072, 3072)])
def test_weight_quant(qt, N, K):
    _say(f"weight_quant qt={qt} N={N} K={K}")
    w = workloads.normal_bf16(np.random.default_rng(N + K), (N, K), 0.02)
    wq, wqt, s = W8.w8a8_quant_weight_tensorwise(bf16_dev(w), qtype=qt, transposed=(N % 16 == 0))
    torch.cuda.synchronize()
    ref_q, ref_qt, ref_s = oracle.quant_weight_tensorwise(qt, w, transposed=True)
    assert_equal(s.cpu().numpy().view(np.uint32), np.array([ref_s]).view(np.uint32), "scale")
    assert_equal(bytes_host(wq), ref_q, "codes")
    if wqt is not None:
        assert_equal(bytes_host(wqt), ref_qt, "transposed codes")


def test_weight_quant_zero_tensor():
    w = np.zeros((32, 64), np.uint16)
    wq, _, s = W8.w8a8_quant_weight_tensorwise(bf16_dev(w))
    torch.cuda.synchronize()
    assert s.cpu().numpy().view(np.uint32)[0] == 0x2EDBE6FF
    assert not bytes_host(wq).any()


# ------------------------------------------------------------ int8 product
@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (64, 256, 256), (33, 257, 48), (300, 520, 144), (256, 256, 4096),
                                   (513, 17, 272), (7, 1000, 32)])
def test_gemm_i32_exact(M, N, K):
    _say(f"gemm_i32 M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a = rng.integers(-128, 128, (M, K), dtype=np.int8)
    b = rng.integers(-128, 128, (N, K), dtype=np.int8)
    acc = W8.w8a8_gemm_i32(codes_dev(a, False), codes_dev(b, False))
    torch.cuda.synchronize()
    assert_equal(acc.cpu().numpy(), oracle.gemm_i32(a, b), "int32 accumulators")


def test_gemm_i32_extremes():
    K = 4096
    a = np.full((3, K), -128, np.int8)
    a[1] = 127
    a[2, ::2] = 127
    b = np.full((5, K), -128, np.int8)
    b[3] = 127
    acc = W8.w8a8_gemm_i32(codes_dev(a, False), codes_dev(b, False))
    torch.cuda.synchronize()
    assert_equal(acc.cpu().numpy(), oracle.gemm_i32(a, b), "extremes")


def test_gemm_i32_longest_exact_k():
    """K = 131072 with codes at +-127 (the quantizers' range): |acc| reaches
    127^2 K = 2,114,060,288, just below 2^31, and must stay exact."""
    K = 131072
    a = np.full((3, K), 127, np.int8)
    a[1] = -127
    a[2, 1::2] = -127
    b = np.full((2, K), 127, np.int8)
    b[1, ::3] = -127
    acc = W8.w8a8_gemm_i32(codes_dev(a, False), codes_dev(b, False))
    torch.cuda.synchronize()
    ref = oracle.gemm_i32(a, b)
    assert abs(int(ref[0, 0])) == 127 * 127 * K
    assert_equal(acc.cpu().numpy(), ref, "int32 accumulators at the longest exact K")


def test_gemm_i32_max_k():
    """K at its limit (2^22, 65,536 stages through one tile) with ragged M, N;
    random codes keep |acc| far below 2^31, so the sum is exact."""
    _say("gemm_i32 M3 N5 K=2^22")
    rng = np.random.default_rng(17)
    M, N, K = 3, 5, 1 << 22
    a = rng.integers(-128, 128, (M, K), dtype=np.int8)
    b = rng.integers(-128, 128, (N, K), dtype=np.int8)
    acc = W8.w8a8_gemm_i32(codes_dev(a, False), codes_dev(b, False))
    torch.cuda.synchronize()
    assert_equal(acc.cpu().numpy(), oracle.gemm_i32(a, b), "accumulators at K = 2^22")


def test_act_quant_longest_rows():
    """Rows of 2^22 + 16 values (the two-pass kernel), both code types."""
    K = (1 << 22) + 16
    rng = np.random.default_rng(19)
    x = workloads.f32_to_bf16_bits((rng.standard_normal((2, K)) * np.array([[1.0], [300.0]])).astype(np.float32))
    for qt in (INT8, FP8):
        _say(f"act_quant K={K} qt={qt}")
        _act_quant_check(x, qt, what=f"K={K}")


def test_gemm_i32_full_size_sampled():
    _say("gemm_i32 M4096 N12288 K3072 sampled rows")
    rng = np.random.default_rng(11)
    M, N, K = 4096, 12288, 3072
    a = rng.integers(-128, 128, (M, K), dtype=np.int8)
    b = rng.integers(-128, 128, (N, K), dtype=np.int8)
    acc = W8.w8a8_gemm_i32(codes_dev(a, False), codes_dev(b, False))
    torch.cuda.synchronize()
    rows = sample_rows(M, 16)
    got = acc.cpu().numpy()[rows]
    assert_equal(got, oracle.gemm_i32(a[rows], b), "sampled accumulators")


# ------------------------------------------------------------ linear
def _gpu_linear(x, w, bias, qt):
    xq, sx = W8.w8a8_quant_act_rowwise(bf16_dev(x), qtype=qt)
    wq, _, sw = W8.w8a8_quant_weight_tensorwise(bf16_dev(w), qtype=qt)
    y = W8.w8a8_linear(xq, sx, wq, sw, None if bias is None else bf16_dev(bias))
    torch.cuda.synchronize()
    return bf16_host(y)


@pytest.mark.parametrize("qt", [INT8, FP8])
@pytest.mark.parametrize("with_bias", [True, False])
def test_linear_tiny(qt, with_bias):
    _say(f"linear tiny qt={qt} bias={with_bias}")
    d = workloads.tiny()
    bias = d["bias"] if with_bias else None
    got = _gpu_linear(d["x"], d["w"], bias, qt)
    xq, sx = oracle.quant_act_rowwise(qt, d["x"])
    wq, _, sw = oracle.quant_weight_tensorwise(qt, d["w"])
    ref = oracle.linear(qt, xq, sx, wq, sw, bias)
    assert_bf16_close(got, ref, "tiny linear")
    if qt == FP8:
        assert_frobenius(got, ref, "tiny e4m3 linear")


@pytest.mark.parametrize("M,N,K", [(1, 24, 16), (5, 200, 48), (257, 300, 272), (130, 64, 1040)])
def test_linear_ragged(M, N, K):
    _say(f"linear ragged M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    x = workloads.activations_bf16(rng, M, K, outliers=2)
    w = workloads.normal_bf16(rng, (N, K), 0.02)
    b = workloads.normal_bf16(rng, (N,), 0.02)
    for qt in (INT8, FP8):
        got = _gpu_linear(x, w, b, qt)
        xq, sx = oracle.quant_act_rowwise(qt, x)
        wq, _, sw = oracle.quant_weight_tensorwise(qt, w)
        ref = oracle.linear(qt, xq, sx, wq, sw, b)
        assert_bf16_close(got, ref, f"ragged qt={qt}")
        if qt == FP8:
            assert_frobenius(got, ref, "ragged e4m3 linear")


@pytest.mark.parametrize("which", ["w1", "w2"])
def test_linear_dit_sampled(which):
    _say(f"linear dit {which} sampled rows")
    d = workloads.dit()
    x, w = d["x"], d[which]
    b = d["b1"] if which == "w1" else d["b2"]
    got = _gpu_linear(x, w, b, INT8)
    rows = sample_rows(x.shape[0], 8)
    xq, sx = oracle.quant_act_rowwise(INT8, x[rows])
    wq, _, sw = oracle.quant_weight_tensorwise(INT8, w)
    assert_bf16_close(got[rows], oracle.linear(INT8, xq, sx, wq, sw, b), f"dit {which}")


def test_linear_headline_full_sampled():
    """The timed step itself: X [4096, 3072] with outlier channels, W [12288,
    3072], bias, int8 -- the inputs and the launches the benchmark times
    (act-quant, then the product with the bf16 epilogue), on sampled rows:
    codes and row scales bit for bit, Y within the bf16 bound."""
    _say("linear headline M4096 K3072 N12288 int8 sampled rows")
    d = workloads.svdq()
    x, w, b = d["x"], d["r"], d["bias"]
    xq, sx = W8.w8a8_quant_act_rowwise(bf16_dev(x))
    wq, _, sw = W8.w8a8_quant_weight_tensorwise(bf16_dev(w))
    y = W8.w8a8_linear(xq, sx, wq, sw, bf16_dev(b))
    torch.cuda.synchronize()
    rows = sample_rows(x.shape[0], 8)
    rxq, rsx = oracle.quant_act_rowwise(INT8, x[rows])
    rwq, _, rsw = oracle.quant_weight_tensorwise(INT8, w)
    assert_equal(sx.cpu().numpy()[rows].view(np.uint32), rsx.view(np.uint32), "row scales")
    assert_equal(bytes_host(xq)[rows], rxq, "activation codes")
    assert_equal(sw.cpu().numpy().reshape(-1).view(np.uint32),
                 np.atleast_1d(np.float32(rsw)).view(np.uint32), "weight scale")
    assert_equal(bytes_host(wq), rwq, "weight codes [12288, 3072]")
    assert_bf16_close(bf16_host(y)[rows], oracle.linear(INT8, rxq, rsx, rwq, rsw, b), "headline Y")


def test_fp8_exact_on_small_integer_codes():
    # codes of {0, +-1, +-2, +-4} with unit scales: every f32 partial sum is
    # exact, so the bf16 output must match bit for bit.
    _say("fp8 product exact on small integer codes")
    rng = np.random.default_rng(5)
    vals = np.array([0, 1, -1, 2, -2, 4, -4], np.float32)
    M, N, K = 300, 260, 1024
    xc = oracle.f32_to_e4m3(rng.choice(vals, (M, K)))
    wc = oracle.f32_to_e4m3(rng.choice(vals, (N, K)))
    ones_m = np.ones(M, np.float32)
    y = W8.w8a8_linear(codes_dev(xc, True), f32_dev(ones_m), codes_dev(wc, True), f32_dev([1.0]))
    torch.cuda.synchronize()
    ref = oracle.linear(FP8, xc, ones_m, wc, np.float32(1.0))
    assert_equal(bf16_host(y), ref, "exact fp8 products")


def test_fp8_step_forward_and_backward_sampled():
    _say("fp8 train step: forward and dX (sampled rows and columns)")
    d = workloads.fp8_step()
    x, w, dy = d["x"], d["w"], d["dy"]
    M, K = x.shape
    N = w.shape[0]
    wq, wqt, sw = W8.w8a8_quant_weight_tensorwise(bf16_dev(w), qtype=FP8, transposed=True)
    xq, sx = W8.w8a8_quant_act_rowwise(bf16_dev(x), qtype=FP8)
    y = W8.w8a8_linear(xq, sx, wq, sw)
    dyq, sdy = W8.w8a8_quant_act_rowwise(bf16_dev(dy), qtype=FP8)
    dx = W8.w8a8_linear_backward_dx(dyq, sdy, wqt, sw)
    torch.cuda.synchronize()
    rows = sample_rows(M, 4)
    cols = np.unique(np.concatenate([np.arange(0, N, 97), [N - 1]]))
    kcols = np.unique(np.concatenate([np.arange(0, K, 29), [K - 1]]))
    owq, owqt, osw = oracle.quant_weight_tensorwise(FP8, w, transposed=True)
    assert_equal(sw.cpu().numpy().reshape(-1).view(np.uint32), np.atleast_1d(np.float32(osw)).view(np.uint32),
                 "e4m3 weight scale")
    assert_equal(bytes_host(wq), owq, "e4m3 weight codes [12288, 3072]")
    assert_equal(bytes_host(wqt), owqt, "e4m3 transposed weight codes [3072, 12288]")
    oxq, osx = oracle.quant_act_rowwise(FP8, x[rows])
    assert_equal(bytes_host(xq)[rows], oxq, "e4m3 activation codes")
    ref_y = oracle.linear(FP8, oxq, osx, owq[cols], osw)
    got_y = bf16_host(y)[rows][:, cols]
    assert_bf16_close(got_y, ref_y, "fp8 forward")
    assert_frobenius(got_y, ref_y, "fp8 forward")
    odyq, osdy = oracle.quant_act_rowwise(FP8, dy[rows])
    assert_equal(bytes_host(dyq)[rows], odyq, "e4m3 dY codes")
    ref_dx = oracle.linear_backward_dx(FP8, odyq, osdy, np.ascontiguousarray(owq[:, kcols]), osw)
    got_dx = bf16_host(dx)[rows][:, kcols]
    assert_bf16_close(got_dx, ref_dx, "fp8 dX")
    assert_frobenius(got_dx, ref_dx, "fp8 dX")


@pytest.mark.parametrize("qt", [INT8, FP8])
@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (5, 48, 200), (257, 272, 296), (33, 1040, 64)])
def test_backward_dx_ragged(qt, M, N, K):
    """dX = dY . W through the transposed codes, ragged in every dimension
    (dY [M, N] row-quantized, N the reduction length)."""
    _say(f"backward dX qt={qt} M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 5 + N + K)
    w = workloads.normal_bf16(rng, (N, K), 0.02)
    dy = workloads.normal_bf16(rng, (M, N), 1e-3)
    wq, wqt, sw = W8.w8a8_quant_weight_tensorwise(bf16_dev(w), qtype=qt, transposed=True)
    dyq, sdy = W8.w8a8_quant_act_rowwise(bf16_dev(dy), qtype=qt)
    dx = W8.w8a8_linear_backward_dx(dyq, sdy, wqt, sw)
    torch.cuda.synchronize()
    owq, owqt, osw = oracle.quant_weight_tensorwise(qt, w, transposed=True)
    assert_equal(bytes_host(wqt), owqt, "transposed codes")
    odyq, osdy = oracle.quant_act_rowwise(qt, dy)
    ref = oracle.linear_backward_dx(qt, odyq, osdy, owq, osw)
    assert_bf16_close(bf16_host(dx), ref, f"dX qt={qt}")
    if qt == FP8:
        assert_frobenius(bf16_host(dx), ref, "e4m3 dX ragged")


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("qt", [INT8, FP8])
@pytest.mark.parametrize("M,N,K", [(4349, 4096, 512), (4349, 4100, 80)])
def test_linear_192_wide_tiles(qt, M, N, K):
    """Shapes whose 256-wide tiles would leave a partial second round, so the
    product takes 192-wide tiles (on a 256-CU device): the whole output
    against the oracle, M ragged, N a multiple of 8 (unchecked epilogue of
    interior tiles) or not (checked epilogue), K a multiple of the stage ring
    or with a tail."""
    if _cus() != 256:
        pytest.skip("tile-width choice assumes 256 CUs")
    assert W8.probe_gemm_tile_n(M, N) == 192
    _say(f"linear 192-wide tiles qt={qt} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 3 * N + K + qt)
    x = workloads.activations_bf16(rng, M, K, outliers=4)
    w = workloads.normal_bf16(rng, (N, K), 0.02)
    b = workloads.normal_bf16(rng, (N,), 0.02)
    got = _gpu_linear(x, w, b, qt)
    xq, sx = oracle.quant_act_rowwise(qt, x)
    wq, _, sw = oracle.quant_weight_tensorwise(qt, w)
    ref = oracle.linear(qt, xq, sx, wq, sw, b)
    assert_bf16_close(got, ref, f"192-wide qt={qt}")
    if qt == FP8:
        assert_frobenius(got, ref, "192-wide e4m3 linear")


def test_tile_width_choice():
    """256-wide tiles wherever they fill whole rounds or a single round; 192
    for the dX product of the training step (M8192, N3072: 1.5 rounds of
    256-wide tiles)."""
    if _cus() != 256:
        pytest.skip("tile-width choice assumes 256 CUs")
    assert W8.probe_gemm_tile_n(8192, 3072) == 192     # dX [8192, 3072]
    assert W8.probe_gemm_tile_n(4096, 12288) == 256    # 768 tiles, 3 rounds
    assert W8.probe_gemm_tile_n(8192, 12288) == 256    # 1536 tiles, 6 rounds
    assert W8.probe_gemm_tile_n(4608, 3072) == 256     # 216 tiles, one round
    assert W8.probe_gemm_tile_n(4608, 12288) == 256


def test_int8_step_backward_sampled():
    _say("int8 train step dX at M=8192 N=12288 K=3072 (sampled rows and columns)")
    d = workloads.fp8_step()
    w, dy = d["w"], d["dy"]
    M, N = dy.shape
    K = w.shape[1]
    wq, wqt, sw = W8.w8a8_quant_weight_tensorwise(bf16_dev(w), qtype=INT8, transposed=True)
    dyq, sdy = W8.w8a8_quant_act_rowwise(bf16_dev(dy), qtype=INT8)
    dx = W8.w8a8_linear_backward_dx(dyq, sdy, wqt, sw)
    torch.cuda.synchronize()
    rows = sample_rows(M, 4)
    kcols = np.unique(np.concatenate([np.arange(0, K, 29), [K - 1]]))
    owq, owqt, osw = oracle.quant_weight_tensorwise(INT8, w, transposed=True)
    assert_equal(bytes_host(wq), owq, "int8 weight codes [12288, 3072]")
    assert_equal(bytes_host(wqt), owqt, "int8 transposed weight codes [3072, 12288]")
    odyq, osdy = oracle.quant_act_rowwise(INT8, dy[rows])
    ref_dx = oracle.linear_backward_dx(INT8, odyq, osdy, np.ascontiguousarray(owq[:, kcols]), osw)
    assert_bf16_close(bf16_host(dx)[rows][:, kcols], ref_dx, "int8 dX")


# ------------------------------------------------------------ SVDQuant
@pytest.mark.parametrize("qt", [INT8, FP8])
# K > 4096 takes the two-kernel act-quant + down path; r = 24 rounds up to 32
# but reads the factors from global memory in the epilogue
@pytest.mark.parametrize("M,K,N,r", [(64, 256, 256, 32), (37, 96, 130, 5), (130, 512, 520, 16), (16, 64, 48, 64),
                                     (40, 4160, 300, 32), (20, 8192, 64, 24), (33, 1024, 260, 24),
                                     # the fused kernel's largest K (every chunk and step of a wave used), its
                                     # smallest (half a 32-wide step), and a K with a partial last step
                                     (24, 4096, 200, 32), (17, 4096, 64, 16), (5, 16, 24, 16), (19, 48, 40, 32)])
def test_svdq_small(qt, M, K, N, r):
    _say(f"svdq small qt={qt} M={M} K={K} N={N} r={r}")
    rng = np.random.default_rng(M + K + N + r)
    x = workloads.activations_bf16(rng, M, K, outliers=2)
    l1 = workloads.normal_bf16(rng, (r, K), 0.1)
    l2 = workloads.normal_bf16(rng, (N, r), 0.1)
    res = workloads.normal_bf16(rng, (N, K), 0.02)
    b = workloads.normal_bf16(rng, (N,), 0.02)
    rq, _, sr = W8.w8a8_quant_weight_tensorwise(bf16_dev(res), qtype=qt)
    y, xq, sx = W8.svdq_linear(bf16_dev(x), rq, sr, bf16_dev(l1), bf16_dev(l2), bf16_dev(b))
    torch.cuda.synchronize()
    orq, _, osr = oracle.quant_weight_tensorwise(qt, res)
    ref_y, ref_xq, ref_sx = oracle.svdq_linear(qt, x, orq, osr, l1, l2, b)
    assert_equal(bytes_host(xq), ref_xq, "svdq codes")
    assert_equal(sx.cpu().numpy().view(np.uint32), ref_sx.view(np.uint32), "svdq scales")
    assert_bf16_close(bf16_host(y), ref_y, "svdq y")
    if qt == FP8:
        assert_frobenius(bf16_host(y), ref_y, "svdq e4m3 y")


@pytest.mark.parametrize("qt", [INT8, FP8])
@pytest.mark.parametrize("K,r", [(256, 32), (1024, 16)])
def test_svdq_multi_tile(qt, K, r):
    """More 256x256 tiles (17 x 17, ragged) than CUs, so workgroups run several
    tiles back to back (e4m3: the low-rank operands of one tile's epilogue
    share the stage ring with the next tile's loads; int8: u arrives in the
    registers of the tile's last k-step and l2 in the staging areas while the
    next tile's stages load); K = 256 gives single-group tiles."""
    M, N = 4352 - 7, 4160 + 3
    _say(f"svdq multi-tile qt={qt} M={M} K={K} N={N} r={r}")
    rng = np.random.default_rng(K + r)
    x = workloads.activations_bf16(rng, M, K, outliers=2)
    l1 = workloads.normal_bf16(rng, (r, K), 0.1)
    l2 = workloads.normal_bf16(rng, (N, r), 0.1)
    res = workloads.normal_bf16(rng, (N, K), 0.02)
    b = workloads.normal_bf16(rng, (N,), 0.02)
    rq, _, sr = W8.w8a8_quant_weight_tensorwise(bf16_dev(res), qtype=qt)
    y, xq, sx = W8.svdq_linear(bf16_dev(x), rq, sr, bf16_dev(l1), bf16_dev(l2), bf16_dev(b))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(M, 6), [255, 256, M - 1]]))
    orq, _, osr = oracle.quant_weight_tensorwise(qt, res)
    ref_y, _, _ = oracle.svdq_linear(qt, x[rows], orq, osr, l1, l2, b)
    assert_bf16_close(bf16_host(y)[rows], ref_y, "svdq y, several tiles per workgroup")
    if qt == FP8:
        assert_frobenius(bf16_host(y)[rows], ref_y, "svdq e4m3 y, several tiles per workgroup")


def test_svdq_full_sampled():
    _say("svdq M4096 K3072 N12288 r32 sampled rows")
    d = workloads.svdq()
    x, l1, l2, res, b = d["x"], d["l1"], d["l2"], d["r"], d["bias"]
    rq, _, sr = W8.w8a8_quant_weight_tensorwise(bf16_dev(res), qtype=INT8)
    y, xq, sx = W8.svdq_linear(bf16_dev(x), rq, sr, bf16_dev(l1), bf16_dev(l2), None)
    torch.cuda.synchronize()
    rows = sample_rows(x.shape[0], 4)
    orq, _, osr = oracle.quant_weight_tensorwise(INT8, res)
    ref_y, ref_xq, ref_sx = oracle.svdq_linear(INT8, x[rows], orq, osr, l1, l2, None)
    assert_equal(bytes_host(xq)[rows], ref_xq, "svdq codes")
    assert_bf16_close(bf16_host(y)[rows], ref_y, "svdq y")


# ------------------------------------------------------------ Q8_0
@pytest.mark.parametrize("n", [1, 5, 31, 32, 33, 37, 255, 256, 257, 1000, 8191, 8192, 8193, 100_003])
def test_q8_0_small(n):
    rng = np.random.default_rng(n)
    v = (rng.standard_normal(n) * 10.0 ** rng.integers(-8, 4, n)).astype(np.float32)
    v[: min(n, 40)] = 0.0                      # a zero block (and a partial one when n < 40)
    if n > 80:
        v[64:96] = np.float32(3e-6) * rng.standard_normal(32).astype(np.float32)  # f16-subnormal scale
    blob = W8.q8_0_quantize(f32_dev(v))
    torch.cuda.synchronize()
    ref = oracle.q8_0_quantize(v)
    assert_equal(bytes_host(blob), ref, f"q8_0 bytes n={n}")
    y = W8.q8_0_dequantize(torch.from_numpy(ref).cuda(), n)
    torch.cuda.synchronize()
    assert_equal(y.cpu().numpy().view(np.uint32), oracle.q8_0_dequantize(ref, n).view(np.uint32), "dequant")


def test_q8_0_exact_ties():
    """Blocks whose quotients value / scale fall exactly half-way between
    integers, with scales 1, 3 and 2^-3 (3 has an inexact reciprocal): the
    kernel's quotient must round like the IEEE division before the RNE."""
    rng = np.random.default_rng(5)
    halves = (rng.integers(-127, 127, (30, 32)) + 0.5).astype(np.float64)
    halves[:, 0] = 127.0                        # the block absmax: scale = c exactly
    halves[:, 1] = -126.5
    blocks = [halves[i] * c for i, c in enumerate([1.0, 3.0, 0.125] * 10)]
    v = np.concatenate(blocks).astype(np.float32)
    assert np.array_equal(v.astype(np.float64), np.concatenate(blocks))   # exact in f32
    blob = W8.q8_0_quantize(f32_dev(v))
    torch.cuda.synchronize()
    assert_equal(bytes_host(blob), oracle.q8_0_quantize(v), "q8_0 bytes on ties")


def test_q8_0_f32_scale_block():
    """The golden block whose codes tell the page's reading (codes from the f32
    scale, quotient rounded to f32) from the f16-scale and unrounded-quotient
    readings, repeated at power-of-two magnitudes (the same codes)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "q8_0_f32_scale_block.json")) as f:
        g = json.load(f)
    base = np.zeros(32, np.float64)
    for i, (num, den) in enumerate(g["values_num_den"]):
        base[i] = num / den
    v = np.concatenate([base * 2.0 ** e for e in (0, -7, 5, -20, 12)] + [base[:7]]).astype(np.float32)
    blob = W8.q8_0_quantize(f32_dev(v))
    torch.cuda.synchronize()
    got = bytes_host(blob)
    assert_equal(got, oracle.q8_0_quantize(v), "q8_0 bytes of the f32-scale block")
    for b in range(5):
        assert got[34 * b + 2: 34 * b + 10].view(np.int8).tolist() == g["codes_first8"]


def test_q8_0_full_config():
    _say("q8_0 n=16,777,221 full")
    v = workloads.q8_0_vector()
    blob = W8.q8_0_quantize(f32_dev(v))
    y = W8.q8_0_dequantize(blob, v.size)
    torch.cuda.synchronize()
    ref = oracle.q8_0_quantize(v)
    assert_equal(bytes_host(blob), ref, "q8_0 bytes")
    assert_equal(y.cpu().numpy().view(np.uint32), oracle.q8_0_dequantize(ref, v.size).view(np.uint32), "dequant")


# ------------------------------------------------------------ GGUF A8
@pytest.mark.parametrize("qt", [INT8, FP8])
# K = 15392: the longest row staged whole (481 blocks); K = 16384: rows streamed in chunks
# K <= 4096 (128 blocks) takes the register-resident kernel: 4096 is its
# largest row, 4128 the smallest that the staged-row kernel takes
@pytest.mark.parametrize("N,K", [(1, 32), (5, 64), (37, 160), (130, 2048), (9, 2080), (11, 4096), (7, 4128),
                                 (300, 3072), (3, 15392), (5, 16384)])
def test_gguf_a8_requant(qt, N, K):
    _say(f"gguf a8 requant qt={qt} N={N} K={K}")
    rng = np.random.default_rng(N * 7 + K)
    blob = workloads.q8_0_weight_blocks(rng, N, K, zero_rows=1)
    wq, s = W8.gguf_a8_requant_q8_0(torch.from_numpy(blob).cuda(), N, K, qtype=qt)
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.gguf_a8_requant_q8_0(qt, blob, N, K)
    assert_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32), "scales")
    assert_equal(bytes_host(wq), ref_q, "codes")


@pytest.mark.parametrize("qt", [INT8, FP8])
def test_gguf_a8_requant_exact_ties(qt):
    """Rows whose absmax is 127 d1 with d1 in {1, 3, 0.75} and whose other
    blocks have d = d1 / 2 and odd codes: every such value / scale is an odd
    multiple of 1/2, a tie of the int8 rounding."""
    rng = np.random.default_rng(6)
    N, K = 6, 256
    nb = K // 32
    d = np.empty((N, nb), np.float16)
    q = rng.integers(-63, 64, (N, nb, 32)) * 2 + 1          # odd codes
    for n, d1 in enumerate([1.0, 3.0, 0.75] * 2):
        d[n] = np.float16(d1 / 2)
        d[n, 0] = np.float16(d1)
        q[n, 0] = rng.integers(-127, 128, 32)
        q[n, 0, 3] = 127
    blob = np.empty((N * nb, 34), np.uint8)
    blob[:, :2] = d.reshape(-1).view(np.uint8).reshape(-1, 2)
    blob[:, 2:] = q.reshape(-1, 32).astype(np.int8).view(np.uint8)
    blob = blob.ravel()
    wq, s = W8.gguf_a8_requant_q8_0(torch.from_numpy(blob).cuda(), N, K, qtype=qt)
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.gguf_a8_requant_q8_0(qt, blob, N, K)
    assert_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32), "scales")
    assert_equal(bytes_host(wq), ref_q, "codes")


@pytest.mark.parametrize("qt", [INT8, FP8])
def test_gguf_a8_requant_signed_scales(qt):
    """Blocks with negative, zero and negative-zero scales d and many zero
    codes: q d is -0 for q = 0 under a negative d, which e4m3 codes as 0x80
    (its own code, unlike +0), and |q d| must take |d|."""
    rng = np.random.default_rng(11)
    N, K = 5, 160
    nb = K // 32
    d = (rng.uniform(0.001, 0.02, (N, nb)) * rng.choice([-1.0, 1.0], (N, nb))).astype(np.float16)
    d[0, 1] = np.float16(0.0)
    d[1, 2] = np.float16(-0.0)
    d[2] = -np.abs(d[2])                                     # a row with only negative scales
    q = rng.integers(-127, 128, (N, nb, 32))
    q[rng.random((N, nb, 32)) < 0.3] = 0
    q[3, :, :] = 0                                           # an all-zero row under mixed signs
    blob = np.empty((N * nb, 34), np.uint8)
    blob[:, :2] = d.reshape(-1).view(np.uint8).reshape(-1, 2)
    blob[:, 2:] = q.reshape(-1, 32).astype(np.int8).view(np.uint8)
    blob = blob.ravel()
    wq, s = W8.gguf_a8_requant_q8_0(torch.from_numpy(blob).cuda(), N, K, qtype=qt)
    torch.cuda.synchronize()
    ref_q, ref_s = oracle.gguf_a8_requant_q8_0(qt, blob, N, K)
    if qt == FP8:
        assert (ref_q == 0x80).any()                         # the case is exercised
    assert_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32), "scales")
    assert_equal(bytes_host(wq), ref_q, "codes")


def test_gguf_a8_requant_full():
    _say("gguf a8 requant N=12288 K=3072 full")
    d = workloads.gguf()
    N, K = d["N"], d["K"]
    blocks = torch.from_numpy(d["w_blocks"]).cuda()
    for qt in (INT8, FP8):
        wq, s = W8.gguf_a8_requant_q8_0(blocks, N, K, qtype=qt)
        torch.cuda.synchronize()
        ref_q, ref_s = oracle.gguf_a8_requant_q8_0(qt, d["w_blocks"], N, K)
        assert_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32), f"scales qt={qt}")
        assert_equal(bytes_host(wq), ref_q, f"codes qt={qt}")


def _gguf_chain(x_bits, blob, N, K, bias_bits, qt, rows=None):
    """GPU: act-quant + requant + gguf_a8_linear; oracle: the same chain on `rows`."""
    xq, sx = W8.w8a8_quant_act_rowwise(bf16_dev(x_bits), qtype=qt)
    wq, sw = W8.gguf_a8_requant_q8_0(torch.from_numpy(blob).cuda(), N, K, qtype=qt)
    b = None if bias_bits is None else bf16_dev(bias_bits)
    y = W8.gguf_a8_linear(xq, sx, wq, sw, b)
    torch.cuda.synchronize()
    sel = np.arange(x_bits.shape[0]) if rows is None else rows
    rxq, rsx = oracle.quant_act_rowwise(qt, x_bits[sel])
    rwq, rsw = oracle.gguf_a8_requant_q8_0(qt, blob, N, K)
    return bf16_host(y)[sel], oracle.linear_axiswise(qt, rxq, rsx, rwq, rsw, bias_bits)


@pytest.mark.parametrize("qt", [INT8, FP8])
@pytest.mark.parametrize("M,N,K", [(64, 256, 256), (1, 24, 32), (5, 200, 64), (257, 300, 288), (130, 520, 1056)])
def test_gguf_a8_linear(qt, M, N, K):
    _say(f"gguf a8 linear qt={qt} M={M} N={N} K={K}")
    rng = np.random.default_rng(M + 3 * N + K)
    x = workloads.activations_bf16(rng, M, K, outliers=2)
    blob = workloads.q8_0_weight_blocks(rng, N, K, zero_rows=1)
    b = workloads.normal_bf16(rng, (N,), 0.02) if M % 2 else None
    got, ref = _gguf_chain(x, blob, N, K, b, qt)
    assert_bf16_close(got, ref, f"gguf a8 linear qt={qt}")
    if qt == FP8:
        assert_frobenius(got, ref, "gguf a8 float linear")


def test_gguf_a8_linear_full_sampled():
    _say("gguf a8 linear M=4096 N=12288 K=3072 sampled rows")
    d = workloads.gguf()
    rows = sample_rows(d["x"].shape[0], 6)
    for qt in (INT8, FP8):
        got, ref = _gguf_chain(d["x"], d["w_blocks"], d["N"], d["K"], d["bias"], qt, rows=rows)
        assert_bf16_close(got, ref, f"gguf full qt={qt}")
        if qt == FP8:
            assert_frobenius(got, ref, "gguf a8 float linear, full size")


# ------------------------------------------------------------ SVDQuant preparation
def _planted_bf16(rng, N, K, sigma):
    u, _ = np.linalg.qr(rng.standard_normal((N, len(sigma))))
    v, _ = np.linalg.qr(rng.standard_normal((K, len(sigma))))
    return oracle.f64_to_bf16((u * sigma[None, :]) @ v.T)


def _svd_prep_check(w_bits, r, iters, seed, sig_tol, lr_tol, energy_tol, what):
    from oracle import svd_prep
    N, K = w_bits.shape
    s = W8.svdq_prepare_subspace(r)
    omega = workloads.normal_bf16(np.random.default_rng(seed), (s, K), 1.0)
    l1, l2, res, sg = W8.svdq_prepare(bf16_dev(w_bits), r, bf16_dev(omega), iters=iters)
    torch.cuda.synchronize()
    l1_g, l2_g, res_g, sg_g = bf16_host(l1), bf16_host(l2), bf16_host(res), sg.cpu().numpy().astype(np.float64)
    sig_o, l1_o, l2_o, res_o = svd_prep.svdq_prepare(w_bits, r)
    # singular values, relative to the largest
    assert np.max(np.abs(sg_g - sig_o)) <= sig_tol * max(sig_o[0], 1e-30), (what, sg_g[:4], sig_o[:4])
    # the low-rank part (sign- and basis-invariant)
    p_g, p_o = svd_prep.low_rank(l2_g, l1_g), svd_prep.low_rank(l2_o, l1_o)
    assert np.linalg.norm(p_g - p_o) <= lr_tol * max(np.linalg.norm(p_o), 1e-30), what
    # the residual is W minus the stored factors' product, element by element
    # (f32 sums on the GPU, double in the oracle: one bf16 rounding apart)
    ref = svd_prep.residual(w_bits, l2_g, l1_g)
    got_v, ref_v = oracle.bf16_to_f64(res_g), oracle.bf16_to_f64(ref)
    slack = 2.0 ** -7 * np.abs(ref_v) + 2.0 ** -20 * np.max(np.abs(p_g)) + 1e-30
    assert np.all(np.abs(got_v - ref_v) <= slack), what
    # and its energy is close to the optimum (Eckart-Young)
    e_g, e_o = np.sum(got_v ** 2), np.sum(oracle.bf16_to_f64(res_o) ** 2)
    assert e_g <= e_o * (1.0 + energy_tol) + 1e-30, (what, e_g, e_o)
    _svd_prep_apriori(w_bits, omega, r, iters, sg_g, p_g, what)
    return sg_g, sig_o


def _svd_prep_apriori(w_bits, omega, r, iters, sg_g, p_g, what):
    """The GPU preparation inside the windows that the subspace iteration's
    theory fixes for this W and this test matrix (oracle.svd_prep.rsi_bounds:
    singular values, spectral and Frobenius residual of the rank-r part),
    widened by the precision of the GPU's arithmetic.  The sig_tol / lr_tol /
    e_tol checks above are tighter regression guards set from measurement; these
    windows are derived beforehand.

    Precision terms: the singular values come from Zk = W^T Q, f32 sums of
    2N exact products of bf16 W with Q stored as hi + lo bf16 halves (each
    element within 2^-18 of Q); Higham's inner-product bound gives
    |dZk| <= eps |W|^T |Q| with eps = 2^-18 + gamma_2N (1 + 2^-18),
    gamma_n = n u / (1 - n u), u = 2^-24, and Weyl's inequality moves each
    singular value by at most ||dZk||_F <= eps sqrt(s) ||W||_F (plus the f32
    storage of sigma).  The rounding of the factors to bf16 (within 2^-9
    elementwise) moves l2 . l1 by at most 2 2^-9 sqrt(sigma_1 sum sigma_j) +
    2^-18 sum sigma_j in the spectral and the Frobenius norm.  The residuals
    take the singular-value error delta to first order (the identity
    ||W - A_r||_F^2 = ||W||_F^2 - sum_{j<=r} sigma^_j^2 of an orthonormal split)."""
    from oracle import svd_prep
    N, K = w_bits.shape
    s = omega.shape[0]
    b = svd_prep.rsi_bounds(w_bits, omega, r, iters)
    w = oracle.bf16_to_f64(w_bits)
    u = 2.0 ** -24
    n2 = 2 * N
    eps = 2.0 ** -18 + n2 * u / (1 - n2 * u) * (1 + 2.0 ** -18)
    delta = eps * np.sqrt(s) * np.linalg.norm(w) + u * b["hi"][0] + 1e-30
    assert np.all(sg_g >= b["lo"] - delta) and np.all(sg_g <= b["hi"] + delta), (what, "sigma window")
    shi = b["hi"] + delta
    rnd = 2 * 2.0 ** -9 * np.sqrt(shi[0] * shi.sum()) + 2.0 ** -18 * shi.sum()
    e = w - p_g
    gram = e.T @ e if e.shape[0] >= e.shape[1] else e @ e.T
    spec_g = np.sqrt(max(np.linalg.eigvalsh(gram)[-1], 0.0))
    assert spec_g <= b["spec"] + 2 * delta + rnd, (what, "spectral residual", spec_g, b["spec"])
    fro_b = np.sum(w * w) - np.sum(np.maximum(b["lo"] - delta, 0.0) ** 2)
    assert np.linalg.norm(e) <= np.sqrt(max(fro_b, 0.0)) + rnd, (what, "Frobenius residual")


# Tolerances from the subspace-iteration error at this spectrum (sigma_i =
# 4 * 2^(-i/4)): with power iterations the factors are limited by their bf16
# rounding (~2e-4 of the low-rank part); without, or with no oversampling
# (r = 64 = s), by the captured subspace.
@pytest.mark.parametrize("r,iters,sig_tol,lr_tol,e_tol", [(16, 2, 1e-5, 1e-3, 1e-4), (32, 2, 1e-5, 1e-3, 1e-3),
                                                          (8, 0, 1e-3, 5e-2, 5e-2), (48, 1, 2e-4, 2e-3, 1e-2),
                                                          (64, 2, 2e-4, 3e-3, 2e-2)])
def test_svdq_prepare_planted(r, iters, sig_tol, lr_tol, e_tol):
    _say(f"svdq_prepare planted spectrum r={r} iters={iters}")
    rng = np.random.default_rng(r + 100 * iters)
    N, K = 512, 384
    sigma = 4.0 * 2.0 ** (-np.arange(128) / 4.0)
    w = _planted_bf16(rng, N, K, sigma)
    _svd_prep_check(w, r, iters, r + 7, sig_tol=sig_tol, lr_tol=lr_tol, energy_tol=e_tol, what=f"r={r}")


@pytest.mark.parametrize("N,K", [(8, 8), (24, 640), (1000, 72)])
def test_svdq_prepare_shapes(N, K):
    _say(f"svdq_prepare shape N={N} K={K}")
    rng = np.random.default_rng(N + K)
    sigma = 2.0 ** -np.arange(min(N, K), dtype=np.float64)
    w = _planted_bf16(rng, N, K, sigma)
    r = min(4, N, K)
    _svd_prep_check(w, r, 2, 3, sig_tol=1e-4, lr_tol=1e-2, energy_tol=1e-2, what=f"{N}x{K}")


def test_svdq_prepare_zero():
    _say("svdq_prepare zero matrix")
    w = np.zeros((64, 128), np.uint16)
    omega = workloads.normal_bf16(np.random.default_rng(0), (W8.svdq_prepare_subspace(16), 128), 1.0)
    l1, l2, res, sg = W8.svdq_prepare(bf16_dev(w), 16, bf16_dev(omega))
    torch.cuda.synchronize()
    assert not bf16_host(l1).any() and not bf16_host(l2).any() and not bf16_host(res).any()
    assert not sg.cpu().numpy().any()


def test_svdq_prepare_full_workload():
    """The SVDQuant workload's weight W = bf16(L2 L1 + R) at 12288 x 3072,
    r = 32: the preparation recovers the planted low-rank part."""
    _say("svdq_prepare N=12288 K=3072 r=32 (planted: L2 L1 + R)")
    d = workloads.svdq()
    l2p, l1p, rp = (oracle.bf16_to_f64(d[k]) for k in ("l2", "l1", "r"))
    w = oracle.f64_to_bf16(l2p @ l1p + rp)
    _svd_prep_check(w, 32, 2, 11, sig_tol=1e-5, lr_tol=2e-3, energy_tol=1e-4, what="full")


# ------------------------------------------------------------ Hadamard rotation
@pytest.mark.parametrize("qt", [INT8, FP8])
@pytest.mark.parametrize("M,K,ldq", [(5, 16, None), (37, 48, 64), (64, 96, None), (130, 1024, 1040), (9, 2048, None),
                                     (300, 3072, None), (17, 4096, None), (8, 1040, None), (3, 12288, None)])
def test_hadamard_act_quant(qt, M, K, ldq):
    _say(f"hadamard act-quant qt={qt} M={M} K={K} ldq={ldq}")
    rng = np.random.default_rng(M * 31 + K)
    x = workloads.activations_bf16(rng, M, K, outliers=min(4, K // 16))
    if M > 4:
        x[1] = 0                                            # an all-zero row
    xq, sx = W8.w8a8_quant_act_rowwise_hadamard(bf16_dev(x), qtype=qt, ldq=ldq)
    torch.cuda.synchronize()
    got_q = bytes_host(xq)
    ref_q, ref_s = oracle.quant_act_rowwise_hadamard(qt, x, ldq=got_q.shape[1])
    assert_equal(sx.cpu().numpy().view(np.uint32), ref_s.view(np.uint32), "scales")
    assert_equal(got_q, ref_q, "codes")


@pytest.mark.parametrize("M,K", [(7, 16), (33, 96), (64, 1024), (20, 3072), (5, 12288)])
def test_hadamard_rotate(M, K):
    _say(f"hadamard rotate M={M} K={K}")
    x = workloads.normal_bf16(np.random.default_rng(K + M), (M, K), 0.02)
    y = W8.w8a8_hadamard_rotate(bf16_dev(x))
    torch.cuda.synchronize()
    assert_equal(bf16_host(y), oracle.hadamard_rotate_bf16(x), "rotated bf16")


def test_hadamard_linear_full_sampled():
    """Rotated act-quant of X [4096, 3072] + rotated, tensor-wise quantized W
    [12288, 3072] + the int8 linear, against the oracle chain on sampled rows."""
    _say("hadamard linear M=4096 K=3072 N=12288 sampled rows")
    d = workloads.dit(M=4096, N1=256)
    x, w, b = d["x"], d["w2"], d["b2"]
    xq, sx = W8.w8a8_quant_act_rowwise_hadamard(bf16_dev(x))
    wr = W8.w8a8_hadamard_rotate(bf16_dev(w))
    wq, _, sw = W8.w8a8_quant_weight_tensorwise(wr)
    y = W8.w8a8_linear(xq, sx, wq, sw, bf16_dev(b))
    torch.cuda.synchronize()
    rows = sample_rows(x.shape[0], 6)
    oxq, osx = oracle.quant_act_rowwise_hadamard(INT8, x[rows])
    owr = oracle.hadamard_rotate_bf16(w)
    assert_equal(bf16_host(wr), owr, "rotated weight")
    owq, _, osw = oracle.quant_weight_tensorwise(INT8, owr)
    assert_bf16_close(bf16_host(y)[rows], oracle.linear(INT8, oxq, osx, owq, osw, b), "hadamard linear")


# ------------------------------------------------------------ determinism, graphs
def test_determinism_and_graph_capture():
    _say("determinism + graph capture of act-quant + linear")
    d = workloads.tiny(seed=4)
    rng = np.random.default_rng(9)
    x = bf16_dev(workloads.activations_bf16(rng, 300, 512, outliers=3))
    w = bf16_dev(workloads.normal_bf16(rng, (520, 512), 0.02))
    bias = bf16_dev(workloads.normal_bf16(rng, (520,), 0.02))
    wq, _, sw = W8.w8a8_quant_weight_tensorwise(w)
    xq = torch.empty((300, 512), dtype=torch.int8, device="cuda")
    sx = torch.empty(300, dtype=torch.float32, device="cuda")
    y = torch.empty((300, 520), dtype=torch.bfloat16, device="cuda")

    def step():
        W8.w8a8_quant_act_rowwise(x, out=xq, scale=sx)
        W8.w8a8_linear(xq, sx, wq, sw, bias, out=y)

    step()
    torch.cuda.synchronize()
    ref = bf16_host(y).copy()
    step()
    torch.cuda.synchronize()
    assert_equal(bf16_host(y), ref, "second eager run")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_equal(bf16_host(y), ref, f"graph replay {i}")
        _ = (x.float() * 2).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
    del d


def _graph_case(name):
    """(step, outputs) of one entry point on small inputs; step() writes into
    the preallocated outputs only."""
    rng = np.random.default_rng(23)
    M, N, K = 96, 160, 256
    x = bf16_dev(workloads.activations_bf16(rng, M, K, outliers=2))
    w = bf16_dev(workloads.normal_bf16(rng, (N, K), 0.02))
    bias = bf16_dev(workloads.normal_bf16(rng, (N,), 0.02))
    dev = x.device
    if name == "weight_quant":
        wq = torch.empty((N, K), dtype=torch.int8, device=dev)
        wqt = torch.empty((K, N), dtype=torch.int8, device=dev)
        sw = torch.empty(4, dtype=torch.float32, device=dev)
        ws = torch.empty(W8.w8a8_weight_workspace_bytes(N, K), dtype=torch.uint8, device=dev)
        return (lambda: W8.w8a8_quant_weight_tensorwise(w, transposed=True, out=wq, out_t=wqt, scale=sw,
                                                         workspace=ws)), [wq, wqt, sw[:1]]
    if name == "backward_dx":
        wq, wqt, sw = W8.w8a8_quant_weight_tensorwise(w, qtype=FP8, transposed=True)
        dy = bf16_dev(workloads.normal_bf16(rng, (M, N), 1e-3))
        dyq, sdy = W8.w8a8_quant_act_rowwise(dy, qtype=FP8)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        return (lambda: W8.w8a8_linear_backward_dx(dyq, sdy, wqt, sw, out=dx)), [dx]
    if name.startswith("svdq"):
        r = 32 if name == "svdq_r32" else 8
        l1 = bf16_dev(workloads.normal_bf16(rng, (r, K), 0.1))
        l2 = bf16_dev(workloads.normal_bf16(rng, (N, r), 0.1))
        rq, _, sr = W8.w8a8_quant_weight_tensorwise(w)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        ws = torch.empty(W8.svdq_workspace_bytes(M, r), dtype=torch.uint8, device=dev)
        return (lambda: W8.svdq_linear(x, rq, sr, l1, l2, bias, out=y, xq_out=xq, x_scale_out=sx,
                                       workspace=ws)), [y, xq, sx]
    if name == "q8_0":
        v = torch.from_numpy((rng.standard_normal(1000) * 3).astype(np.float32)).to(dev)
        blocks = torch.empty(W8.q8_0_nbytes(1000), dtype=torch.uint8, device=dev)
        back = torch.empty(1000, dtype=torch.float32, device=dev)

        def q8():
            W8.q8_0_quantize(v, out=blocks)
            W8.q8_0_dequantize(blocks, 1000, out=back)
        return q8, [blocks, back]
    if name == "gguf_a8":
        blob = torch.from_numpy(workloads.q8_0_weight_blocks(rng, N, K)).to(dev)
        wq = torch.empty((N, K), dtype=torch.int8, device=dev)
        sw = torch.empty(N, dtype=torch.float32, device=dev)
        xq, sx = W8.w8a8_quant_act_rowwise(x)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def gg():
            W8.gguf_a8_requant_q8_0(blob, N, K, out=wq, scale=sw)
            W8.gguf_a8_linear(xq, sx, wq, sw, bias, out=y)
        return gg, [wq, sw, y]
    if name == "hadamard":
        xq = torch.empty((M, K), dtype=torch.int8, device=dev)
        sx = torch.empty(M, dtype=torch.float32, device=dev)
        return (lambda: W8.w8a8_quant_act_rowwise_hadamard(x, out=xq, scale=sx)), [xq, sx]
    raise ValueError(name)


@pytest.mark.parametrize("name", ["weight_quant", "backward_dx", "svdq_r32", "svdq_r8", "q8_0", "gguf_a8",
                                  "hadamard"])
def test_graph_capture_of_every_entry_point(name):
    """Each entry point captured in a HIP graph and replayed three times, with
    the outputs cleared and unrelated eager work between replays: every replay
    equals the eager result bit for bit."""
    _say(f"graph capture: {name}")
    step, outs = _graph_case(name)
    step()
    torch.cuda.synchronize()
    ref = [bytes_host(o).copy() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        for o in outs:
            o.view(torch.uint8).zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert_equal(bytes_host(o), r, f"{name} replay {i}")
        _ = torch.randn(1 << 16, device="cuda").sum()      # unrelated eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------------ diagnostics
def test_probe_mfma_runs():
    _say("probe mfma i8")
    z = torch.zeros(65536, dtype=torch.int8, device="cuda")
    sink = W8.probe_mfma_i8(z, z, 4)
    torch.cuda.synchronize()
    assert sink.numel() == W8.library().w8a8_probe_sink_count()
    assert not sink.any()                      # zero operands accumulate zeros
    r = torch.randint(-128, 128, (65536,), dtype=torch.int8, device="cuda")
    s1 = W8.probe_mfma_i8(r, r, 4).clone()
    s2 = W8.probe_mfma_i8(r, r, 4)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and s1.any()    # deterministic, not optimized away


# ------------------------------------------------------------ e4m3 conversion
def _oracle_e4m3_runs(sign_bit, last_bits):
    """Start index (bit pattern offset from sign_bit) and oracle code of every
    run of equal codes over the f32 bit patterns sign_bit + [0, last_bits]:
    the oracle's encoding is monotone in the magnitude, so each code's run
    starts at the smallest pattern that reaches it (binary search)."""
    def code(offsets):
        v = (np.asarray(offsets, np.uint64) + sign_bit).astype(np.uint32).view(np.float32)
        return oracle.f32_to_e4m3(v).astype(np.int64) & 0x7F
    top = int(code([last_bits])[0])
    want = np.arange(1, top + 1)
    lo = np.zeros(top, np.int64)
    hi = np.full(top, last_bits, np.int64)
    while (lo < hi).any():
        mid = (lo + hi) // 2
        ge = code(mid) >= want
        hi = np.where(ge, mid, hi)
        lo = np.where(ge, lo, mid + 1)
    starts = np.concatenate([[0], lo])
    codes = np.concatenate([[0], want]) | (0x80 if sign_bit else 0)
    assert (oracle.f32_to_e4m3((starts.astype(np.uint64) + sign_bit).astype(np.uint32).view(np.float32)) ==
            codes).all()
    return starts, codes


@pytest.mark.parametrize("sign_bit", [0, 0x80000000])
def test_e4m3_conversion_every_f32_up_to_448(sign_bit):
    """The hardware conversion the quantizers use (clamp to +-448, then
    v_cvt_pk_fp8_f32) on every f32 bit pattern from +-0 to +-448 (1.14e9
    values per sign), against the oracle's OCP E4M3FN encoding: the GPU codes
    form runs, and every run must start at the oracle's boundary with the
    oracle's code -- so each of the values gets the oracle's code."""
    last = 0x43E00000                      # 448.0f
    _say(f"e4m3 conversion of every f32 in sign {sign_bit:#x} [0, 448]")
    starts, codes = _oracle_e4m3_runs(sign_bit, last)
    got = W8.probe_cvt_e4m3(sign_bit, last + 1)
    change = torch.nonzero(got[1:] != got[:-1]).flatten() + 1
    g_starts = np.concatenate([[0], change.cpu().numpy()])
    g_codes = got[torch.from_numpy(g_starts).cuda()].cpu().numpy()
    torch.cuda.synchronize()
    assert_equal(g_starts, starts, "run starts (bit-pattern offsets)")
    assert_equal(g_codes, codes, "run codes")
    del got, change
    torch.cuda.empty_cache()
