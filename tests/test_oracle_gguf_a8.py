"""Pins of the oracle's GGUF A8 path (OneTrainer wiki "Quantization", GGUF A8
int / GGUF A8 float): the axis-wise re-quantization of a Q8_0 weight and the
linear with per-output-channel weight scales.  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "gguf_a8_requant.json")) as f:
        return json.load(f)


def _blocks(rows, K):
    """Q8_0 bytes of a weight given per row as a list of {d_hex, leading codes}."""
    nb = K // 32
    out = np.zeros((len(rows), nb, 34), np.uint8)
    for n, row in enumerate(rows):
        assert len(row) == nb
        for b, blk in enumerate(row):
            d = int(blk["d_hex"], 16)
            out[n, b, 0], out[n, b, 1] = d & 0xFF, d >> 8
            c = np.array(blk["codes"], np.int64).astype(np.int8).view(np.uint8)
            out[n, b, 2:2 + c.size] = c
    return out.ravel()


def _expected_codes(spec, N, K, hexcodes=False):
    e = np.zeros((N, K), np.uint8)
    for n, row in enumerate(spec):
        for k, v in row.items():
            e[n, int(k)] = int(v, 16) if hexcodes else np.uint8(np.int8(v))
    return e


def test_requant_worked_example_int8():
    g = _gold()["int8"]
    wq, s = oracle.gguf_a8_requant_q8_0(oracle.INT8, _blocks(g["rows"], g["K"]), g["N"], g["K"])
    assert [f"{int(v):08X}" for v in s.view(np.uint32)] == g["scale_f32_hex"]
    assert np.array_equal(wq, _expected_codes(g["codes_nonzero"], g["N"], g["K"]))


def test_requant_worked_example_e4m3():
    g = _gold()["e4m3"]
    wq, s = oracle.gguf_a8_requant_q8_0(oracle.FP8_E4M3, _blocks(g["rows"], g["K"]), g["N"], g["K"])
    assert [f"{int(v):08X}" for v in s.view(np.uint32)] == g["scale_f32_hex"]
    assert np.array_equal(wq, _expected_codes(g["codes_hex_nonzero"], g["N"], g["K"], hexcodes=True))


def _random_q8_0_weight(N, K, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w[rng.integers(0, N, 4), rng.integers(0, K, 4)] *= 30.0
    return oracle.q8_0_quantize(w.ravel())


@pytest.mark.parametrize("qt", [oracle.INT8, oracle.FP8_E4M3])
def test_requant_matches_numpy_chain(qt):
    """Library cross-check: numpy dequantizes (int8 code times the f16 scale as
    f32), takes the row absmax, divides in f32 and rounds half to even (rint)
    or to e4m3 (torch's RNE cast), independently of the oracle's C code."""
    import torch

    N, K = 37, 160
    blob = _random_q8_0_weight(N, K, 1)
    wq, s = oracle.gguf_a8_requant_q8_0(qt, blob, N, K)
    blk = blob.reshape(N * K // 32, 34)
    d = blk[:, :2].copy().view(np.float16).astype(np.float32)          # [blocks, 1]
    q = blk[:, 2:].view(np.int8).astype(np.float32)                     # [blocks, 32]
    v = (q * d).reshape(N, K)
    amax = np.abs(v).max(axis=1)
    qmax = np.float32(127.0 if qt == oracle.INT8 else 448.0)
    ref_s = np.where(amax < np.float32(1e-10), np.float32(1e-10), amax / qmax).astype(np.float32)
    assert np.array_equal(s.view(np.uint32), ref_s.view(np.uint32))
    quo = (v / ref_s[:, None]).astype(np.float32)
    if qt == oracle.INT8:
        ref = np.clip(np.rint(quo), -128, 127).astype(np.int8).view(np.uint8)
    else:
        ref = torch.from_numpy(np.clip(quo, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(wq, ref)


@pytest.mark.parametrize("qt", [oracle.INT8, oracle.FP8_E4M3])
def test_requant_invariants(qt):
    N, K = 64, 96
    blob = _random_q8_0_weight(N, K, 2)
    wq, s = oracle.gguf_a8_requant_q8_0(qt, blob, N, K)
    v = oracle.q8_0_dequantize(blob, N * K).reshape(N, K)
    qmax = 127 if qt == oracle.INT8 else 448
    dec = wq.view(np.int8).astype(np.float64) if qt == oracle.INT8 else oracle.e4m3_to_f64(wq)
    # every row's absmax element encodes to +-QMAX
    idx = np.abs(v).argmax(axis=1)
    assert np.all(np.abs(dec[np.arange(N), idx]) == qmax)
    if qt == oracle.INT8:
        # |v - q s| <= s / 2 (one rounding of an exact-ish quotient)
        err = np.abs(v.astype(np.float64) - dec * s[:, None].astype(np.float64))
        assert np.all(err <= s[:, None] * (0.5 + 1e-6))
        assert not np.any(wq.view(np.int8) == -128)


def test_requant_of_integer_rows_is_identity():
    """A Q8_0 row whose scale is 1 and whose codes reach 127 holds integers;
    re-quantizing it with QMAX 127 gives scale 1 and the same codes."""
    rng = np.random.default_rng(3)
    N, K = 5, 128
    codes = rng.integers(-127, 128, (N, K)).astype(np.int8)
    codes[:, 7] = 127
    blob = np.zeros((N, K // 32, 34), np.uint8)
    blob[:, :, 0], blob[:, :, 1] = 0x00, 0x3C
    blob[:, :, 2:] = codes.reshape(N, K // 32, 32).view(np.uint8)
    wq, s = oracle.gguf_a8_requant_q8_0(oracle.INT8, blob.ravel(), N, K)
    assert np.all(s == 1.0)
    assert np.array_equal(wq.view(np.int8), codes)


@pytest.mark.parametrize("qt", [oracle.INT8, oracle.FP8_E4M3])
def test_axiswise_linear_reduces_to_tensorwise(qt):
    """With the same scale in every channel the axis-wise linear is the
    tensor-wise one (same double arithmetic, bit for bit)."""
    rng = np.random.default_rng(4)
    M, N, K = 9, 23, 64
    x = oracle.f32_to_bf16(rng.standard_normal((M, K)).astype(np.float32))
    w = oracle.f32_to_bf16((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    bias = oracle.f32_to_bf16((rng.standard_normal(N) * 0.02).astype(np.float32))
    xq, sx = oracle.quant_act_rowwise(qt, x)
    wq, _, sw = oracle.quant_weight_tensorwise(qt, w)
    a = oracle.linear(qt, xq, sx, wq, sw, bias)
    b = oracle.linear_axiswise(qt, xq, sx, wq, np.full(N, sw, np.float32), bias)
    assert np.array_equal(a, b)


def test_axiswise_linear_matches_numpy_f64():
    rng = np.random.default_rng(5)
    M, N, K = 7, 11, 96
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    wq = rng.integers(-127, 128, (N, K)).astype(np.int8)
    sx = (rng.random(M) * 0.01 + 1e-3).astype(np.float32)
    sw = (rng.random(N) * 0.001 + 1e-4).astype(np.float32)
    bias = oracle.f32_to_bf16((rng.standard_normal(N) * 0.02).astype(np.float32))
    y = oracle.linear_axiswise(oracle.INT8, xq, sx, wq, sw, bias)
    acc = xq.astype(np.int64) @ wq.astype(np.int64).T
    ref = acc.astype(np.float64) * sx[:, None].astype(np.float64) * sw[None, :].astype(np.float64)
    ref += oracle.bf16_to_f64(bias)[None, :]
    assert np.array_equal(y, oracle.f64_to_bf16(ref))
    # a swapped index (sw[m] for sw[n]) would break this
    assert not np.array_equal(oracle.linear_axiswise(oracle.INT8, xq, sx, wq, sw[::-1].copy(), bias), y)
