"""Pins of the oracle's GGUF Q8_0 quantize/dequantize (entrenar q8_0.rs) against
a worked example, the page's size formulas, invariants and the f16 bound.
CPU only."""
import json
import os
from fractions import Fraction

import numpy as np

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_q8_0_worked_example_n37():
    g = _gold("q8_0_n37.json")
    x = np.array(g["values"], np.float32)
    blob = oracle.q8_0_quantize(x)
    assert blob.size == g["nbytes"] == oracle.q8_0_nbytes(x.size)
    assert f"{int(blob[0]) | (int(blob[1]) << 8):04X}" == g["block0_scale_f16_hex"]
    assert blob[2:34].view(np.int8).tolist() == g["block0_codes"]
    assert f"{int(blob[34]) | (int(blob[35]) << 8):04X}" == g["block1_scale_f16_hex"]
    assert blob[36:41].view(np.int8).tolist() == g["block1_codes"]
    assert not blob[41:68].any()
    y = oracle.q8_0_dequantize(blob, x.size)
    assert y.tolist() == g["dequantized"]
    assert np.abs(y - x).max() == g["max_roundtrip_error"]


def test_q8_0_sizes_against_page_formulas():
    g = _gold("q8_0_sizes.json")
    n = g["n"]
    blocks = -(-n // 32)
    assert blocks == g["num_blocks"]
    assert 2 * blocks + n == g["gguf_bytes"] and 4 * blocks + n == g["memory_bytes"]
    assert abs(4 * n / g["gguf_bytes"] - g["compression_ratio"]) < 1e-6
    assert oracle.q8_0_nbytes(n) == g["padded_nbytes"] == g["gguf_bytes"] + g["pad_codes"]
    for k in (0, 1, 31, 32, 33, 64, 65):
        assert oracle.q8_0_nbytes(k) == 34 * (-(-k // 32))


def test_q8_0_invariants_and_f16_bound():
    rng = np.random.default_rng(9)
    for n in (1, 31, 32, 33, 1000, 4099):
        x = (rng.standard_normal(n) * 10.0 ** rng.integers(-3, 3, n)).astype(np.float32)
        blob = oracle.q8_0_quantize(x)
        nb = -(-n // 32)
        blocks = blob.reshape(nb, 34)
        d = blocks[:, :2].copy().view(np.uint16).ravel()
        codes = blocks[:, 2:].view(np.int8)
        xp = np.zeros(nb * 32, np.float32)
        xp[:n] = x
        xb = xp.reshape(nb, 32)
        amax = np.abs(xb).max(1)
        s = (amax / np.float32(127)).astype(np.float32)
        # stored scale is the f16 rounding of the f32 scale
        assert np.array_equal(d, s.astype(np.float16).view(np.uint16))
        # the largest element maps to +-127; pad codes are zero
        assert (np.abs(codes[np.arange(nb), np.abs(xb).argmax(1)]) == 127).all()
        assert not codes.ravel()[n:].any()
        # per element |x - q d| <= s/2 + 127 |s - d|
        y = oracle.q8_0_dequantize(blob, n)
        dd = d.view(np.float16).astype(np.float64)
        bound = s.astype(np.float64) / 2 + 127 * np.abs(s.astype(np.float64) - dd)
        err = np.abs(y.astype(np.float64) - x.astype(np.float64))
        assert (err <= np.repeat(bound, 32)[:n] * (1 + 2**-20)).all()
        # dequantize is the exact product code * f16 scale
        assert np.array_equal(y, (codes.astype(np.float64) * dd[:, None]).ravel()[:n].astype(np.float32))


def test_q8_0_zero_block():
    x = np.zeros(64, np.float32)
    x[32] = 1.0
    blob = oracle.q8_0_quantize(x)
    assert blob[0] == 0 and blob[1] == 0 and not blob[2:34].any()    # f16(1e-10) = 0
    y = oracle.q8_0_dequantize(blob, 64)
    assert not y[:32].any()


def _f32_scale_block():
    g = _gold("q8_0_f32_scale_block.json")
    x = np.zeros(g["n"], np.float32)
    for i, (num, den) in enumerate(g["values_num_den"]):
        x[i] = np.float32(num / den)
        assert Fraction(float(x[i])) == Fraction(num, den)     # every value exact in f32
    return g, x


def test_q8_0_codes_from_the_f32_scale():
    """Codes come from the f32 block scale, the quotient rounded to f32 first
    (Q8_0::quantize divides by the f32 scale; f16 only on export).  Each of the
    two other readings changes at least one code of this block."""
    g, x = _f32_scale_block()
    blob = oracle.q8_0_quantize(x)
    assert blob.size == 34
    assert f"{int(blob[0]) | (int(blob[1]) << 8):04X}" == g["scale_f16_hex"]
    s = np.float32(1.0) / np.float32(127.0)
    assert f"{int(s.view(np.uint32)):08X}" == g["scale_f32_hex"]
    codes = blob[2:34].view(np.int8)
    assert codes[:8].tolist() == g["codes_first8"]
    assert not codes[8:].any()
    assert g["codes_first8"] != g["codes_if_scale_were_f16"]
    assert g["codes_first8"] != g["codes_if_quotient_unrounded"]
    y = oracle.q8_0_dequantize(blob, g["n"])
    want = [Fraction(a, b) for a, b in g["dequantized_first8_num_den"]]
    assert [Fraction(float(v)) for v in y[:8]] == want


def test_q8_0_outlier_vector_sample():
    v = workloads.q8_0_vector(n=100_003, seed=0)
    blob = oracle.q8_0_quantize(v)
    y = oracle.q8_0_dequantize(blob, v.size)
    assert blob.size == 34 * 3126
    rel = np.abs(y - v).max() / np.abs(v).max()
    assert rel < 0.01
