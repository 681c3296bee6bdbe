"""Pins of the oracle's number formats (bf16, f16, OCP e4m3) against library
casts and the format definitions.  CPU only."""
import numpy as np
import pytest
import torch

import oracle


def _finite_f32_patterns(rng, n):
    u = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    return f[np.isfinite(f)]


def test_bf16_decode_all_patterns_matches_torch():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f64(b)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_f32_to_bf16_matches_torch_rne():
    rng = np.random.default_rng(1)
    f = np.concatenate([
        _finite_f32_patterns(rng, 300_000),
        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895e38, 3.4e38, -3.4e38, 1e-45, -1e-45]),
    ])
    ours = oracle.f32_to_bf16(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_f64_to_bf16_rounds_once():
    # Values within 2^-30 of a bf16 midpoint: rounding through f32 first lands on
    # the midpoint and then ties to even, which is wrong in the second and fourth
    # case; direct rounding of the double picks the nearer neighbour.
    v = np.array([1 + 2**-8 + 2**-30, 1 + 2**-8 - 2**-30, 1 + 3 * 2**-8 + 2**-30, 1 + 3 * 2**-8 - 2**-30])
    assert oracle.f64_to_bf16(v).tolist() == [0x3F81, 0x3F80, 0x3F82, 0x3F81]
    # exact midpoints tie to even
    assert oracle.f64_to_bf16(np.array([1 + 2**-8, 1 + 3 * 2**-8])).tolist() == [0x3F80, 0x3F82]


def test_f16_matches_numpy_rne():
    rng = np.random.default_rng(2)
    f = np.concatenate([
        (rng.standard_normal(200_000) * 10.0 ** rng.integers(-9, 6, 200_000)).astype(np.float32),
        np.float32([65504.0, 65519.996, 65520.0, 7e4, 2**-24, 2**-25, 2**-25 * 1.0001, 3 * 2**-25,
                    6.1e-5, 1 / 127, 1e-10, -0.0, 0.0]),
    ])
    ours = oracle.f32_to_f16(f)
    with np.errstate(over="ignore"):                     # 7e4 and 65520 overflow to inf on purpose
        ref = f.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    # overflow and tie corner cases spelled out (IEEE binary16, RNE)
    assert oracle.f32_to_f16(np.float32([65519.996, 65520.0, 2**-25, 3 * 2**-25])).tolist() == \
        [0x7BFF, 0x7C00, 0x0000, 0x0002]


def test_f16_decode_all_patterns_matches_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isinf(ours), np.isinf(ref))


def test_e4m3_decode_all_codes():
    c = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(c)
    ref = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.isnan(ours).sum() == 2 and np.isnan(ours[[0x7F, 0xFF]]).all()
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # definition: max finite 448, smallest subnormal 2^-9, smallest normal 2^-6
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0**-9 and ours[0x08] == 2.0**-6
    assert np.signbit(ours[0x80]) and ours[0x80] == 0.0


def test_f32_to_e4m3_matches_torch_within_range():
    rng = np.random.default_rng(3)
    allbf = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    allbf = allbf[np.isfinite(allbf) & (np.abs(allbf) <= 448)]
    rnd = (rng.uniform(-1, 1, 300_000) * 2.0 ** rng.integers(-14, 9, 300_000)).astype(np.float32)
    rnd = rnd[np.abs(rnd) <= 448]
    f = np.concatenate([allbf, rnd])
    ours = oracle.f32_to_e4m3(f)
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_midpoints_tie_to_even():
    # Every midpoint between adjacent finite codes is exact in f32; it must go to
    # the code with an even mantissa LSB (an even code number).
    vals = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    got = oracle.f32_to_e4m3(mids).astype(int)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    # one f32 ulp on either side of each midpoint goes to the nearer code
    below = np.nextafter(mids, np.float32(0)).astype(np.float32)
    above = np.nextafter(mids, np.float32(1e9)).astype(np.float32)
    assert np.array_equal(oracle.f32_to_e4m3(below).astype(int), lo)
    assert np.array_equal(oracle.f32_to_e4m3(above).astype(int), lo + 1)


@pytest.mark.parametrize("v,code", [(448.0, 0x7E), (460.0, 0x7E), (-448.0, 0xFE), (-0.0, 0x80), (0.0, 0x00)])
def test_e4m3_edges(v, code):
    assert int(oracle.f32_to_e4m3(np.float32([v]))[0]) == code


def test_absmax_scale_rule_and_floor():
    # s = 1e-10f when absmax < 1e-10f, else f32(absmax / qmax) -- one rounding
    floor = np.float32(1e-10)
    assert oracle.absmax_scale(0.0, 127.0) == floor
    assert oracle.absmax_scale(np.nextafter(floor, np.float32(0)), 127.0) == floor
    assert oracle.absmax_scale(floor, 127.0) == np.float32(np.float32(1e-10) / np.float32(127.0))  # not floored
    assert oracle.absmax_scale(127.0, 127.0) == np.float32(1.0)
    assert oracle.absmax_scale(448.0, 448.0) == np.float32(1.0)
    rng = np.random.default_rng(5)
    for a in (rng.random(2000) * 10.0 ** rng.integers(-9, 6, 2000)).astype(np.float32):
        for q in (127.0, 448.0):
            want = np.float32(a) / np.float32(q) if a >= floor else floor
            assert oracle.absmax_scale(a, q) == want, (a, q)


def test_f64_to_f16_rounds_once_from_double():
    # numpy's float64 -> float16 cast rounds once, directly
    rng = np.random.default_rng(6)
    v = rng.standard_normal(200_000) * 10.0 ** rng.integers(-8, 5, 200_000)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f64_to_f16(v), ref)
    # a tie of f16 that is not a tie in double: 1 + 2^-11 is the midpoint of
    # 1 and 1 + 2^-10; a hair above it must round up, which rounding through
    # f32 first (to the exact midpoint, then to even) would miss
    h = oracle.f64_to_f16(np.array([1 + 2.0**-11, 1 + 2.0**-11 + 2.0**-40, 1 + 2.0**-11 - 2.0**-40]))
    assert h.tolist() == [0x3C00, 0x3C01, 0x3C00]


def test_f64_to_e4m3_rounds_once_from_double():
    # 1.0625 is the midpoint of e4m3 1.0 (0x38) and 1.125 (0x39): ties to the
    # even code 0x38; just above it 0x39 (f32 would first round it to 1.0625)
    e = oracle.f64_to_e4m3(np.array([1.0625, 1.0625 + 2.0**-40, 1.0625 - 2.0**-40, -1.0625 - 2.0**-40]))
    assert e.tolist() == [0x38, 0x39, 0x38, 0xB9]
    # wherever a double is exactly an f32, the direct and the f32 paths agree
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(100_000) * 10.0 ** rng.integers(-4, 3, 100_000)).astype(np.float32)
    f = np.clip(f, -448, 448)
    assert np.array_equal(oracle.f64_to_e4m3(f.astype(np.float64)), oracle.f32_to_e4m3(f))
