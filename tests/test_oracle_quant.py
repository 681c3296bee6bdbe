"""Pins of the oracle's absmax quantizers (row-wise activations, tensor-wise
weights): worked examples, closed-form invariants and special cases.  CPU only."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bf16(vals):
    return workloads.f32_to_bf16_bits(np.asarray(vals, np.float32))


def test_int8_rne_worked_example():
    g = _gold("int8_rne_row.json")
    q, s = oracle.quant_act_rowwise(oracle.INT8, _bf16([g["row"]]))
    assert s[0] == np.float32(g["scale"])
    assert q[0].view(np.int8).tolist() == g["codes"]


def test_fp8_worked_example():
    g = _gold("fp8_e4m3_row.json")
    q, s = oracle.quant_act_rowwise(oracle.FP8_E4M3, _bf16([g["row"]]))
    assert s[0] == np.float32(g["scale"])
    assert [f"{c:02X}" for c in q[0]] == g["codes_hex"]


def test_scale_floor_and_zero_rows():
    # Q8_0::quantize floors the scale at 1e-10 (f32) when max_abs < 1e-10; the
    # same rule serves every quantizer.  1e-10f has bits 0x2EDBE6FF.
    x = np.zeros((3, 64), np.uint16)
    x[1, 5] = _bf16([9e-11])[0]           # below the floor
    x[2, 7] = _bf16([-2e-10])[0]          # above the floor -> amax / QMAX
    for qt, qmax in ((oracle.INT8, 127.0), (oracle.FP8_E4M3, 448.0)):
        q, s = oracle.quant_act_rowwise(qt, x)
        assert s[0].view(np.uint32) == 0x2EDBE6FF and s[1].view(np.uint32) == 0x2EDBE6FF
        assert not q[0].any()
        amax2 = np.float32(workloads.bf16_bits_to_f32(x[2, 7:8])[0])
        assert s[2] == np.float32(abs(amax2) / np.float32(qmax))
    # the element below the floor: 9e-11 / 1e-10 = 0.9 -> int8 code 1
    q, _ = oracle.quant_act_rowwise(oracle.INT8, x)
    assert q[1].view(np.int8)[5] == 1


def _near_tie_rows(rng, M, K, qmax):
    """Rows whose quotients land on and near half-integers: amax fixed to qmax*2^e
    times a random bf16 factor so that scale is inexact."""
    x = rng.standard_normal((M, K)).astype(np.float32) * np.float32(3.0)
    return workloads.f32_to_bf16_bits(x)


@pytest.mark.parametrize("qt,qmax", [(oracle.INT8, 127), (oracle.FP8_E4M3, 448)])
def test_absmax_element_maps_to_qmax_and_bounds(qt, qmax):
    rng = np.random.default_rng(5)
    x = workloads.activations_bf16(rng, 96, 512)
    q, s = oracle.quant_act_rowwise(qt, x)
    xf = workloads.bf16_bits_to_f32(x).astype(np.float64)
    am = np.abs(xf).argmax(axis=1)
    if qt == oracle.INT8:
        codes = q.view(np.int8).astype(np.float64)
        # fl(a / fl(a/Q)) = Q (1 +- 2^-23) rounds to +-Q exactly
        assert np.array_equal(np.abs(codes[np.arange(96), am]), np.full(96, 127.0))
        # |x - q s| <= s/2 (the dequant error bound), codes never reach -128
        err = np.abs(xf - codes * s[:, None].astype(np.float64))
        assert (err <= s[:, None].astype(np.float64) / 2 * (1 + 2**-20)).all()
        assert codes.min() >= -127
    else:
        dec = oracle.e4m3_to_f64(q)
        assert np.array_equal(np.abs(dec[np.arange(96), am]), np.full(96, 448.0))
        # e4m3 relative spacing is 2^-3: |x/s - e4m3| <= 2^-4 |x/s| for normals,
        # and <= 2^-10 absolute in the subnormal range
        qv = xf / s[:, None]
        bound = np.maximum(np.abs(qv) * 2**-4, 2.0**-10) * (1 + 2**-20)
        assert (np.abs(qv - dec) <= bound).all()


def test_int8_divides_rather_than_multiplies_by_reciprocal():
    # The Q8_0 page divides value / scale.  Find rows where x * fl(1/s) rounds to
    # a different integer than fl(x / s) (numpy's IEEE f32 division); the oracle
    # must agree with the division every time.
    rng = np.random.default_rng(7)
    found = 0
    for _ in range(200):
        amax = np.float32(workloads.bf16_bits_to_f32(_bf16([rng.uniform(1, 100)]))[0])
        s = np.float32(amax / np.float32(127.0))
        r = np.float32(np.float32(1.0) / s)
        xs = workloads.bf16_bits_to_f32(_bf16(rng.uniform(-amax, amax, 4096)))
        div = np.rint(xs / s)
        mul = np.rint(xs * r)
        bad = np.nonzero(div != mul)[0]
        if bad.size == 0:
            continue
        row = np.concatenate([[amax], xs[bad]]).astype(np.float32)
        q, sq = oracle.quant_act_rowwise(oracle.INT8, _bf16([row]))
        assert sq[0] == s
        assert q[0].view(np.int8)[1:].tolist() == np.rint(xs[bad] / s).astype(int).tolist()
        found += bad.size
    assert found > 0


def test_int8_ties_go_to_even():
    # Quotients that are exact half-integers must round to even, at any scale.
    for e in range(-6, 7):
        s = np.float32(2.0**e)
        amax = np.float32(127.0) * s
        halves = (np.arange(-126, 127) + np.float32(0.5)).astype(np.float32) * s
        row = np.concatenate([[amax], halves]).astype(np.float32)
        q, sq = oracle.quant_act_rowwise(oracle.INT8, _bf16([row]))
        assert sq[0] == s
        h = np.arange(-126, 127) + 0.5
        want = np.where(np.floor(h) % 2 == 0, np.floor(h), np.floor(h) + 1)
        # bf16 keeps 8 significant bits: only halves below 128 survive the cast
        assert q[0].view(np.int8)[1:].tolist() == want.astype(int).tolist()


def test_pad_columns_are_zero():
    x = workloads.random_rows(3, 5, 40)
    q, s = oracle.quant_act_rowwise(oracle.INT8, x, ldq=64)
    assert q.shape == (5, 64) and not q[:, 40:].any()
    q2, s2 = oracle.quant_act_rowwise(oracle.INT8, x)
    assert np.array_equal(q[:, :40], q2) and np.array_equal(s, s2)


def test_code_clamps():
    assert oracle.code_int8(1000.0, 1.0) == 127
    assert oracle.code_int8(-1000.0, 1.0) == -128
    assert oracle.code_e4m3(1000.0, 1.0) == 0x7E
    assert oracle.code_e4m3(-1000.0, 1.0) == 0xFE


@pytest.mark.parametrize("qt", [oracle.INT8, oracle.FP8_E4M3])
def test_weight_tensorwise_one_scale_and_transpose(qt):
    rng = np.random.default_rng(11)
    w = workloads.normal_bf16(rng, (48, 80), 0.02)
    q, qtr, s = oracle.quant_weight_tensorwise(qt, w, transposed=True)
    wf = workloads.bf16_bits_to_f32(w)
    qmax = np.float32(127.0 if qt == oracle.INT8 else 448.0)
    assert s == np.float32(np.abs(wf).max() / qmax)
    assert np.array_equal(qtr, q.T)
    # the tensor-wise result equals the row-wise quantizer applied to the whole
    # tensor flattened into one row (same absmax group)
    q1, s1 = oracle.quant_act_rowwise(qt, w.reshape(1, -1))
    assert s1[0] == s and np.array_equal(q1.reshape(48, 80), q)
