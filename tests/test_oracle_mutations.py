"""The oracle's pins catch plausible mistakes: each case below plants one
mistake in a copy of oracle/w8a8_oracle.c (a dropped term, a wrong sign,
index or constant, a different rounding), builds it, and runs the CPU pin
tests of the part it touches against that build (through W8A8_ORACLE_LIB).
At least one pin must fail.  A control build of the unchanged source must
pass the same tests, so a broken harness cannot pass for caught mistakes.
CPU only."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "w8a8_oracle.c")

QUANT, LINEAR, Q80, FORMATS, GGUF, HADAMARD = ("test_oracle_quant.py", "test_oracle_linear.py", "test_oracle_q8_0.py",
                                               "test_oracle_formats.py", "test_oracle_gguf_a8.py",
                                               "test_oracle_hadamard.py")

# name, text in the source (must occur exactly once), its mutated form, pin files
MUTATIONS = [
    ("round half up instead of half to even",
     "    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;", "    return f + 1.0;", [QUANT, Q80]),
    ("int8 code from the reciprocal instead of the quotient",
     "    float q = x / s;                                     /* one f32 rounding */\n    double r = round_half_even",
     "    float q = x * (1.0f / s);\n    double r = round_half_even", [QUANT, Q80]),
    ("no 1e-10 floor of the scale",
     "    if (amax < floor_) return floor_;", "    if (amax < 0.0f) return floor_;", [QUANT, Q80]),
    ("act-quant QMAX 128",
     "    const float qmax = qtype == 0 ? 127.0f : 448.0f;\n    for (int64_t m = 0; m < M; ++m) {\n"
     "        const uint16_t *row = x + m * ldx;",
     "    const float qmax = qtype == 0 ? 128.0f : 448.0f;\n    for (int64_t m = 0; m < M; ++m) {\n"
     "        const uint16_t *row = x + m * ldx;", [QUANT]),
    ("e4m3 QMAX 240 in the weight quantizer",
     "    const float qmax = qtype == 0 ? 127.0f : 448.0f;\n    float amax = 0.0f;\n    for (int64_t i = 0; i < N * K; ++i)",
     "    const float qmax = qtype == 0 ? 127.0f : 240.0f;\n    float amax = 0.0f;\n    for (int64_t i = 0; i < N * K; ++i)",
     [QUANT]),
    ("linear without the weight scale",
     "            double v = acc * (double)sx[m] * (double)sw;\n            if (bias)",
     "            double v = acc * (double)sx[m];\n            if (bias)", [LINEAR]),
    ("linear bias subtracted",
     "            double v = acc * (double)sx[m] * (double)sw;\n            if (bias) v += orc_bf16_to_f64(bias[n]);",
     "            double v = acc * (double)sx[m] * (double)sw;\n            if (bias) v -= orc_bf16_to_f64(bias[n]);",
     [LINEAR]),
    ("dX reads W transposed",
     "            double acc = code_dot(qtype, dyq + m * N, wq + k, N, K);",
     "            double acc = code_dot(qtype, dyq + m * N, wq + k * N, N, 1);", [LINEAR]),
    ("SVDQuant low-rank term subtracted",
     "            double v = acc * (double)sx_out[m] * (double)sr + low;",
     "            double v = acc * (double)sx_out[m] * (double)sr - low;", [LINEAR]),
    ("SVDQuant L1 indexed [K, r]",
     "orc_bf16_to_f64(l1[j * K + k])", "orc_bf16_to_f64(l1[k * r + j])", [LINEAR]),
    ("Q8_0 pad codes 1",
     "            blk[2 + (i - start)] = i < end ? (uint8_t)orc_code_int8(x[i], s) : 0;",
     "            blk[2 + (i - start)] = i < end ? (uint8_t)orc_code_int8(x[i], s) : 1;", [Q80]),
    ("Q8_0 codes from the stored f16 scale",
     "            blk[2 + (i - start)] = i < end ? (uint8_t)orc_code_int8(x[i], s) : 0;",
     "            blk[2 + (i - start)] = i < end ? (uint8_t)orc_code_int8(x[i], (float)orc_f16_to_f64(d)) : 0;",
     [Q80]),
    ("Q8_0 scale bytes big-endian",
     "        blk[0] = (uint8_t)(d & 0xff);\n        blk[1] = (uint8_t)(d >> 8);",
     "        blk[0] = (uint8_t)(d >> 8);\n        blk[1] = (uint8_t)(d & 0xff);", [Q80]),
    ("Q8_0 dequantize reads the scale as bf16",
     "        y[i] = (float)((double)q * orc_f16_to_f64(d));", "        y[i] = (float)((double)q * orc_bf16_to_f64(d));",
     [Q80]),
    ("e4m3 subnormals one binade low",
     "    if (e == 0) v = ldexp((double)m / 8.0, -6);", "    if (e == 0) v = ldexp((double)m / 8.0, -7);", [FORMATS]),
    ("f16 subnormals one binade low",
     "    else if (e == 0) v = ldexp((double)m, -24);", "    else if (e == 0) v = ldexp((double)m, -25);",
     [FORMATS, Q80]),
    ("ties of the format encoders go up",
     "    return (lo % 2 == 0) ? lo : hi;", "    return hi;", [FORMATS]),
    ("GGUF A8 row absmax without the absolute value",
     "            float a = fabsf(v_work[k]);", "            float a = v_work[k];", [GGUF]),
    ("GGUF A8 linear takes the weight scale by row of X",
     "            double v = acc * (double)sx[m] * (double)sw[n];", "            double v = acc * (double)sx[m] * (double)sw[m];",
     [GGUF]),
    ("Hadamard difference reversed",
     "                        v[i + h] = a - d;", "                        v[i + h] = d - a;", [HADAMARD]),
    ("Hadamard normalized by 1/b",
     "    const float c = (float)(1.0 / sqrt((double)b));", "    const float c = (float)(1.0 / (double)b);", [HADAMARD]),
    ("Hadamard blocks capped at 512",
     "    while (K % (b * 2) == 0 && b * 2 <= 1024) b *= 2;", "    while (K % (b * 2) == 0 && b * 2 <= 512) b *= 2;",
     [HADAMARD]),
]


def _build(src_text, path):
    with open(path + ".c", "w") as f:
        f.write(src_text)
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-o", path,
           path + ".c", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def _pins(lib, files):
    env = dict(os.environ, W8A8_ORACLE_LIB=lib, PYTHONDONTWRITEBYTECODE="1")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *[os.path.join(HERE, f) for f in files]]
    return subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)


@pytest.fixture(scope="module")
def source():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    with open(SRC) as f:
        return f.read()


def test_control_build_passes_the_pins(source, tmp_path):
    lib = str(tmp_path / "control.so")
    _build(source, lib)
    r = _pins(lib, [QUANT, LINEAR, Q80, FORMATS, GGUF, HADAMARD])
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]


def test_every_planted_mistake_fails_a_pin(source, tmp_path):
    for name, old, _, _ in MUTATIONS:
        assert source.count(old) == 1, f"mutation site not unique or gone: {name}"

    def run(i):
        name, old, new, files = MUTATIONS[i]
        lib = str(tmp_path / f"mutant{i}.so")
        _build(source.replace(old, new), lib)
        return name, _pins(lib, files)

    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(run, range(len(MUTATIONS))))
    survivors = [name for name, r in results if r.returncode == 0]
    assert not survivors, f"mistakes no pin catches: {survivors}"
    # caught by a failing assertion (pytest's exit status 1), not by a crash
    # or a collection error
    other = [(name, r.returncode, r.stdout[-500:]) for name, r in results if r.returncode != 1]
    assert not other, other
