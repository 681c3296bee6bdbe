"""The GPU quantizers' one-correction quotient against IEEE f32 division,
exhaustively over every bf16 (value, absmax) pair for both QMAX, and on 10^8
random f32 pairs (tests/quotient_check.c).  CPU only."""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "quotient_check.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path_factory.mktemp("quotient") / "quotient_check")
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-Wall", SRC, "-o", exe,
           "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, *args):
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=600)
    m = re.search(r"pairs (\d+) mismatches (\d+) tiny_last_bit_differences (\d+)", r.stdout)
    assert m, r.stdout + r.stderr
    return r.returncode, int(m.group(1)), int(m.group(2)), r.stdout


def test_every_bf16_pair_gives_the_ieee_codes(checker):
    rc, pairs, bad, out = _run(checker, "bf16")
    # 32,640 positive finite bf16 absmax values, every |x| <= absmax, both
    # signs, two QMAX: sum over a of 2 (a + 1), twice
    assert pairs == 2 * sum(2 * (a + 1) for a in range(1, 0x7F80))
    assert rc == 0 and bad == 0, out


def test_1e8_random_f32_pairs_give_the_ieee_codes(checker):
    rc, pairs, bad, out = _run(checker, "f32", "100000000", "20261203")
    assert pairs == 100_000_000
    assert rc == 0 and bad == 0, out
