"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
quantized-linear arithmetic, so both the CPU oracle and the HIP path can be fed
from it without sharing any of the method's code.

Recipe (every workload): numpy PCG64 (`default_rng(seed)`, seed 0 unless
stated), normals drawn in float64, scaled, cast to float32 and then rounded to
bf16 with torch's CPU cast (round to nearest even).  bf16 arrays are returned as
uint16 bit patterns.  "N(0, s)" means standard deviation s.  Outlier channels
are `rng.choice(K, 8, replace=False)` and are multiplied by 20 in every row.

Workloads (transformer-shaped stand-ins for the activations and weights of the
models the pages mention; no dataset is involved):
  tiny   X [64,256] N(0,1), W [256,256] N(0,0.02), bias [256] N(0,0.02)
  q8_0   f32 [16,777,221] N(0,1), floor(0.001 n) distinct indices scaled x50
  dit    X [4608,3072] N(0,1) + 8 outlier channels x20,
         W1 [3072,3072], W2 [12288,3072] N(0,0.02), biases N(0,0.02)
  svdq   X [4096,3072] as dit, L1 [32,3072], L2 [12288,32] N(0,0.1),
         R [12288,3072] N(0,0.02), bias [12288] N(0,0.02)
  fp8    W [12288,3072] N(0,0.02), X [8192,3072] N(0,1), dY [8192,12288] N(0,1e-3)
  gguf   W [12288,3072] as GGUF Q8_0 blocks (synthetic block contents, see
         q8_0_weight_blocks), X [4096,3072] as dit, bias [12288] N(0,0.02)
"""
import numpy as np
import torch

_CHUNK = 1 << 24


def f32_to_bf16_bits(a):
    """float32 array -> bf16 bit patterns (uint16), via torch's RNE CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_f32(rng, shape, std=1.0):
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    for i in range(0, n, _CHUNK):
        m = min(_CHUNK, n - i)
        out[i:i + m] = (rng.standard_normal(m, dtype=np.float64) * std).astype(np.float32)
    return out.reshape(shape)


def normal_bf16(rng, shape, std=1.0):
    return f32_to_bf16_bits(normal_f32(rng, shape, std))


def activations_bf16(rng, M, K, outliers=8, factor=20.0):
    x = normal_f32(rng, (M, K), 1.0)
    if outliers:
        cols = rng.choice(K, outliers, replace=False)
        x[:, cols] *= np.float32(factor)
    return f32_to_bf16_bits(x)


def tiny(seed=0):
    rng = np.random.default_rng(seed)
    x = normal_bf16(rng, (64, 256), 1.0)
    w = normal_bf16(rng, (256, 256), 0.02)
    bias = normal_bf16(rng, (256,), 0.02)
    return {"x": x, "w": w, "bias": bias}


def q8_0_vector(n=16_777_221, seed=0):
    rng = np.random.default_rng(seed)
    v = normal_f32(rng, (n,), 1.0)
    idx = rng.choice(n, n // 1000, replace=False)
    v[idx] *= np.float32(50.0)
    return v


def dit(seed=0, M=4608, K=3072, N1=3072, N2=12288):
    rng = np.random.default_rng(seed)
    x = activations_bf16(rng, M, K)
    w1 = normal_bf16(rng, (N1, K), 0.02)
    w2 = normal_bf16(rng, (N2, K), 0.02)
    b1 = normal_bf16(rng, (N1,), 0.02)
    b2 = normal_bf16(rng, (N2,), 0.02)
    return {"x": x, "w1": w1, "w2": w2, "b1": b1, "b2": b2}


def svdq(seed=0, M=4096, K=3072, N=12288, r=32):
    rng = np.random.default_rng(seed)
    x = activations_bf16(rng, M, K)
    l1 = normal_bf16(rng, (r, K), 0.1)
    l2 = normal_bf16(rng, (N, r), 0.1)
    res = normal_bf16(rng, (N, K), 0.02)
    bias = normal_bf16(rng, (N,), 0.02)
    return {"x": x, "l1": l1, "l2": l2, "r": res, "bias": bias}


def fp8_step(seed=0, M=8192, K=3072, N=12288):
    rng = np.random.default_rng(seed)
    w = normal_bf16(rng, (N, K), 0.02)
    x = activations_bf16(rng, M, K, outliers=0)
    dy = normal_bf16(rng, (M, N), 1e-3)
    return {"w": w, "x": x, "dy": dy}


def random_rows(seed, M, K, std=1.0):
    """Generic N(0, std) bf16 matrix for edge-case shapes."""
    return normal_bf16(np.random.default_rng(seed), (M, K), std)


def q8_0_weight_blocks(rng, N, K, zero_rows=0):
    """A weight [N, K] as GGUF Q8_0 bytes (row n = K / 32 blocks of {f16 d, 32
    int8 codes}), drawn directly rather than quantized: per block a scale
    d = f16(0.02 * 3 / 127 * exp(N(0, 0.3))) and codes rint(N(0, 1) * 127 / 3)
    clipped to [-127, 127], with one code of each block set to +-127 (as a
    block's absmax element is).  The first `zero_rows` rows are all-zero codes.
    Returns uint8 [N * K / 32 * 34]."""
    assert K % 32 == 0
    nb = N * K // 32
    d = (0.02 * 3.0 / 127.0 * np.exp(rng.standard_normal(nb) * 0.3)).astype(np.float16)
    q = np.clip(np.rint(rng.standard_normal((nb, 32)) * (127.0 / 3.0)), -127, 127)
    pick = rng.integers(0, 32, nb)
    q[np.arange(nb), pick] = np.where(rng.random(nb) < 0.5, -127.0, 127.0)
    q = q.astype(np.int8)
    if zero_rows:
        q[: zero_rows * (K // 32)] = 0
    out = np.empty((nb, 34), np.uint8)
    out[:, :2] = d.view(np.uint8).reshape(nb, 2)
    out[:, 2:] = q.view(np.uint8)
    return out.ravel()


def gguf(seed=0, M=4096, K=3072, N=12288):
    rng = np.random.default_rng(seed)
    x = activations_bf16(rng, M, K)
    blocks = q8_0_weight_blocks(rng, N, K)
    bias = normal_bf16(rng, (N,), 0.02)
    return {"x": x, "w_blocks": blocks, "bias": bias, "N": N, "K": K}
