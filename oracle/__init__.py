"""CPU oracle for the W8A8 quantized-linear path -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never links or calls it.  Every function
here is a thin numpy <-> ctypes marshaller around oracle/w8a8_oracle.c, which
holds all of the arithmetic (plain C, one rounding per named step); see that
file for the passages of the pages each function follows.

Arrays: bf16 and f16 travel as uint16 bit patterns, e4m3 codes as uint8, int8
codes as int8 (viewed as uint8 where the C side takes bytes).

oracle.svd_prep holds the SVDQuant weight preparation (numpy, float64).
"""
import ctypes
import os

import numpy as np

from .build import LIB, SRC, build_oracle

INT8 = 0
FP8_E4M3 = 1
Q8_0_BLOCK = 32
Q8_0_BYTES = 34

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # W8A8_ORACLE_LIB: another build of w8a8_oracle.c (the mutation tests load
    # deliberately broken copies through it to show that the pins catch them)
    path = os.environ.get("W8A8_ORACLE_LIB")
    if not path:
        path = LIB
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build_oracle()
    lib = ctypes.CDLL(path)
    P, I64, I, F, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
    sig = {
        "orc_bf16_to_f64": (D, [ctypes.c_uint16]),
        "orc_f16_to_f64": (D, [ctypes.c_uint16]),
        "orc_e4m3_to_f64": (D, [ctypes.c_uint8]),
        "orc_f64_to_bf16": (ctypes.c_uint16, [D]),
        "orc_f32_to_bf16": (ctypes.c_uint16, [F]),
        "orc_f64_to_f16": (ctypes.c_uint16, [D]),
        "orc_f32_to_f16": (ctypes.c_uint16, [F]),
        "orc_f64_to_e4m3": (ctypes.c_uint8, [D]),
        "orc_f32_to_e4m3": (ctypes.c_uint8, [F]),
        "orc_absmax_scale": (F, [F, F]),
        "orc_code_int8": (ctypes.c_int8, [F, F]),
        "orc_code_e4m3": (ctypes.c_uint8, [F, F]),
        "orc_quant_act_rowwise": (I, [I, P, I64, I64, I64, P, I64, P]),
        "orc_quant_weight_tensorwise": (I, [I, P, I64, I64, P, P, P]),
        "orc_gemm_i32": (I, [P, P, I64, I64, I64, P]),
        "orc_linear": (I, [I, P, P, P, F, P, I64, I64, I64, P]),
        "orc_linear_backward_dx": (I, [I, P, P, P, F, I64, I64, I64, P]),
        "orc_svdq_linear": (I, [I, P, I64, I64, P, F, P, P, I64, P, I64, P, P, P, P]),
        "orc_q8_0_nbytes": (I64, [I64]),
        "orc_q8_0_quantize": (I, [P, I64, P]),
        "orc_q8_0_dequantize": (I, [P, I64, P]),
        "orc_convert_array": (I, [I, P, I64, P]),
        "orc_gguf_a8_requant_q8_0": (I, [I, P, I64, I64, P, P, P]),
        "orc_linear_axiswise": (I, [I, P, P, P, P, P, I64, I64, I64, P]),
        "orc_hadamard_block": (I64, [I64]),
        "orc_hadamard_rows_f32": (I, [P, I64, I64, I64, P]),
        "orc_quant_act_rowwise_hadamard": (I, [I, P, I64, I64, I64, P, I64, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"oracle {name} rejected its arguments")


# ---------------------------------------------------------------- formats
_CONV = {  # name: (kind, input dtype, output dtype)
    "f32_to_bf16": (0, np.float32, np.uint16),
    "f64_to_bf16": (1, np.float64, np.uint16),
    "f32_to_f16": (2, np.float32, np.uint16),
    "f64_to_f16": (3, np.float64, np.uint16),
    "f32_to_e4m3": (4, np.float32, np.uint8),
    "f64_to_e4m3": (5, np.float64, np.uint8),
    "bf16_to_f64": (6, np.uint16, np.float64),
    "f16_to_f64": (7, np.uint16, np.float64),
    "e4m3_to_f64": (8, np.uint8, np.float64),
}


def _convert(name, values):
    kind, din, dout = _CONV[name]
    a = np.ascontiguousarray(np.asarray(values, dtype=din))
    out = np.empty(a.shape, dtype=dout)
    _check(_load().orc_convert_array(kind, _p(a), a.size, _p(out)), name)
    return out


def f32_to_bf16(v):
    return _convert("f32_to_bf16", v)


def f64_to_bf16(v):
    return _convert("f64_to_bf16", v)


def f32_to_f16(v):
    return _convert("f32_to_f16", v)


def f64_to_f16(v):
    return _convert("f64_to_f16", v)


def f32_to_e4m3(v):
    return _convert("f32_to_e4m3", v)


def f64_to_e4m3(v):
    return _convert("f64_to_e4m3", v)


def bf16_to_f64(b):
    return _convert("bf16_to_f64", b)


def f16_to_f64(h):
    return _convert("f16_to_f64", h)


def e4m3_to_f64(c):
    return _convert("e4m3_to_f64", c)


def code_int8(x, s):
    return int(_load().orc_code_int8(float(x), float(s)))


def code_e4m3(x, s):
    return int(_load().orc_code_e4m3(float(x), float(s)))


def absmax_scale(amax, qmax):
    return np.float32(_load().orc_absmax_scale(float(amax), float(qmax)))


# ---------------------------------------------------------------- quantizers
def quant_act_rowwise(qtype, x_bf16, ldq=None):
    """x_bf16: uint16 [M, K].  Returns (codes uint8 [M, ldq], scales f32 [M])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    ldq = K if ldq is None else ldq
    q = np.empty((M, ldq), np.uint8)
    s = np.empty(M, np.float32)
    _check(_load().orc_quant_act_rowwise(qtype, _p(x), M, K, K, _p(q), ldq, _p(s)), "quant_act_rowwise")
    return q, s


def quant_weight_tensorwise(qtype, w_bf16, transposed=False):
    """w_bf16: uint16 [N, K].  Returns (codes [N, K], codes^T [K, N] or None, scale f32)."""
    w = _c(w_bf16, np.uint16)
    N, K = w.shape
    q = np.empty((N, K), np.uint8)
    qt = np.empty((K, N), np.uint8) if transposed else None
    s = np.empty(1, np.float32)
    _check(_load().orc_quant_weight_tensorwise(qtype, _p(w), N, K, _p(q), _p(qt), _p(s)), "quant_weight")
    return q, qt, s[0]


# ---------------------------------------------------------------- products
def gemm_i32(xq, wq):
    xq = _c(xq, np.int8)
    wq = _c(wq, np.int8)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K
    acc = np.empty((M, N), np.int32)
    _check(_load().orc_gemm_i32(_p(xq), _p(wq), M, N, K, _p(acc)), "gemm_i32 (int32 overflow)")
    return acc


def linear(qtype, xq, sx, wq, sw, bias=None):
    """Dequantized 8-bit linear -> bf16 bits [M, N]."""
    xq = _c(np.asarray(xq).view(np.uint8), np.uint8)
    wq = _c(np.asarray(wq).view(np.uint8), np.uint8)
    sx = _c(sx, np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and sx.shape == (M,)
    b = None if bias is None else _c(bias, np.uint16)
    y = np.empty((M, N), np.uint16)
    _check(_load().orc_linear(qtype, _p(xq), _p(sx), _p(wq), float(sw), _p(b), M, N, K, _p(y)), "linear")
    return y


def linear_backward_dx(qtype, dyq, sdy, wq, sw):
    """dX = dY . W from quantized dY [M, N] and W codes [N, K] -> bf16 bits [M, K]."""
    dyq = _c(np.asarray(dyq).view(np.uint8), np.uint8)
    wq = _c(np.asarray(wq).view(np.uint8), np.uint8)
    sdy = _c(sdy, np.float32)
    M, N = dyq.shape
    K = wq.shape[1]
    assert wq.shape[0] == N
    dx = np.empty((M, K), np.uint16)
    _check(_load().orc_linear_backward_dx(qtype, _p(dyq), _p(sdy), _p(wq), float(sw), M, N, K, _p(dx)),
           "linear_backward_dx")
    return dx


def svdq_linear(qtype, x_bf16, rq, sr, l1, l2, bias=None):
    """Returns (y bf16 bits [M, N], xq [M, K], sx [M])."""
    x = _c(x_bf16, np.uint16)
    rq = _c(np.asarray(rq).view(np.uint8), np.uint8)
    l1 = _c(l1, np.uint16)
    l2 = _c(l2, np.uint16)
    M, K = x.shape
    N = rq.shape[0]
    r = l1.shape[0]
    assert l1.shape == (r, K) and l2.shape == (N, r) and rq.shape == (N, K)
    b = None if bias is None else _c(bias, np.uint16)
    y = np.empty((M, N), np.uint16)
    xq = np.empty((M, K), np.uint8)
    sx = np.empty(M, np.float32)
    u = np.empty(max(r, 1), np.float64)
    _check(_load().orc_svdq_linear(qtype, _p(x), M, K, _p(rq), float(sr), _p(l1), _p(l2), r, _p(b), N,
                                   _p(y), _p(xq), _p(sx), _p(u)), "svdq_linear")
    return y, xq, sx


# ---------------------------------------------------------------- Q8_0
def q8_0_nbytes(n):
    return int(_load().orc_q8_0_nbytes(int(n)))


def q8_0_quantize(x_f32):
    x = _c(x_f32, np.float32).ravel()
    out = np.empty(q8_0_nbytes(x.size), np.uint8)
    _check(_load().orc_q8_0_quantize(_p(x), x.size, _p(out)), "q8_0_quantize")
    return out


def q8_0_dequantize(blocks, n):
    b = _c(blocks, np.uint8)
    assert b.size >= q8_0_nbytes(n)
    y = np.empty(n, np.float32)
    _check(_load().orc_q8_0_dequantize(_p(b), n, _p(y)), "q8_0_dequantize")
    return y


# ---------------------------------------------------------------- GGUF A8
def gguf_a8_requant_q8_0(qtype, blocks, N, K):
    """Q8_0 weight [N, K] (K % 32 == 0; row n = K / 32 blocks) -> (codes [N, K], scales f32 [N])."""
    b = _c(blocks, np.uint8).ravel()
    assert K % Q8_0_BLOCK == 0 and b.size >= N * (K // Q8_0_BLOCK) * Q8_0_BYTES
    wq = np.empty((N, K), np.uint8)
    s = np.empty(N, np.float32)
    v = np.empty(max(K, 1), np.float32)
    _check(_load().orc_gguf_a8_requant_q8_0(qtype, _p(b), N, K, _p(wq), _p(s), _p(v)), "gguf_a8_requant_q8_0")
    return wq, s


def linear_axiswise(qtype, xq, sx, wq, sw, bias=None):
    """Dequantized 8-bit linear with per-output-channel weight scales sw [N] -> bf16 bits [M, N]."""
    xq = _c(np.asarray(xq).view(np.uint8), np.uint8)
    wq = _c(np.asarray(wq).view(np.uint8), np.uint8)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K and sx.shape == (M,) and sw.shape == (N,)
    b = None if bias is None else _c(bias, np.uint16)
    y = np.empty((M, N), np.uint16)
    _check(_load().orc_linear_axiswise(qtype, _p(xq), _p(sx), _p(wq), _p(sw), _p(b), M, N, K, _p(y)),
           "linear_axiswise")
    return y


# ---------------------------------------------------------------- Hadamard rotation
def hadamard_block(K):
    return int(_load().orc_hadamard_block(int(K)))


def hadamard_rows_f32(x_bf16):
    """Rotated rows (block-diagonal normalized Walsh-Hadamard along K), f32 [M, K]."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    out = np.empty((M, K), np.float32)
    _check(_load().orc_hadamard_rows_f32(_p(x), M, K, K, _p(out)), "hadamard_rows_f32")
    return out


def hadamard_rotate_bf16(x_bf16):
    """Rotated rows rounded to bf16 (the weight-side rotation) -> uint16 [M, K]."""
    return f32_to_bf16(hadamard_rows_f32(x_bf16))


def quant_act_rowwise_hadamard(qtype, x_bf16, ldq=None):
    """Row-wise quantization of the rotated rows.  Returns (codes [M, ldq], scales f32 [M])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    ldq = K if ldq is None else ldq
    q = np.empty((M, ldq), np.uint8)
    s = np.empty(M, np.float32)
    w = np.empty(max(K, 1), np.float32)
    _check(_load().orc_quant_act_rowwise_hadamard(qtype, _p(x), M, K, K, _p(q), ldq, _p(s), _p(w)),
           "quant_act_rowwise_hadamard")
    return q, s
