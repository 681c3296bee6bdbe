"""MI355X (gfx950) W8A8 quantized linear: Python binding of libw8a8.so.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
the shared library (C ABI in include/w8a8.h); torch provides device memory and
the current stream.  The functions carry the C names:

  w8a8_quant_weight_tensorwise  tensor-wise int8 / e4m3 weight quantization
  w8a8_quant_act_rowwise        row-wise (token-wise) activation quantization
  w8a8_quant_act_rowwise_hadamard   the same on Hadamard-rotated rows
  w8a8_hadamard_rotate          rows rotated by the block Walsh-Hadamard matrix -> bf16
  w8a8_linear                   8-bit product + fused dequant epilogue -> bf16
  w8a8_linear_backward_dx       dX = dY . W from quantized dY and W^T codes
  w8a8_gemm_i32                 raw int32 accumulators (test export)
  svdq_linear                   residual 8-bit product + bf16 low-rank branch
  svdq_linear_noalloc           the same with its workspace in a fixed per-GPU scratch (allocates nothing)
  svdq_prepare                  W -> bf16 low-rank pair (truncated SVD) + bf16 residual
  q8_0_quantize / q8_0_dequantize / q8_0_nbytes   GGUF Q8_0 blocks
  gguf_a8_requant_q8_0          Q8_0 weight -> int8 / e4m3 codes, one scale per output channel
  gguf_a8_linear                8-bit product with per-channel weight scales -> bf16
  probe_mfma_i8                 diagnostic: sustained int8 MFMA loop (include/w8a8_probe.h)
  probe_cvt_e4m3                diagnostic: the hardware e4m3 conversion on consecutive f32 bit patterns
  probe_gemm_tile_n             diagnostic: the tile width along N w8a8_linear picks for an M x N output

Codes are torch.int8 (int8) or torch.float8_e4m3fn (e4m3); bf16 tensors are
torch.bfloat16; scales are float32.  Output tensors may be passed in (`out=`)
or are allocated on the input's device.  Nothing falls back to the CPU: if the
library is missing, importing this package raises.
"""
import ctypes
import os
import re

import torch

from .build import LIB as _LIB_PATH

INT8 = 0
FP8_E4M3 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
HEADER = os.path.join(os.path.dirname(_HERE), "include", "w8a8.h")
PROBE_HEADER = os.path.join(os.path.dirname(_HERE), "include", "w8a8_probe.h")


class W8A8Error(RuntimeError):
    """A non-OK status returned by the library."""


def _load_library():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python -m w8a8_quantized_linear_quant_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    sigs = {
        "w8a8_status_str": (ctypes.c_char_p, [I]),
        "w8a8_weight_workspace_bytes": (ctypes.c_size_t, [I64, I64]),
        "w8a8_quant_weight_tensorwise": (I, [I, P, I64, I64, P, P, P, P, P]),
        "w8a8_quant_act_rowwise": (I, [I, P, I64, I64, I64, P, I64, P, P]),
        "w8a8_linear": (I, [I, P, P, P, P, P, I64, I64, I64, P, P]),
        "w8a8_linear_backward_dx": (I, [I, P, P, P, P, I64, I64, I64, P, P]),
        "w8a8_gemm_i32": (I, [P, P, I64, I64, I64, P, P]),
        "svdq_workspace_bytes": (ctypes.c_size_t, [I64, I64]),
        "svdq_linear": (I, [I, P, I64, I64, P, P, P, P, I64, P, I64, P, P, P, P, P]),
        "svdq_linear_noalloc": (I, [I, P, I64, I64, P, P, P, P, I64, P, I64, P, P, P, P]),
        "q8_0_nbytes": (ctypes.c_size_t, [I64]),
        "q8_0_quantize": (I, [P, I64, P, P]),
        "q8_0_dequantize": (I, [P, I64, P, P]),
        "gguf_a8_requant_q8_0": (I, [I, P, I64, I64, P, P, P]),
        "gguf_a8_linear": (I, [I, P, P, P, P, P, I64, I64, I64, P, P]),
        "svdq_prepare_subspace": (I64, [I64]),
        "svdq_prepare_workspace_bytes": (ctypes.c_size_t, [I64, I64, I64]),
        "svdq_prepare": (I, [P, I64, I64, I64, P, I, P, P, P, P, P, P]),
        "w8a8_quant_act_rowwise_hadamard": (I, [I, P, I64, I64, I64, P, I64, P, P]),
        "w8a8_hadamard_rotate": (I, [P, I64, I64, I64, P, I64, P]),
        "w8a8_probe_sink_count": (I64, []),
        "w8a8_probe_mfma_i8": (I, [P, P, I64, P, P]),
        "w8a8_probe_cvt_e4m3": (I, [ctypes.c_uint32, I64, P, P]),
        "w8a8_probe_gemm_tile_n": (I, [I64, I64]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load_library()


def exported_names_in_header(path=HEADER):
    """Function names the C header declares (used to check the exports)."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)   # preprocessor lines
    return sorted(set(re.findall(r"\b([A-Za-z_][A-Za-z0-9_]*)\s*\(", text)) -
                  {"if", "defined", "sizeof", "extern"})


def library():
    return _lib


def _check(status):
    if status != 0:
        raise W8A8Error(_lib.w8a8_status_str(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _qtype_of(codes):
    if codes.dtype == torch.int8:
        return INT8
    if codes.dtype == torch.float8_e4m3fn:
        return FP8_E4M3
    raise TypeError(f"codes must be torch.int8 or torch.float8_e4m3fn, got {codes.dtype}")


def _code_dtype(qtype):
    if qtype not in (INT8, FP8_E4M3):
        raise ValueError(f"qtype must be INT8 ({INT8}) or FP8_E4M3 ({FP8_E4M3}), got {qtype}")
    return torch.int8 if qtype == INT8 else torch.float8_e4m3fn


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _arg(t, dtype, name, device, min_numel=0):
    """An input tensor: dtype (None: any), on `device`, at least `min_numel`
    elements; returned contiguous (a copy only if it was not)."""
    _need(t, dtype, name)
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {min_numel}")
    return t.contiguous()


def _out(t, shape, dtype, device, name):
    """An output of exactly `shape`: allocated if None, else checked (dtype,
    device, shape, contiguous): the kernels write every element of it."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _need(t, dtype, name)
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the operands on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _buf(t, numel, dtype, device, name, alloc=None):
    """A flat output or workspace of at least `numel` elements: allocated
    (`alloc` elements, default numel) if None, else checked."""
    if t is None:
        return torch.empty(max(numel, alloc or 0, 1), dtype=dtype, device=device)
    _need(t, dtype, name)
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the operands on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs at least {numel}")
    return t


def _mat(t, name):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got {t.dim()}-D")
    return t


# ------------------------------------------------------------------ weights
def w8a8_weight_workspace_bytes(N, K):
    return int(_lib.w8a8_weight_workspace_bytes(N, K))


def w8a8_quant_weight_tensorwise(w, qtype=INT8, transposed=False, out=None, out_t=None, scale=None,
                                 workspace=None):
    """w: bf16 [N, K].  Returns (codes [N, K], codes^T [K, N] or None, scale f32 [1])."""
    cd = _code_dtype(qtype)
    _need(w, torch.bfloat16, "w")
    dev = w.device
    w = _mat(_arg(w, torch.bfloat16, "w", dev), "w")
    N, K = w.shape
    wq = _out(out, (N, K), cd, dev, "out")
    wq_t = _out(out_t, (K, N), cd, dev, "out_t") if (transposed or out_t is not None) else None
    s = _buf(scale, 1, torch.float32, dev, "scale", alloc=4)
    ws = _buf(workspace, w8a8_weight_workspace_bytes(N, K), torch.uint8, dev, "workspace")
    _check(_lib.w8a8_quant_weight_tensorwise(qtype, _ptr(w), N, K, _ptr(wq), _ptr(wq_t), _ptr(s), _ptr(ws),
                                             _stream(dev)))
    return wq, wq_t, s[:1]


# -------------------------------------------------------------- activations
def w8a8_quant_act_rowwise(x, qtype=INT8, ldq=None, out=None, scale=None):
    """x: bf16 [M, K] (row stride may exceed K).  Returns (codes [M, ldq], scales f32 [M])."""
    cd = _code_dtype(qtype)
    _need(x, torch.bfloat16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    ldx = x.stride(0)
    if M > 0 and (ldx % 8 != 0 or x.data_ptr() % 16 != 0):
        # no hidden copy: rows must start on 16-byte boundaries
        raise ValueError(f"x rows must start on 16-byte boundaries (row stride {ldx} must be a multiple of 8, "
                         "data 16-byte aligned); pass a [:, :K] view of a buffer with padded rows")
    if M > 0 and x.untyped_storage().nbytes() - 2 * x.storage_offset() < 2 * M * ldx:
        raise ValueError(f"x's storage must span M * row stride = {M * ldx} elements")
    ldq = ldq if ldq is not None else K + (-K) % 16
    dev = x.device
    xq = _out(out, (M, ldq), cd, dev, "out")
    s = _buf(scale, M, torch.float32, dev, "scale")
    _check(_lib.w8a8_quant_act_rowwise(qtype, _ptr(x), M, K, ldx, _ptr(xq), ldq, _ptr(s), _stream(dev)))
    return xq, s[:M]


def w8a8_quant_act_rowwise_hadamard(x, qtype=INT8, ldq=None, out=None, scale=None):
    """x: bf16 [M, K], K % 16 == 0.  Codes [M, ldq] and scales [M] of the Hadamard-rotated rows."""
    cd = _code_dtype(qtype)
    _need(x, torch.bfloat16, "x")
    dev = x.device
    x = _mat(_arg(x, torch.bfloat16, "x", dev), "x")
    M, K = x.shape
    ldq = ldq if ldq is not None else K
    xq = _out(out, (M, ldq), cd, dev, "out")
    s = _buf(scale, M, torch.float32, dev, "scale")
    _check(_lib.w8a8_quant_act_rowwise_hadamard(qtype, _ptr(x), M, K, K, _ptr(xq), ldq, _ptr(s), _stream(dev)))
    return xq, s[:M]


def w8a8_hadamard_rotate(x, out=None):
    """x: bf16 [M, K], K % 16 == 0 -> bf16 [M, K] rotated rows."""
    _need(x, torch.bfloat16, "x")
    dev = x.device
    x = _mat(_arg(x, torch.bfloat16, "x", dev), "x")
    M, K = x.shape
    y = _out(out, (M, K), torch.bfloat16, dev, "out")
    _check(_lib.w8a8_hadamard_rotate(_ptr(x), M, K, K, _ptr(y), K, _stream(dev)))
    return y


# --------------------------------------------------------------- the linear
def _product_args(xq, x_scale, wq, w_scale, w_scale_numel, bias):
    qt = _qtype_of(xq)
    if wq.dtype != xq.dtype:
        raise TypeError("xq and wq must hold the same code type")
    _need(xq, None, "xq")
    dev = xq.device
    xq = _mat(_arg(xq, None, "xq", dev), "xq")
    wq = _mat(_arg(wq, None, "wq", dev), "wq")
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("xq and wq must share K")
    x_scale = _arg(x_scale, torch.float32, "x_scale", dev, M)
    w_scale = _arg(w_scale, torch.float32, "w_scale", dev, w_scale_numel(N))
    if bias is not None:
        bias = _arg(bias, torch.bfloat16, "bias", dev, N)
    return qt, dev, xq, x_scale, wq, w_scale, bias, M, N, K


def w8a8_linear(xq, x_scale, wq, w_scale, bias=None, out=None):
    """Dequantized 8-bit linear.  xq [M, K], wq [N, K] codes (same dtype) -> bf16 [M, N]."""
    qt, dev, xq, x_scale, wq, w_scale, bias, M, N, K = _product_args(xq, x_scale, wq, w_scale, lambda n: 1, bias)
    y = _out(out, (M, N), torch.bfloat16, dev, "out")
    _check(_lib.w8a8_linear(qt, _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), _ptr(bias), M, N, K, _ptr(y),
                            _stream(dev)))
    return y


def w8a8_linear_backward_dx(dyq, dy_scale, wq_t, w_scale, out=None):
    """dX = dY . W.  dyq [M, N] codes, wq_t [K, N] transposed weight codes -> bf16 [M, K]."""
    qt = _qtype_of(dyq)
    if wq_t.dtype != dyq.dtype:
        raise TypeError("dyq and wq_t must hold the same code type")
    _need(dyq, None, "dyq")
    dev = dyq.device
    dyq = _mat(_arg(dyq, None, "dyq", dev), "dyq")
    wq_t = _mat(_arg(wq_t, None, "wq_t", dev), "wq_t")
    M, N = dyq.shape
    K = wq_t.shape[0]
    if wq_t.shape[1] != N:
        raise ValueError("dyq and wq_t must share N")
    dy_scale = _arg(dy_scale, torch.float32, "dy_scale", dev, M)
    w_scale = _arg(w_scale, torch.float32, "w_scale", dev, 1)
    dx = _out(out, (M, K), torch.bfloat16, dev, "out")
    _check(_lib.w8a8_linear_backward_dx(qt, _ptr(dyq), _ptr(dy_scale), _ptr(wq_t), _ptr(w_scale), M, N, K,
                                        _ptr(dx), _stream(dev)))
    return dx


def w8a8_gemm_i32(xq, wq, out=None):
    """Raw int32 accumulators of the int8 product: xq [M, K] @ wq[N, K]^T."""
    _need(xq, torch.int8, "xq")
    dev = xq.device
    xq = _mat(_arg(xq, torch.int8, "xq", dev), "xq")
    wq = _mat(_arg(wq, torch.int8, "wq", dev), "wq")
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("xq and wq must share K")
    acc = _out(out, (M, N), torch.int32, dev, "out")
    _check(_lib.w8a8_gemm_i32(_ptr(xq), _ptr(wq), M, N, K, _ptr(acc), _stream(dev)))
    return acc


# ------------------------------------------------------------------ SVDQuant
def svdq_workspace_bytes(M, r):
    return int(_lib.svdq_workspace_bytes(M, r))


def _svdq_args(x, rq, r_scale, l1, l2, bias, out, xq_out, x_scale_out):
    qt = _qtype_of(rq)
    _need(x, torch.bfloat16, "x")
    dev = x.device
    x = _mat(_arg(x, torch.bfloat16, "x", dev), "x")
    rq = _mat(_arg(rq, None, "rq", dev), "rq")
    l1 = _mat(_arg(l1, torch.bfloat16, "l1", dev), "l1")
    l2 = _mat(_arg(l2, torch.bfloat16, "l2", dev), "l2")
    M, K = x.shape
    N = rq.shape[0]
    r = l1.shape[0]
    if rq.shape[1] != K or l1.shape[1] != K:
        raise ValueError("x, rq and l1 must share K")
    if tuple(l2.shape) != (N, r):
        raise ValueError(f"l2 must be [N, r] = [{N}, {r}], got {tuple(l2.shape)}")
    r_scale = _arg(r_scale, torch.float32, "r_scale", dev, 1)
    if bias is not None:
        bias = _arg(bias, torch.bfloat16, "bias", dev, N)
    y = _out(out, (M, N), torch.bfloat16, dev, "out")
    xq = _out(xq_out, (M, K), rq.dtype, dev, "xq_out")
    sx = _buf(x_scale_out, M, torch.float32, dev, "x_scale_out")
    return qt, dev, x, rq, r_scale, l1, l2, bias, M, N, K, r, y, xq, sx


def svdq_linear(x, rq, r_scale, l1, l2, bias=None, out=None, xq_out=None, x_scale_out=None, workspace=None):
    """x bf16 [M, K]; rq residual codes [N, K]; l1 bf16 [r, K]; l2 bf16 [N, r].
    Returns (y bf16 [M, N], xq [M, K], x_scale [M])."""
    qt, dev, x, rq, r_scale, l1, l2, bias, M, N, K, r, y, xq, sx = _svdq_args(x, rq, r_scale, l1, l2, bias, out,
                                                                             xq_out, x_scale_out)
    ws = _buf(workspace, svdq_workspace_bytes(M, r), torch.uint8, dev, "workspace", alloc=16)
    _check(_lib.svdq_linear(qt, _ptr(x), M, K, _ptr(rq), _ptr(r_scale), _ptr(l1), _ptr(l2), r, _ptr(bias), N,
                            _ptr(y), _ptr(xq), _ptr(sx), _ptr(ws), _stream(dev)))
    return y, xq, sx[:M]


def svdq_linear_noalloc(x, rq, r_scale, l1, l2, bias=None, out=None, xq_out=None, x_scale_out=None):
    """svdq_linear with its workspace in the library's fixed per-GPU scratch
    (W8A8_SVDQ_NOALLOC_SCRATCH_BYTES): the C call allocates nothing.  Pass
    `out`, `xq_out` and `x_scale_out` to allocate nothing here either."""
    qt, dev, x, rq, r_scale, l1, l2, bias, M, N, K, r, y, xq, sx = _svdq_args(x, rq, r_scale, l1, l2, bias, out,
                                                                             xq_out, x_scale_out)
    _check(_lib.svdq_linear_noalloc(qt, _ptr(x), M, K, _ptr(rq), _ptr(r_scale), _ptr(l1), _ptr(l2), r, _ptr(bias),
                                    N, _ptr(y), _ptr(xq), _ptr(sx), _stream(dev)))
    return y, xq, sx[:M]


SVDQ_NOALLOC_SCRATCH_BYTES = 4 * 1024 * 1024


def svdq_prepare_subspace(r):
    return int(_lib.svdq_prepare_subspace(r))


def svdq_prepare_workspace_bytes(N, K, r):
    return int(_lib.svdq_prepare_workspace_bytes(N, K, r))


def svdq_prepare(w, r, omega, iters=2, l1=None, l2=None, residual=None, sigma=None, workspace=None):
    """w bf16 [N, K]; omega bf16 [svdq_prepare_subspace(r), K] (Gaussian).
    Returns (l1 bf16 [r, K], l2 bf16 [N, r], residual bf16 [N, K], sigma f32 [r])."""
    _need(w, torch.bfloat16, "w")
    dev = w.device
    w = _mat(_arg(w, torch.bfloat16, "w", dev), "w")
    omega = _arg(omega, torch.bfloat16, "omega", dev)
    N, K = w.shape
    if tuple(omega.shape) != (svdq_prepare_subspace(r), K):
        raise ValueError("omega must be [svdq_prepare_subspace(r), K]")
    l1 = _out(l1, (r, K), torch.bfloat16, dev, "l1")
    l2 = _out(l2, (N, r), torch.bfloat16, dev, "l2")
    res = _out(residual, (N, K), torch.bfloat16, dev, "residual")
    sg = _buf(sigma, r, torch.float32, dev, "sigma", alloc=4)
    ws = _buf(workspace, svdq_prepare_workspace_bytes(N, K, r), torch.uint8, dev, "workspace", alloc=16)
    _check(_lib.svdq_prepare(_ptr(w), N, K, r, _ptr(omega), iters, _ptr(l1), _ptr(l2), _ptr(res),
                             _ptr(sg), _ptr(ws), _stream(dev)))
    return l1, l2, res, sg[:r]


# ---------------------------------------------------------------------- Q8_0
def q8_0_nbytes(n):
    return int(_lib.q8_0_nbytes(n))


def q8_0_quantize(x, out=None):
    """x f32 (any shape, contiguous) -> uint8 [q8_0_nbytes(x.numel())] GGUF Q8_0 blocks."""
    _need(x, torch.float32, "x")
    dev = x.device
    x = _arg(x, torch.float32, "x", dev)
    n = x.numel()
    blocks = _buf(out, q8_0_nbytes(n), torch.uint8, dev, "out", alloc=16)
    _check(_lib.q8_0_quantize(_ptr(x), n, _ptr(blocks), _stream(dev)))
    return blocks[:q8_0_nbytes(n)]


def q8_0_dequantize(blocks, n, out=None):
    """blocks uint8 (>= q8_0_nbytes(n) bytes) -> f32 [n]."""
    _need(blocks, torch.uint8, "blocks")
    dev = blocks.device
    blocks = _arg(blocks, torch.uint8, "blocks", dev, q8_0_nbytes(n))
    y = _buf(out, n, torch.float32, dev, "out", alloc=4)
    _check(_lib.q8_0_dequantize(_ptr(blocks), n, _ptr(y), _stream(dev)))
    return y[:n]


# ------------------------------------------------------------------- GGUF A8
def gguf_a8_requant_q8_0(blocks, N, K, qtype=INT8, out=None, scale=None):
    """Q8_0 weight [N, K] (uint8 blocks, row n = K / 32 blocks) -> (codes [N, K], scales f32 [N])."""
    cd = _code_dtype(qtype)
    _need(blocks, torch.uint8, "blocks")
    dev = blocks.device
    blocks = _arg(blocks, torch.uint8, "blocks", dev, q8_0_nbytes(N * K) if K % 32 == 0 else 0)
    wq = _out(out, (N, K), cd, dev, "out")
    s = _buf(scale, N, torch.float32, dev, "scale", alloc=4)
    _check(_lib.gguf_a8_requant_q8_0(qtype, _ptr(blocks), N, K, _ptr(wq), _ptr(s), _stream(dev)))
    return wq, s[:N]


def gguf_a8_linear(xq, x_scale, wq, w_scale, bias=None, out=None):
    """8-bit linear with per-output-channel weight scales w_scale f32 [N] -> bf16 [M, N]."""
    qt, dev, xq, x_scale, wq, w_scale, bias, M, N, K = _product_args(xq, x_scale, wq, w_scale, lambda n: n, bias)
    y = _out(out, (M, N), torch.bfloat16, dev, "out")
    _check(_lib.gguf_a8_linear(qt, _ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), _ptr(bias), M, N, K, _ptr(y),
                               _stream(dev)))
    return y


# ---------------------------------------------------------------- diagnostics
def probe_mfma_i8(a, b, pairs, sink=None):
    """Sustained int8 MFMA loop on operand bytes `a`, `b` (device tensors of at
    least 65536 bytes each): `pairs` iterations of 64 v_mfma_i32_16x16x64_i8
    per wave, one workgroup of 4 waves per CU.  Returns the sink tensor; the
    integer operations are pairs * 32 * 2 * 32**3 * 4 * CUs."""
    import torch
    for t in (a, b):
        if t.numel() * t.element_size() < 65536 or not t.is_contiguous():
            raise ValueError("probe operands: contiguous, at least 65536 bytes")
    n = _lib.w8a8_probe_sink_count()
    sink = _buf(sink, n, torch.int32, a.device, "sink")
    _check(_lib.w8a8_probe_mfma_i8(_ptr(a), _ptr(b), int(pairs), _ptr(sink), _stream(a.device)))
    return sink


def probe_cvt_e4m3(first_bits, n, out=None, device=None):
    """e4m3 codes (uint8 [n], on the GPU) of the f32 values with bit patterns
    first_bits, first_bits + 1, ..., by the quantizers' clamp and conversion."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    codes = _buf(out, n, torch.uint8, dev, "out", alloc=16)
    _check(_lib.w8a8_probe_cvt_e4m3(ctypes.c_uint32(first_bits), n, _ptr(codes), _stream(dev)))
    return codes[:n]


def probe_gemm_tile_n(M, N):
    """Tile width along N (256 or 192) that w8a8_linear and
    w8a8_linear_backward_dx take for an M x N output on the current device."""
    return int(_lib.w8a8_probe_gemm_tile_n(int(M), int(N)))
