"""The Python binding refuses output, scale and workspace tensors that do not
fit before anything is launched (a too-small `out` would otherwise be written
past its end), and makes non-contiguous inputs contiguous."""
import numpy as np
import pytest
import torch

import workloads
from helpers import bf16_dev, bytes_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def w8():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import w8a8_quantized_linear_quant_amd as m
    return m


def _inputs(w8, M=64, N=96, K=128):
    rng = np.random.default_rng(3)
    x = bf16_dev(workloads.activations_bf16(rng, M, K, outliers=2))
    w = bf16_dev(workloads.normal_bf16(rng, (N, K), 0.02))
    xq, sx = w8.w8a8_quant_act_rowwise(x)
    wq, _, sw = w8.w8a8_quant_weight_tensorwise(w)
    torch.cuda.synchronize()
    return x, w, xq, sx, wq, sw


def test_outputs_of_the_wrong_shape_dtype_or_place(w8):
    print("[binding] output checks", flush=True)
    x, w, xq, sx, wq, sw = _inputs(w8)
    M, N = xq.shape[0], wq.shape[0]
    dev = xq.device
    with pytest.raises(ValueError):
        w8.w8a8_linear(xq, sx, wq, sw, out=torch.empty((M, N - 1), dtype=torch.bfloat16, device=dev))
    with pytest.raises(TypeError):
        w8.w8a8_linear(xq, sx, wq, sw, out=torch.empty((M, N), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        w8.w8a8_linear(xq, sx, wq, sw, out=torch.empty((M, N), dtype=torch.bfloat16))  # host memory
    with pytest.raises(ValueError):
        w8.w8a8_linear(xq, sx, wq, sw, out=torch.empty((N, M), dtype=torch.bfloat16, device=dev).t())
    with pytest.raises(ValueError):
        w8.w8a8_quant_act_rowwise(x, out=torch.empty((M, 64), dtype=torch.int8, device=dev))
    with pytest.raises(ValueError):
        w8.w8a8_quant_act_rowwise(x, scale=torch.empty(M - 1, dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        w8.q8_0_quantize(torch.zeros(100, device=dev), out=torch.empty(100, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        w8.w8a8_quant_weight_tensorwise(w, workspace=torch.empty(1, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        w8.gguf_a8_requant_q8_0(torch.zeros(33, dtype=torch.uint8, device=dev), 1, 32)  # 34 bytes needed


def test_scale_vectors_too_short(w8):
    print("[binding] scale and bias lengths", flush=True)
    x, w, xq, sx, wq, sw = _inputs(w8)
    with pytest.raises(ValueError):
        w8.w8a8_linear(xq, sx[:-1], wq, sw)
    with pytest.raises(ValueError):
        w8.w8a8_linear(xq, sx, wq, sw, bias=torch.zeros(wq.shape[0] - 1, dtype=torch.bfloat16, device=xq.device))
    with pytest.raises(ValueError):
        w8.gguf_a8_linear(xq, sx, wq, sw)      # per-channel scales: one is not enough
    with pytest.raises(TypeError):
        w8.w8a8_linear(xq, sx.double(), wq, sw)


def test_bad_qtype(w8):
    x, *_ = _inputs(w8)
    with pytest.raises(ValueError):
        w8.w8a8_quant_act_rowwise(x, qtype=2)


def test_non_contiguous_inputs_are_copied(w8):
    print("[binding] non-contiguous inputs", flush=True)
    x, w, xq, sx, wq, sw = _inputs(w8)
    y_ref = w8.w8a8_linear(xq, sx, wq, sw)
    wq_nc = torch.empty((wq.shape[1], wq.shape[0]), dtype=wq.dtype, device=wq.device).t()
    wq_nc.copy_(wq)
    assert not wq_nc.is_contiguous()
    y = w8.w8a8_linear(xq, sx, wq_nc, sw)
    torch.cuda.synchronize()
    assert np.array_equal(bytes_host(y), bytes_host(y_ref))
