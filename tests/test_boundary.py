"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments before launching anything.  Only
error paths and zero-size no-ops are called (they touch no device memory)."""
import ctypes

import pytest
import torch

import w8a8_quantized_linear_quant_amd as w8

lib = w8.library()
OK, INVALID, SHAPE, ALIGN, UNSUPPORTED, HIPERR, SCRATCH_LIMIT = range(7)
A = 1 << 20       # a 16-byte aligned fake address (never dereferenced)
MIS = A + 1       # misaligned by one byte
NULL = None


def test_exports_match_header():
    names = w8.exported_names_in_header()
    assert len(names) == 20
    probe = w8.exported_names_in_header(w8.PROBE_HEADER)
    assert probe == ["w8a8_probe_cvt_e4m3", "w8a8_probe_gemm_tile_n", "w8a8_probe_mfma_i8", "w8a8_probe_sink_count"]
    for n in names + probe:
        assert hasattr(lib, n), n


def test_probe_rejects():
    assert lib.w8a8_probe_cvt_e4m3(0, -1, A, NULL) == INVALID
    assert lib.w8a8_probe_cvt_e4m3(0, 4, NULL, NULL) == INVALID
    assert lib.w8a8_probe_cvt_e4m3(0xFFFFFFF0, 17, A, NULL) == INVALID   # past 2^32 bit patterns
    assert lib.w8a8_probe_cvt_e4m3(0, 4, MIS, NULL) == ALIGN
    assert lib.w8a8_probe_cvt_e4m3(0, 0, A, NULL) == OK
    assert lib.w8a8_probe_mfma_i8(NULL, A, 1, A, NULL) == INVALID
    assert lib.w8a8_probe_mfma_i8(A, A, -1, A, NULL) == INVALID
    assert lib.w8a8_probe_mfma_i8(MIS, A, 1, A, NULL) == ALIGN
    assert lib.w8a8_probe_mfma_i8(A, A, 0, A, NULL) == OK
    assert lib.w8a8_probe_gemm_tile_n(0, 3072) == 0
    assert lib.w8a8_probe_gemm_tile_n(8192, -1) == 0


def test_tile_width_model_on_256_cus():
    # without a device the library prices tile widths for 256 CUs
    if torch.cuda.is_available():
        pytest.skip("the GPU's own CU count decides; covered by the GPU tests")
    assert lib.w8a8_probe_gemm_tile_n(8192, 3072) == 192    # 384 tiles of 256: 1.5 rounds
    assert lib.w8a8_probe_gemm_tile_n(4349, 4100) == 192
    assert lib.w8a8_probe_gemm_tile_n(4096, 12288) == 256   # whole rounds
    assert lib.w8a8_probe_gemm_tile_n(4608, 3072) == 256    # one round
    assert lib.w8a8_probe_gemm_tile_n(1, 1) == 256


def test_status_strings():
    for code in range(7):
        assert lib.w8a8_status_str(code).decode().startswith("W8A8_")
    assert b"unknown" in lib.w8a8_status_str(99)


def test_sizes():
    assert lib.q8_0_nbytes(16_777_221) == 17_825_826
    assert lib.q8_0_nbytes(0) == 0 and lib.q8_0_nbytes(-1) == 0
    assert [lib.q8_0_nbytes(n) for n in (1, 31, 32, 33, 64, 65)] == [34, 34, 34, 68, 68, 102]
    assert lib.svdq_workspace_bytes(4096, 32) == 2 * 4096 * 32 * 2
    assert lib.svdq_workspace_bytes(10, 5) == 2 * 10 * 16 * 2
    assert lib.svdq_workspace_bytes(10, 0) == 0 and lib.svdq_workspace_bytes(10, 65) == 0
    assert lib.w8a8_weight_workspace_bytes(12288, 3072) > 0


def test_act_quant_rejects():
    f = lib.w8a8_quant_act_rowwise
    assert f(2, A, 4, 64, 64, A, 64, A, NULL) == INVALID           # bad qtype
    assert f(0, A, -1, 64, 64, A, 64, A, NULL) == INVALID          # negative M
    assert f(0, NULL, 4, 64, 64, A, 64, A, NULL) == INVALID        # null x
    assert f(0, A, 4, 64, 60, A, 64, A, NULL) == SHAPE             # ldx < K
    assert f(0, A, 4, 64, 68, A, 64, A, NULL) == SHAPE             # ldx % 8
    assert f(0, A, 4, 64, 64, A, 72, A, NULL) == SHAPE             # ldq % 16
    assert f(0, MIS, 4, 64, 64, A, 64, A, NULL) == ALIGN
    assert f(1, A, 4, 64, 64, A, 64, MIS, NULL) == ALIGN
    assert f(0, NULL, 0, 64, 64, NULL, 64, NULL, NULL) == OK       # M = 0: no-op
    big = (1 << 30) + 16
    assert f(0, A, 4, big, big, A, big, A, NULL) == SHAPE          # K > 2^30


def test_linear_rejects():
    f = lib.w8a8_linear
    assert f(0, A, A, A, A, NULL, 64, 64, 40, A, NULL) == SHAPE    # K % 16
    assert f(0, A, A, A, A, NULL, 64, 64, 0, A, NULL) == SHAPE     # K = 0
    assert f(0, A, A, A, A, NULL, -1, 64, 64, A, NULL) == INVALID
    assert f(0, NULL, A, A, A, NULL, 64, 64, 64, A, NULL) == INVALID
    assert f(0, A, NULL, A, A, NULL, 64, 64, 64, A, NULL) == INVALID
    assert f(0, MIS, A, A, A, NULL, 64, 64, 64, A, NULL) == ALIGN
    assert f(0, A, A, A, A, MIS, 64, 64, 64, A, NULL) == ALIGN     # misaligned bias
    assert f(7, A, A, A, A, NULL, 64, 64, 64, A, NULL) == INVALID
    assert f(0, A, A, A, A, NULL, 0, 64, 64, A, NULL) == OK        # M = 0: no-op
    assert f(1, A, A, A, A, NULL, 64, 0, 64, A, NULL) == OK        # N = 0: no-op
    g = lib.w8a8_gemm_i32
    assert g(A, A, 8, 8, 24, A, NULL) == SHAPE
    assert g(A, A, 8, 8, 32, MIS, NULL) == ALIGN
    b = lib.w8a8_linear_backward_dx
    assert b(1, A, A, A, A, 8, 24, 32, A, NULL) == SHAPE           # reduction N % 16
    # size limits: K <= 2^22 (the reduction), M, N <= 2^30
    assert f(0, A, A, A, A, NULL, 64, 64, (1 << 22) + 16, A, NULL) == SHAPE
    assert f(0, A, A, A, A, NULL, (1 << 30) + 1, 64, 64, A, NULL) == SHAPE
    assert f(0, A, A, A, A, NULL, 64, (1 << 30) + 1, 64, A, NULL) == SHAPE
    assert g(A, A, 8, 8, (1 << 22) + 16, A, NULL) == SHAPE
    assert b(0, A, A, A, A, 8, (1 << 22) + 16, 32, A, NULL) == SHAPE


def test_weight_quant_rejects():
    f = lib.w8a8_quant_weight_tensorwise
    assert f(0, A, 64, 60, A, NULL, A, A, NULL) == SHAPE           # K % 8
    assert f(0, A, 24, 64, A, A, A, A, NULL) == SHAPE              # transposed copy needs N % 16
    assert f(0, A, 64, 64, A, NULL, A, NULL, NULL) == INVALID      # no workspace
    assert f(0, A, 64, 64, MIS, NULL, A, A, NULL) == ALIGN
    assert f(3, A, 64, 64, A, NULL, A, A, NULL) == INVALID
    assert f(0, A, 1 << 21, 1 << 20, A, NULL, A, A, NULL) == SHAPE  # N * K = 2^41 > 2^40
    assert f(0, A, 8, (1 << 31) + 8, A, NULL, A, A, NULL) == SHAPE  # K > 2^31


def test_svdq_rejects():
    f = lib.svdq_linear
    args = lambda **kw: [kw.get("qt", 0), A, kw.get("M", 64), kw.get("K", 64), A, A, A, A, kw.get("r", 16),
                         NULL, kw.get("N", 64), A, A, A, kw.get("ws", A), NULL]
    assert f(*args(r=0)) == INVALID
    assert f(*args(r=65)) == INVALID
    assert f(*args(K=40)) == SHAPE
    assert f(*args(ws=None)) == INVALID
    assert f(*args(ws=MIS)) == ALIGN


def test_q8_0_rejects():
    assert lib.q8_0_quantize(A, -1, A, NULL) == INVALID
    assert lib.q8_0_quantize(NULL, 5, A, NULL) == INVALID
    assert lib.q8_0_quantize(MIS, 5, A, NULL) == ALIGN
    assert lib.q8_0_dequantize(A, 5, MIS, NULL) == ALIGN
    assert lib.q8_0_quantize(NULL, 0, NULL, NULL) == OK
    assert lib.q8_0_dequantize(NULL, 0, NULL, NULL) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        w8.w8a8_quant_act_rowwise(x)
    with pytest.raises(TypeError):
        w8.w8a8_quant_act_rowwise(x.float())
    with pytest.raises(ValueError):                      # neither INT8 nor FP8_E4M3
        w8.w8a8_quant_weight_tensorwise(x, qtype=5)


def test_gguf_a8_rejects():
    f = lib.gguf_a8_requant_q8_0
    assert f(2, A, 8, 64, A, A, NULL) == INVALID                    # bad qtype
    assert f(0, A, -1, 64, A, A, NULL) == INVALID
    assert f(0, A, 8, 48, A, A, NULL) == SHAPE                      # K % 32
    assert f(0, A, 1 << 20, 1 << 16, A, A, NULL) == SHAPE           # blocks >= 2 GB
    assert f(0, NULL, 8, 64, A, A, NULL) == INVALID                 # null blocks
    assert f(0, A, 8, 64, A, NULL, NULL) == INVALID                 # null scales
    assert f(0, MIS, 8, 64, A, A, NULL) == ALIGN
    assert f(1, A, 8, 64, A, MIS, NULL) == ALIGN
    assert f(0, NULL, 0, 64, NULL, NULL, NULL) == OK                # N = 0: no-op
    g = lib.gguf_a8_linear
    assert g(0, A, A, A, A, NULL, 64, 64, 40, A, NULL) == SHAPE     # K % 16
    assert g(0, A, A, A, NULL, NULL, 64, 64, 64, A, NULL) == INVALID
    assert g(0, A, A, A, MIS, NULL, 64, 64, 64, A, NULL) == ALIGN
    assert g(3, A, A, A, A, NULL, 64, 64, 64, A, NULL) == INVALID
    assert g(0, NULL, NULL, NULL, NULL, NULL, 0, 64, 64, NULL, NULL) == OK


def test_svdq_prepare_rejects_and_sizes():
    assert [lib.svdq_prepare_subspace(r) for r in (1, 16, 32, 48, 49, 64)] == [32, 32, 48, 64, 64, 64]
    assert lib.svdq_prepare_subspace(0) == 0 and lib.svdq_prepare_subspace(65) == 0
    assert lib.svdq_prepare_workspace_bytes(12288, 3072, 32) >= 2 * 12288 * 3072
    assert lib.svdq_prepare_workspace_bytes(8, 8, 0) == 0
    f = lib.svdq_prepare

    def args(N=64, K=64, r=8, it=2, w=A, om=A):
        return (w, N, K, r, om, it, A, A, A, A, A, NULL)

    assert f(*args(r=0)) == INVALID
    assert f(*args(r=65)) == INVALID
    assert f(*args(it=-1)) == INVALID
    assert f(*args(N=60)) == SHAPE                                  # N % 8
    assert f(*args(K=16, r=24)) == SHAPE                            # r > K
    assert f(*args(N=1 << 24, K=64)) == SHAPE                       # N < 2^24
    assert f(*args(w=NULL)) == INVALID
    assert f(*args(om=MIS)) == ALIGN


def test_hadamard_rejects():
    f = lib.w8a8_quant_act_rowwise_hadamard
    assert f(0, A, 4, 40, 40, A, 48, A, NULL) == SHAPE              # K % 16
    assert f(2, A, 4, 64, 64, A, 64, A, NULL) == INVALID
    assert f(0, MIS, 4, 64, 64, A, 64, A, NULL) == ALIGN
    assert f(0, NULL, 0, 64, 64, NULL, 64, NULL, NULL) == OK         # M = 0
    g = lib.w8a8_hadamard_rotate
    assert g(A, 4, 40, 40, A, 40, NULL) == SHAPE
    assert g(A, -1, 64, 64, A, 64, NULL) == INVALID
    assert g(A, 4, 64, 64, MIS, 64, NULL) == ALIGN
    assert g(NULL, 0, 64, 64, NULL, 64, NULL) == OK
    big = (1 << 30) + 16
    assert g(A, 4, big, big, A, big, NULL) == SHAPE                  # K > 2^30
    assert f(0, A, 4, big, big, A, big, A, NULL) == SHAPE


def test_svdq_noalloc_scratch_limit():
    """svdq_linear_noalloc rejects, before touching the device, a call whose
    u (2 M roundup(r, 16) bf16) exceeds the fixed scratch; M = 0 is a no-op."""
    import re
    with open(w8.HEADER) as f:
        m = re.search(r"#define W8A8_SVDQ_NOALLOC_SCRATCH_BYTES \((\d+) \* 1024 \* 1024\)", f.read())
    assert m and int(m.group(1)) << 20 == w8.SVDQ_NOALLOC_SCRATCH_BYTES
    f = lib.svdq_linear_noalloc
    K, N, r = 64, 64, 32
    over = w8.SVDQ_NOALLOC_SCRATCH_BYTES // (2 * 2 * 32) + 1            # one row too many at r = 32
    assert w8.svdq_workspace_bytes(over, r) > w8.SVDQ_NOALLOC_SCRATCH_BYTES
    assert f(0, A, over, K, A, A, A, A, r, NULL, N, A, A, A, NULL) == SCRATCH_LIMIT
    assert f(0, A, 70000, K, A, A, A, A, 17, NULL, N, A, A, A, NULL) == SCRATCH_LIMIT  # rp = 32
    assert f(0, A, 0, K, A, A, A, A, r, NULL, N, A, A, A, NULL) == OK
    # the shared argument checks come first
    assert f(0, A, 64, K, A, A, A, A, 65, NULL, N, A, A, A, NULL) == INVALID
    assert f(0, A, 64, 40, A, A, A, A, r, NULL, N, A, A, A, NULL) == SHAPE
    assert f(0, MIS, 64, K, A, A, A, A, r, NULL, N, A, A, A, NULL) == ALIGN
