"""Host <-> device marshalling and comparison helpers for the GPU parity tests."""
import numpy as np
import torch

TOL_REL = 2.0 ** -7
TOL_ABS = 1e-3


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def codes_dev(codes, fp8):
    t = torch.from_numpy(np.ascontiguousarray(codes).view(np.int8)).cuda()
    return t.view(torch.float8_e4m3fn) if fp8 else t


def bf16_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bytes_host(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_bf16_close(got_bits, ref_bits, what=""):
    """|got - ref| <= 2^-7 |ref| + 1e-3 elementwise on bf16 values."""
    got = bf16_to_f64(got_bits)
    ref = bf16_to_f64(ref_bits)
    assert got.shape == ref.shape
    err = np.abs(got - ref)
    bound = TOL_REL * np.abs(ref) + TOL_ABS
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; first {i.tolist()} "
                             f"got {got[tuple(i.T)]} ref {ref[tuple(i.T)]}")
    return float((err / (np.abs(ref) + 1e-30)).max())


FROB_REL = 1e-3


def assert_frobenius(got_bits, ref_bits, what="", tol=FROB_REL):
    """Relative Frobenius error ||got - ref||_F / ||ref||_F <= tol in f64 (the
    bar of the e4m3 products, where both sides use identical e4m3 codes)."""
    got = bf16_to_f64(got_bits)
    ref = bf16_to_f64(ref_bits)
    assert got.shape == ref.shape
    den = float(np.sqrt(np.sum(ref * ref)))
    num = float(np.sqrt(np.sum((got - ref) ** 2)))
    rel = num / den if den > 0 else num
    assert rel <= tol, f"{what}: relative Frobenius error {rel:.3e} > {tol:g}"
    return rel


def assert_equal(got, ref, what=""):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {bad[:5].tolist()}: "
                             f"got {got[tuple(bad[:5].T)]} ref {ref[tuple(bad[:5].T)]}")


def sample_rows(M, n, seed=0, tile=256):
    """Rows spanning every tile boundary region: first, last, tile edges, random."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1}
    for t in range(0, M, tile):
        rows.update({t, min(t + tile - 1, M - 1)})
    rows = sorted(rows)
    extra = rng.choice(M, size=min(n, M), replace=False)
    return np.array(sorted(set(rows) | set(extra.tolist())))[: max(n, 1) + len(rows)]
