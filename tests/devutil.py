"""Host <-> device helpers and comparisons for the GPU parity tests."""
import numpy as np
import torch


def to_dev(a, dtype, dev="cuda:0"):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host(t, dtype):
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a, dtype):
    a = np.asarray(a)
    if dtype == "bf16":
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def bf16_ulp(ref_bits):
    """Spacing of bf16 numbers at each reference value (2^(e-7); subnormals 2^-133)."""
    e = ((np.asarray(ref_bits, np.uint16).astype(np.int64) >> 7) & 0xFF)
    e = np.maximum(e, 1)
    return np.ldexp(1.0, (e - 127 - 7).astype(np.int64))


def assert_rows_close(got, ref, dtype, what):
    """The acceptance bar: f32 max-abs <= 1e-6, bf16 within 1 bf16 ulp of the oracle."""
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    g, r = as_f64(got, dtype), as_f64(ref, dtype)
    if dtype == "f32":
        err = np.abs(g - r)
        assert np.all(err <= 1e-6), f"{what}: max abs err {err.max():.3e} > 1e-6"
    else:
        ulp = bf16_ulp(ref)
        bad = np.abs(g - r) > ulp
        assert not bad.any(), f"{what}: {int(bad.sum())} elements beyond 1 bf16 ulp"


def assert_f32_close(got, ref, what, tol=1e-6):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    assert np.all(err <= tol), f"{what}: max abs err {err.max():.3e} > {tol}"


def n_diff(got, ref):
    return int(np.sum(np.asarray(got) != np.asarray(ref)))
