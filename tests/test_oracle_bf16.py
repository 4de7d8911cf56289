"""The oracle's float32 -> bfloat16 rounding, pinned to torch's CPU conversion."""
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O


def torch_bf16_bits(a32):
    t = torch.from_numpy(np.ascontiguousarray(a32, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_round_trip_is_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_to_f32(bits)
    finite = np.isfinite(f)
    assert np.array_equal(O.f32_to_bf16(f[finite]), bits[finite])


def test_matches_torch_on_random_and_ties():
    rng = np.random.default_rng(0)
    a = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # exact ties: low 16 bits == 0x8000, both parities of the kept lsb
    hi = rng.integers(0, 1 << 16, size=50_000, dtype=np.uint32)
    hi = hi[(hi & 0x7F80) != 0x7F80]  # keep finite patterns
    ties = ((hi << 16) | 0x8000).view(np.float32)
    near = ((hi << 16) | rng.integers(0x7FF0, 0x8010, size=hi.size, dtype=np.uint32)).view(np.float32)
    wide = (rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)).view(np.float32)
    wide = wide[np.isfinite(wide)]
    for arr in (a, ties, near, wide):
        assert np.array_equal(O.f32_to_bf16(arr), torch_bf16_bits(arr))


def test_specials():
    vals = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                     3.4028235e38, 1e-40, -1e-40, 1.17549435e-38], np.float32)
    assert np.array_equal(O.f32_to_bf16(vals), torch_bf16_bits(vals))
    # overflow past the largest bf16 rounds to infinity
    assert O.f32_to_bf16(np.array([3.4028235e38], np.float32))[0] == 0x7F80


@pytest.mark.parametrize("pattern,expect", [
    (0x7FC00000, 0x7FC0),      # quiet NaN stays
    (0x7F800001, 0x7FC0),      # signalling NaN with payload only in the low bits -> quiet
    (0xFFA00000, 0xFFE0),      # negative signalling NaN keeps sign and payload, made quiet
])
def test_nan_is_quieted(pattern, expect):
    f = np.array([pattern], np.uint32).view(np.float32)
    assert O.f32_to_bf16(f)[0] == expect
