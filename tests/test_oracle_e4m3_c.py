"""The plain-C e4m3 cast of the oracle (oracle/e4m3_cast.c) pinned over every fp32 bit pattern:
against torch's CPU float8_e4m3fn conversion of the clamped product (an independent library
routine, round to nearest even; it does not saturate, hence the clamp to +-448 first), against the
numpy oracle's e4m3_round / e4m3_encode on every binade, and on its documented conventions for
NaN, infinities and signed zero."""
import numpy as np
import pytest
import torch

from oracle import e4m3_c
from oracle import numerics as nu

CHUNK = 1 << 26


def _torch_codes(x32: np.ndarray, scale: float) -> np.ndarray:
    p = x32 * np.float32(scale)                      # fp32 product, rounded once
    p = np.clip(p, np.float32(-448.0), np.float32(448.0))
    return torch.from_numpy(p).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("scale", [1.0])
def test_every_fp32_pattern_matches_torch_cast(scale):
    """All 2^32 patterns in chunks: the non-NaN ones equal torch's cast code for code, the NaN
    patterns all give 0x7F."""
    with np.errstate(over="ignore", invalid="ignore"):
        for first in range(0, 1 << 32, CHUNK):
            bits = np.arange(CHUNK, dtype=np.uint32) + np.uint32(first)
            x = bits.view(np.float32)
            got = e4m3_c.cast_patterns(first, CHUNK, scale)
            nan = np.isnan(x)
            ref = _torch_codes(x, scale)
            ok = np.where(nan, got == 0x7F, got == ref)
            if not ok.all():  # name the first pattern that differs
                i = int(np.flatnonzero(~ok)[0])
                raise AssertionError(f"pattern {int(bits[i]):#010x}: got {int(got[i]):#04x}, torch {int(ref[i]):#04x}")


@pytest.mark.parametrize("scale", [2.0 ** -7, 2.0 ** 5, 2.0 ** 40])
def test_scaled_patterns_match_torch_cast(scale):
    """Other power-of-two scales on every 61st pattern (products that overflow clamp to 448)."""
    bits = np.arange(0, (1 << 32) // 61, dtype=np.uint32) * np.uint32(61)
    x = bits.view(np.float32)
    got = e4m3_c.cast(x, scale)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = _torch_codes(x, scale)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.all(got[nan] == 0x7F)


def test_matches_numpy_oracle_on_every_binade():
    """Every fp32 exponent field, 1,024 mantissas each (ends of the binade included), both signs,
    against oracle.numerics (the float64 definition the layer's oracle uses)."""
    e = np.arange(0, 255, dtype=np.uint32)
    m = np.unique(np.concatenate([np.linspace(0, (1 << 23) - 1, 1021).astype(np.uint32),
                                  np.array([1, (1 << 22), (1 << 22) + 1], np.uint32)]))
    bits = ((e[:, None] << 23) | m[None, :]).ravel()
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    x = bits.view(np.float32)
    for scale in (1.0, 2.0 ** -3, 2.0 ** 9):
        with np.errstate(over="ignore"):
            y = np.clip(nu.f32(x.astype(np.float64) * scale), -448.0, 448.0)
        ref = nu.e4m3_encode(nu.e4m3_round(y))
        assert np.array_equal(e4m3_c.cast(x, scale), ref), scale


def test_conventions():
    x = np.array([np.nan, -np.nan, np.inf, -np.inf, 0.0, -0.0, 448.0, -448.0, 464.0, 1e30, 2.0 ** -10,
                  -(2.0 ** -10), 2.0 ** -10 * 1.0000001, 2.0 ** -9, 2.0 ** -6, 0.0068359375], np.float32)
    got = e4m3_c.cast(x, 1.0)
    # 2^-10 is half the smallest subnormal: a tie, to even (zero); just above it rounds up to 2^-9;
    # 0.0068359375 = 3.5 * 2^-9 ties to 4 * 2^-9
    assert list(got) == [0x7F, 0x7F, 0x7E, 0xFE, 0x00, 0x80, 0x7E, 0xFE, 0x7E, 0x7E, 0x00, 0x80, 0x01, 0x01,
                         0x08, 0x04]
    # a zero scale times an infinity is NaN
    assert e4m3_c.cast(np.array([np.inf, 1.0], np.float32), 0.0).tolist() == [0x7F, 0x00]
