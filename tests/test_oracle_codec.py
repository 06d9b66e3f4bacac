"""Pins for the oracle's e4m3fn codec (CPU only).

The oracle's decoder is checked against torch's independent float8_e4m3fn
implementation and the OCP OFP8 specification's anchor values; its encoder
against a brute-force nearest-value search (ties to the even code) written
here in numpy, and against torch's cast on a large set of fp32 bit patterns.
"""
import numpy as np
import pytest
import torch

from pagevalues import page_values


def torch_decode(codes: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(q: np.ndarray) -> np.ndarray:
    """torch's RNE cast, after clamping to the largest finite magnitude."""
    t = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def brute_force_encode(q: np.ndarray) -> np.ndarray:
    """Nearest finite e4m3fn value by exhaustive search, ties to the even code."""
    mags = torch_decode(np.arange(127, dtype=np.uint8))          # codes 0x00..0x7E
    # Above 448 every distance a - m shifts by the same amount, so clipping
    # keeps the nearest value and keeps the fp64 differences exact.
    a = np.minimum(np.abs(q.astype(np.float64)), 1024.0)[:, None]
    dist = np.abs(a - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    tied = dist == best
    even = tied & (np.arange(127)[None, :] % 2 == 0)
    code = np.where(even.any(axis=1), even.argmax(axis=1), tied.argmax(axis=1))
    return (code | (np.signbit(q).astype(np.int64) << 7)).astype(np.uint8)


def test_decode_all_256_codes_match_torch(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_mod.e4m3_decode(codes)
    ref = torch_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(np.flatnonzero(nan), [0x7F, 0xFF])
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_decode_anchor_values_of_the_ofp8_spec(oracle_mod):
    d = lambda c: float(oracle_mod.e4m3_decode(np.array([c], np.uint8))[0])
    assert d(0x7E) == page_values()["e4m3_max"] == 448.0
    assert d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9          # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9      # largest subnormal
    assert d(0x08) == 2.0 ** -6          # smallest normal
    assert d(0x38) == 1.0
    assert d(0x00) == 0.0 and not np.signbit(d(0x00))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))


def test_encode_every_bf16_pattern_against_brute_force(oracle_mod):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    q = (bits.astype(np.uint32) << 16).view(np.float32)
    q = q[np.isfinite(q)]
    assert np.array_equal(oracle_mod.e4m3_encode(q), brute_force_encode(q))


def test_midpoints_tie_to_even_and_neighbours_round_away(oracle_mod):
    mags = torch_decode(np.arange(127, dtype=np.uint8))
    mids = (0.5 * (mags[:-1] + mags[1:])).astype(np.float32)   # exact in fp32
    assert np.array_equal(mids.astype(np.float64), 0.5 * (mags[:-1] + mags[1:]))
    up = np.nextafter(mids, np.float32(np.inf))
    down = np.nextafter(mids, np.float32(0))
    lower = np.arange(126)
    expect_mid = np.where(lower % 2 == 0, lower, lower + 1)
    for sign in (1.0, -1.0):
        s = 0x80 if sign < 0 else 0
        assert np.array_equal(oracle_mod.e4m3_encode(sign * mids), (expect_mid | s).astype(np.uint8))
        assert np.array_equal(oracle_mod.e4m3_encode(sign * up), ((lower + 1) | s).astype(np.uint8))
        assert np.array_equal(oracle_mod.e4m3_encode(sign * down), (lower | s).astype(np.uint8))


def test_saturation_and_signed_zero(oracle_mod):
    big = np.array([448, 448.5, 449, 463.9, 464, 470, 480, 1e30, np.finfo(np.float32).max],
                   dtype=np.float32)
    assert (oracle_mod.e4m3_encode(big) == 0x7E).all()
    assert (oracle_mod.e4m3_encode(-big) == 0xFE).all()
    tiny = np.array([0.0, 1e-9, 2.0 ** -10, 2.0 ** -149], dtype=np.float32)
    assert (oracle_mod.e4m3_encode(tiny) == 0x00).all()
    assert (oracle_mod.e4m3_encode(-tiny) == 0x80).all()
    # anchors of round-to-nearest-even around 1 and the subnormal range
    q = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 15 * 2.0 ** -10], np.float32)
    assert list(oracle_mod.e4m3_encode(q)) == [0x38, 0x3A, 0x00, 0x02, 0x08]


@pytest.mark.slow
def test_encode_all_fp32_patterns_of_the_live_range_match_torch(oracle_mod):
    """Every fp32 with |q| in [2^-11, 2^9) (both signs), chunked."""
    lo, hi = (127 - 11) << 23, (127 + 9) << 23
    step = 1 << 24
    for start in range(lo, hi, step):
        u = np.arange(start, min(hi, start + step), dtype=np.uint32)
        q = u.view(np.float32)
        ours = oracle_mod.e4m3_encode(q)
        assert np.array_equal(ours, torch_encode(q)), hex(start)
        assert np.array_equal(oracle_mod.e4m3_encode(-q), ours | 0x80)


def test_encode_random_fp32_patterns_match_torch(oracle_mod):
    rng = np.random.default_rng(7)
    u = rng.integers(0, 2 ** 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    q = u.view(np.float32)
    q = q[np.isfinite(q)]
    assert np.array_equal(oracle_mod.e4m3_encode(q), torch_encode(q))
