"""Pins of the oracle's bf16 rounding and bf16 dequantizers (CPU).

The oracle rounds by a binary search over bf16 patterns; these tests check
it against torch's float32 -> bfloat16 cast (round to nearest even) and
numpy float32 arithmetic, which share nothing with it, and against closed
forms: exact values stay exact, ties go to the even pattern, overflow gives
infinity, and the decoded codes are exact in bf16.
"""
import numpy as np
import pytest
import torch


def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _decode_torch(codes: np.ndarray) -> np.ndarray:
    """float32 values of e4m3fn codes through torch's float8 type."""
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn) \
        .to(torch.float32).numpy()


def test_round_bf16_matches_torch_cast_on_random_fp32(oracle_mod):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2**32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    assert np.array_equal(oracle_mod.round_bf16(f.astype(np.float64)), _torch_bf16_bits(f))


def test_round_bf16_ties_overflow_and_subnormals(oracle_mod):
    # every midpoint between two adjacent non-negative bf16 values: ties to even
    lo = np.arange(0, 0x7F7F, dtype=np.uint32)
    mid = ((lo << 16) | 0x8000).view(np.float32)
    got = oracle_mod.round_bf16(mid.astype(np.float64))
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    assert np.array_equal(oracle_mod.round_bf16(-mid[:1000].astype(np.float64)), want[:1000] | 0x8000)
    top = float(np.ldexp(1.0, 128))
    mx = float(np.uint32(0x7F7F0000).view(np.float32))
    assert oracle_mod.round_bf16([mx, (mx + top) / 2, top, 1e300])[0] == 0x7F7F
    assert list(oracle_mod.round_bf16([(mx + top) / 2, top, 1e300])) == [0x7F80] * 3
    assert list(oracle_mod.round_bf16([np.nextafter((mx + top) / 2, 0)])) == [0x7F7F]
    tiny = np.ldexp(1.0, -133)   # smallest bf16 subnormal
    assert list(oracle_mod.round_bf16([tiny, tiny / 2, 1.5 * tiny, 0.75 * tiny, -0.0])) == [1, 0, 2, 1, 0x8000]


def test_every_code_is_exact_in_bf16(oracle_mod):
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8).reshape(1, -1)
    ones = np.ones(oracle_mod.block_scale_shape(*codes.shape), dtype=np.float32)
    got = oracle_mod.dequant_block_bf16(codes, ones)
    exact = oracle_mod.e4m3_decode(codes)
    back = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(back, exact)


def test_dequant_block_bf16_matches_float32_multiply_then_torch_cast(oracle_mod):
    rng = np.random.default_rng(12)
    n, k = 300, 1000   # ragged in both directions
    codes = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E
    # scales over many binades, including fp32 subnormals and powers of two
    s = np.ldexp(rng.uniform(1, 2, size=oracle_mod.block_scale_shape(n, k)),
                 rng.integers(-140, 100, size=oracle_mod.block_scale_shape(n, k))).astype(np.float32)
    s.flat[0] = 1.0
    s.flat[1] = np.float32(2.0 ** -140)
    got = oracle_mod.dequant_block_bf16(codes, s)
    grid = np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)[:n, :k]
    want = _torch_bf16_bits(_decode_torch(codes) * grid)   # float32 multiply, then RNE to bf16
    assert np.array_equal(got, want)


def test_dequant_mx_bf16_every_code_times_every_scale_byte(oracle_mod):
    codes = np.tile(np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8), (255, 1))
    codes = np.repeat(codes, 32, axis=1)   # one 32-group per code
    e8m0 = np.repeat(np.arange(255, dtype=np.uint8)[:, None], codes.shape[1] // 32, axis=1)
    got = oracle_mod.dequant_mx_bf16(codes, e8m0)
    pow2 = np.ldexp(np.float32(1.0), e8m0.astype(np.int32) - 127).astype(np.float32)
    with np.errstate(over="ignore"):   # codes near 448 times 2^127 overflow to infinity
        want = _torch_bf16_bits(_decode_torch(codes) * np.repeat(pow2, 32, axis=1))
    assert np.array_equal(got, want)


def test_dequant_bf16_against_the_exact_dequant(oracle_mod):
    from fp8_block_scaled_02_amd import workloads as W
    bits = W.gaussian_weight(20, 0, 256, 384, outlier_rows=True, heavy_tail=False)
    codes, scales = oracle_mod.quantize_block(bits)
    exact = oracle_mod.dequant_block(codes, scales)
    got = (oracle_mod.dequant_block_bf16(codes, scales).astype(np.uint32) << 16).view(np.float32)
    err = np.abs(got.astype(np.float64) - exact)
    assert np.all(err <= np.ldexp(np.abs(exact), -8) * (1 + 2.0 ** -15))
    codes, e8m0 = oracle_mod.quantize_mx(bits)
    exact = oracle_mod.dequant_mx(codes, e8m0)
    got = (oracle_mod.dequant_mx_bf16(codes, e8m0).astype(np.uint32) << 16).view(np.float32)
    # 4 significant bits times a power of two: exact in bf16 (normal range)
    assert np.array_equal(got.astype(np.float64), exact)


@pytest.mark.parametrize("fn", ["dequant_block_bf16", "dequant_mx_bf16"])
def test_dequant_bf16_rejects_bad_shapes(oracle_mod, fn):
    codes = np.zeros((4, 40), dtype=np.uint8)
    with pytest.raises(ValueError):
        getattr(oracle_mod, fn)(codes, np.zeros((3, 3), dtype=np.float32 if "block" in fn else np.uint8))
