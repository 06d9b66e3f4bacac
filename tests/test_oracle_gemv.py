"""Pins for the oracle's fp64 W8A16 GEMV (CPU only).

y = x . deq(W)^T is checked against numpy's float64 matmul on a weight
dequantized independently (torch's fp8 decode times the scale), against
closed forms (one-hot activations, constant codes), and the bound
|x| . |deq W|^T against the same matmul on absolute values.
"""
import math

import numpy as np
import pytest
import torch

from fp8_block_scaled_02_amd import workloads as W

TILE, GROUP = 128, 32


def f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def fp8_value(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def deq_block(codes, scales):
    n, k = codes.shape
    s = np.repeat(np.repeat(scales.astype(np.float64), TILE, 0), TILE, 1)[:n, :k]
    return fp8_value(codes) * s


def deq_mx(codes, e8m0):
    n, k = codes.shape
    e = np.repeat(e8m0.astype(np.int64) - 127, GROUP, axis=1)[:, :k]
    return fp8_value(codes) * np.ldexp(1.0, e)


def random_codes(rng, n, k):
    c = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E        # no NaN codes
    return c


@pytest.mark.parametrize("m", [1, 2, 8, 9, 16, 32])
@pytest.mark.parametrize("nk", [(128, 128), (130, 272), (257, 1008)])
def test_block_gemv_matches_numpy(oracle_mod, m, nk):
    n, k = nk
    rng = np.random.default_rng(m * 1000 + n)
    codes = random_codes(rng, n, k)
    scales = (rng.random(oracle_mod.block_scale_shape(n, k)) * 0.01 + 1e-4).astype(np.float32)
    x = W.activation(90, m, k)
    y, bound = oracle_mod.gemv_block_f64(x, codes, scales)
    deq = deq_block(codes, scales)
    xf = f32(x).astype(np.float64)
    np.testing.assert_allclose(y, xf @ deq.T, rtol=0, atol=1e-13 * bound.max())
    np.testing.assert_allclose(bound, np.abs(xf) @ np.abs(deq).T, rtol=1e-14)
    rows = np.array([n - 1, 0, n // 2])
    ys, bs = oracle_mod.gemv_block_f64(x, codes, scales, rows=rows)
    assert np.array_equal(ys, y[:, rows]) and np.array_equal(bs, bound[:, rows])


@pytest.mark.parametrize("m", [1, 8, 16])
def test_mx_gemv_matches_numpy(oracle_mod, m):
    n, k = 200, 1008
    rng = np.random.default_rng(m)
    codes = random_codes(rng, n, k)
    e8m0 = rng.integers(100, 140, size=oracle_mod.mx_scale_shape(n, k), dtype=np.uint8)
    x = W.activation(91, m, k)
    y, bound = oracle_mod.gemv_mx_f64(x, codes, e8m0)
    deq = deq_mx(codes, e8m0)
    xf = f32(x).astype(np.float64)
    np.testing.assert_allclose(y, xf @ deq.T, rtol=0, atol=1e-13 * bound.max())
    np.testing.assert_allclose(bound, np.abs(xf) @ np.abs(deq).T, rtol=1e-14)


def test_one_hot_activation_selects_a_dequantized_column(oracle_mod):
    n, k = 256, 384
    codes = np.tile(np.arange(256, dtype=np.uint8)[:, None], (1, k))
    codes[(codes & 0x7F) == 0x7F] = 0x00
    scales = np.full(oracle_mod.block_scale_shape(n, k), 0.5, np.float32)
    scales[1, 2] = 3.0
    for col in (0, 200, 383):
        x = np.zeros((1, k), np.uint16)
        x[0, col] = 0x3F80                      # bf16 1.0
        y, bound = oracle_mod.gemv_block_f64(x, codes, scales)
        expect = fp8_value(codes[:, col]) * np.repeat(scales[:, col // TILE], TILE)
        assert np.array_equal(y[0], expect) and np.array_equal(bound[0], np.abs(expect))


def test_constant_codes_reduce_to_a_sum(oracle_mod):
    """Every code 0x38 (= 1.0) with unit scales: y = sum_k x[k], exactly."""
    n, k = 130, 1024
    codes = np.full((n, k), 0x38, np.uint8)
    scales = np.ones(oracle_mod.block_scale_shape(n, k), np.float32)
    x = W.activation(92, 3, k)
    y, _ = oracle_mod.gemv_block_f64(x, codes, scales)
    xf = f32(x).astype(np.float64)
    for i in range(3):
        # bf16 activations of N(0, 1) sum exactly in fp64 over 1024 terms
        assert (y[i] == math.fsum(xf[i])).all()
    e8m0 = np.full(oracle_mod.mx_scale_shape(n, k), 127, np.uint8)
    ym, _ = oracle_mod.gemv_mx_f64(x, codes, e8m0)
    assert np.array_equal(ym, y)


def test_quantized_gemv_stays_within_round_trip_error(oracle_mod):
    """End to end on a config-1-like weight: y from the quantized weight is
    close to the bf16 weight's product (relative to |x| . |w|)."""
    bits = W.gaussian_weight(1, 0, 1024, 1024, outlier_rows=True)
    codes, scales = oracle_mod.quantize_block(bits)
    x = W.activation(1, 1, 1024)
    y, bound = oracle_mod.gemv_block_f64(x, codes, scales)
    wf = f32(bits).astype(np.float64)
    xf = f32(x).astype(np.float64)
    exact = xf @ wf.T
    assert (np.abs(y - exact) <= 2.0 ** -4 * (np.abs(xf) @ np.abs(wf).T)).all()
