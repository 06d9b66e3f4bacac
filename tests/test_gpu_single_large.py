"""GPU parity of single GEMV calls on weights with many rows, which run on
the wide VALU tiles (the streaming kernel at m = 1 with K <= 3072, one job
passed by value) and on the streaming MFMA kernel with one job, and of the
single-call MFMA kernel on either side of its 4- / 8-wave split.

Ragged N (not a multiple of 16 or 128) and ragged K (not a multiple of the
256-column panel), every scale format, the AUTO route and both forced
routes.  Codes and scales are seeded random inputs (finite codes, scales of
the format's kind), so the oracle only runs the GEMV, on sampled rows that
include both ends of the weight and the tile boundaries.
"""
import numpy as np
import pytest

from fp8_block_scaled_02_amd import workloads as W
from gpu_util import assert_within_bound, bf16_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

FORMATS = ("block", "mx", "block_bf16", "row", "tensor")


@pytest.fixture(scope="module")
def fp8w():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import fp8_block_scaled_02_amd as F
    F.lib()
    return F


def _sync():
    import torch
    torch.cuda.synchronize()


def _codes(rng, n, k):
    c = rng.integers(0, 256, size=(n, k), dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] -= 1   # no NaN codes: 0x7F -> 0x7E, 0xFF -> 0xFE
    return c


def _scales(oracle_mod, rng, fmt, n, k):
    shape = oracle_mod.scale_shape(fmt, n, k)
    if fmt == "mx":
        return rng.integers(117, 131, size=shape, dtype=np.uint8)
    v = np.ldexp(rng.uniform(1.0, 2.0, size=shape), rng.integers(-12, -2, size=shape)).astype(np.float32)
    if fmt == "block_bf16":
        return (v.view(np.uint32) >> 16).astype(np.uint16)
    return v


def _dev_scales(fmt, s):
    import torch
    t = to_dev(np.ascontiguousarray(s))
    return t.view(torch.bfloat16) if fmt == "block_bf16" else t


def _rows(n, rng):
    edges = {0, 1, 15, 16, 127, 128, n - 2, n - 1, n // 16 * 16 - 1, n // 16 * 16,
             n // 128 * 128 - 1, n // 128 * 128}
    rows = {r for r in edges if 0 <= r < n}
    rows.update(int(r) for r in rng.choice(n, size=40, replace=False))
    return np.array(sorted(rows), dtype=np.int64)


@pytest.fixture(scope="module")
def weights(fp8w, oracle_mod):
    """One ragged weight per (n, k) and format, on the device and the host."""
    cache = {}

    def get(n, k, fmt):
        key = (n, k, fmt)
        if key not in cache:
            rng = np.random.default_rng([n, k, FORMATS.index(fmt)])
            c = _codes(rng, n, k)
            s = _scales(oracle_mod, rng, fmt, n, k)
            cache.clear()   # keep one weight alive at a time
            cache[key] = (c, s, to_dev(c), _dev_scales(fmt, s))
        return cache[key]
    return get


def _check(fp8w, oracle_mod, weights, n, k, m, fmt, route):
    c, s, dc, ds = weights(n, k, fmt)
    x = W.activation(90, m, k)
    y = fp8w.fp8w_gemv(to_dev_bf16(x), dc, ds, fmt, route=route)
    _sync()
    rows = _rows(n, np.random.default_rng([n, m, route]))
    y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, fmt, rows=rows)
    assert_within_bound(bf16_to_f64(y)[:, rows], y_ref, bound, f"n={n} k={k} m={m} {fmt} route={route}")


# VALU: m = 1 with K <= 3072 takes the streaming kernel, one job by value
# (MX: only when n * ceil(k/32) % 4 == 0 -- K = 2048 here; K = 2064 with
# n = 16405 takes the wide per-tile kernel)
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("k", [2064, 2048])
def test_valu_stream_single_job(fp8w, oracle_mod, weights, fmt, k):
    _check(fp8w, oracle_mod, weights, 16405, k, 1, fmt, 0)


# M = 1 single calls below 16384 rows with K <= 4096 run the one-wave kernel:
# one row per wave up to 4096 rows, two above (an odd N leaves a wave's
# second row past the end), for every chunk count K <= 1024 * C, C = 1..4
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("n", [4095, 4096, 4097, 16383])
@pytest.mark.parametrize("k", [1008, 2048, 3056, 4096])
def test_rows_kernel_either_side_of_the_row_split(fp8w, oracle_mod, weights, fmt, n, k):
    _check(fp8w, oracle_mod, weights, n, k, 1, fmt, 0)


# the same kernel with two to four activation rows held in registers: two
# rows per wave up to 4096 rows, four above, K <= 3072 (K = 3088 and 4096
# take the LDS-staging kernel); forced VALU, as AUTO sends some to MFMA
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("n", [4095, 4097, 16383])
@pytest.mark.parametrize("k", [1008, 2048, 3056, 3072, 3088, 4096])
@pytest.mark.parametrize("m", [2, 3, 4])
def test_rows_kernel_several_activation_rows(fp8w, oracle_mod, weights, fmt, n, k, m):
    import fp8_block_scaled_02_amd as F
    _check(fp8w, oracle_mod, weights, n, k, m, fmt, F.ROUTE_VALU)


# VALU wide tiles without streaming: K above the streaming limit (m = 1:
# 4096-column K segments at K = 4096 and 8176, 3072-column ones at 4112),
# m = 2 and 3 (AUTO) and forced VALU up to m = 8
@pytest.mark.parametrize("fmt", ("block", "mx", "row"))
@pytest.mark.parametrize("m,k", [(1, 4112), (1, 4096), (1, 8176), (2, 2064), (3, 1040), (8, 4112)])
def test_valu_wide_single_call(fp8w, oracle_mod, weights, fmt, m, k):
    import fp8_block_scaled_02_amd as F
    _check(fp8w, oracle_mod, weights, 16405, k, m, fmt, F.ROUTE_VALU if m > 2 else 0)


# MFMA: the streaming kernel with one job from 32768 rows, and from 16384
# rows when m > 16; m = 16 at 16405 rows stays on the single-call kernel
# (forced MFMA: AUTO takes VALU at m = 3 outside MX; the same as AUTO above)
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("n,m", [(32813, 3), (32813, 9), (32813, 16), (32813, 17), (32813, 32),
                                 (16405, 16), (16405, 17), (16405, 32)])
def test_mfma_stream_single_job(fp8w, oracle_mod, weights, fmt, n, m):
    import fp8_block_scaled_02_amd as F
    _check(fp8w, oracle_mod, weights, n, 1040, m, fmt, F.ROUTE_MFMA)


# AUTO at m = 3 on many rows: the VALU wide tiles outside MX, the streaming
# MFMA kernel with MX
@pytest.mark.parametrize("fmt", FORMATS)
def test_auto_m3_many_rows(fp8w, oracle_mod, weights, fmt):
    _check(fp8w, oracle_mod, weights, 32813, 1040, 3, fmt, 0)


# forced MFMA at m = 1 and 2 on the streaming kernel, K over several
# LDS segments at m = 32 (K = 4112 at 2 bytes x 32 rows)
@pytest.mark.parametrize("fmt", ("block", "mx"))
@pytest.mark.parametrize("m,k", [(1, 2064), (2, 1040), (32, 4112)])
def test_mfma_stream_single_job_forced(fp8w, oracle_mod, weights, fmt, m, k):
    import fp8_block_scaled_02_amd as F
    _check(fp8w, oracle_mod, weights, 32813, k, m, fmt, F.ROUTE_MFMA)


# MX exponents at an odd address: the single call leaves the streaming
# kernel (which reads them as aligned dwords) for the wide VALU tiles
@pytest.mark.parametrize("m", [1, 17])
def test_mx_single_call_misaligned_exponents(fp8w, oracle_mod, weights, m):
    import torch
    n, k = 16405, 2064
    c, s, dc, ds = weights(n, k, "mx")
    buf = torch.zeros(s.size + 1, dtype=torch.uint8, device="cuda")
    buf[1:].copy_(ds.reshape(-1))
    x = W.activation(91, m, k)
    y = fp8w.fp8w_gemv(to_dev_bf16(x), dc, buf[1:].view(s.shape), "mx")
    _sync()
    rows = _rows(n, np.random.default_rng([n, m, 7]))
    y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, "mx", rows=rows)
    assert_within_bound(bf16_to_f64(y)[:, rows], y_ref, bound, f"misaligned mx m={m}")


# W8A8 at m <= 2 on many rows: the wide VALU tiles with the activation codes
# widened to bf16 while x is staged.  dec(codes) is exact in bf16, so the
# bf16 reference on the decoded codes, times the activation scale, applies.
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("m", [1, 2])
def test_w8a8_small_m_many_rows(fp8w, oracle_mod, weights, fmt, m):
    n, k = 16405, 2064
    c, s, dc, ds = weights(n, k, fmt)
    x = W.activation(92, m, k)
    xc, xs = oracle_mod.quantize_act_tensor(x)
    y = fp8w.fp8w_gemv_w8a8(to_dev(xc), to_dev(np.array([xs], np.float32)), dc, ds, fmt)
    _sync()
    rows = _rows(n, np.random.default_rng([n, m, 8]))
    xb = (oracle_mod.e4m3_decode(xc).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y_ref, bound = oracle_mod.gemv_format_f64(xb, c, s, fmt, rows=rows)
    assert_within_bound(bf16_to_f64(y)[:, rows], xs * y_ref, xs * bound, f"w8a8 {fmt} m={m}")


# W8A8 from m = 9 on many rows: 128-row tiles with the x codes staged in LDS
# (from 32768 rows, and from 16384 rows when m > 16); K = 4112 at m = 32 spans
# several x segments.  m = 3 on many rows stays on the 16-row tiles.
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("n,m,k", [(32813, 3, 1040), (32813, 9, 2064), (32813, 16, 1040), (32813, 17, 1040),
                                   (32813, 32, 4112), (16405, 17, 2064), (16405, 32, 1040)])
def test_w8a8_tiles_many_rows(fp8w, oracle_mod, weights, fmt, n, m, k):
    c, s, dc, ds = weights(n, k, fmt)
    x = W.activation(93, m, k)
    xc, xs = oracle_mod.quantize_act_tensor(x)
    y = fp8w.fp8w_gemv_w8a8(to_dev(xc), to_dev(np.array([xs], np.float32)), dc, ds, fmt)
    _sync()
    rows = _rows(n, np.random.default_rng([n, m, 9]))
    xb = (oracle_mod.e4m3_decode(xc).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y_ref, bound = oracle_mod.gemv_format_f64(xb, c, s, fmt, rows=rows)
    assert_within_bound(bf16_to_f64(y)[:, rows], xs * y_ref, xs * bound, f"w8a8 tiles {fmt} m={m} [{n}x{k}]")


# MFMA single calls on either side of the 8-wave split: N <= 4096 rows take
# 8 waves per 16-row tile, more rows take 4; m over both MFMA tile widths
@pytest.mark.parametrize("fmt", ("block", "mx"))
@pytest.mark.parametrize("n", [4096, 4112])
@pytest.mark.parametrize("m", [3, 16, 17, 32])
def test_mfma_direct_wave_split(fp8w, oracle_mod, weights, fmt, n, m):
    _check(fp8w, oracle_mod, weights, n, 2320, m, fmt, 0)


# MX single calls whose exponent rows start 8-byte aligned (K = 2304: 72
# groups) read 8 exponents per load: the per-tile MFMA kernel on both sides
# of its wave split and the streaming one (32813 rows)
@pytest.mark.parametrize("n", [4096, 4112, 32813])
@pytest.mark.parametrize("m", [3, 17, 32])
def test_mx_packed_exponents_single(fp8w, oracle_mod, weights, n, m):
    _check(fp8w, oracle_mod, weights, n, 2304, m, "mx", 0)


# W8A8 single calls on either side of the same split (m >= 3 on fewer rows
# than the 128-row W8A8 tiles take)
@pytest.mark.parametrize("fmt", ("block", "mx"))
@pytest.mark.parametrize("n", [4096, 4112])
@pytest.mark.parametrize("m", [3, 16, 17, 32])
def test_w8a8_direct_wave_split(fp8w, oracle_mod, weights, fmt, n, m):
    k = 2320
    c, s, dc, ds = weights(n, k, fmt)
    x = W.activation(94, m, k)
    xc, xs = oracle_mod.quantize_act_tensor(x)
    y = fp8w.fp8w_gemv_w8a8(to_dev(xc), to_dev(np.array([xs], np.float32)), dc, ds, fmt)
    _sync()
    rows = _rows(n, np.random.default_rng([n, m, 10]))
    xb = (oracle_mod.e4m3_decode(xc).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y_ref, bound = oracle_mod.gemv_format_f64(xb, c, s, fmt, rows=rows)
    assert_within_bound(bf16_to_f64(y)[:, rows], xs * y_ref, xs * bound, f"w8a8 direct {fmt} m={m} [{n}x{k}]")


# Single calls at M = 1 with 4096 < K <= 16384 on fewer than 16384 rows (one
# row per wave, K walked in 4096-column segments, ragged last segment, rows
# past the end of a 4-row workgroup), in every non-MX scale format.
@pytest.mark.parametrize("fmt", ("block", "block_bf16", "row", "tensor"))
@pytest.mark.parametrize("n,k", [(1, 4112), (5, 5008), (129, 8176), (300, 12288), (17, 16384), (4099, 9232)])
def test_long_k_single_call_m1(fp8w, oracle_mod, fmt, n, k):
    import torch
    bits = W.gaussian_weight(61, n % 7, n, k, outlier_rows=True)
    c, s = oracle_mod.quantize_format(bits, fmt)
    x = W.activation(62, 1, k)
    sd = to_dev(np.ascontiguousarray(s))
    if fmt == "block_bf16":
        sd = sd.view(torch.bfloat16)
    y = fp8w.fp8w_gemv(to_dev_bf16(x), to_dev(c), sd, fmt)
    torch.cuda.synchronize()
    y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, fmt)
    assert_within_bound(bf16_to_f64(y), y_ref, bound, f"long-K single {fmt} [{n}x{k}]")
