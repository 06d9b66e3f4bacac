"""GPU parity on seeded random shapes: every scale format, every route,
single calls and grouped launches, against the oracle's fp64 product
within the 2^-7 bound.

The shapes are drawn so that ragged N (not a multiple of 16 or 128),
ragged K (not a multiple of 128 or of the 256-column panel), K just above
and below the 3072- and 4096-column segment widths, and every M from 1 to
32 all occur; weights are the oracle's own quantization of seeded Gaussian
bf16 values (with outlier rows for the grid formats and heavy-tailed groups
for MX), so codes and scales are what the quantizers produce.  Sizes stay
small enough for the oracle to finish in seconds.
"""
import numpy as np
import pytest

from fp8_block_scaled_02_amd import workloads as W
from gpu_util import assert_within_bound, bf16_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

FORMATS = ("block", "mx", "block_bf16", "row", "tensor")
K_CHOICES = (16, 32, 48, 112, 240, 272, 496, 1008, 2048, 2304, 3056, 3072, 3088, 4096, 4112, 6160)


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


def _dev_scales(fmt, s):
    import torch
    t = to_dev(np.ascontiguousarray(s))
    return t.view(torch.bfloat16) if fmt == "block_bf16" else t


def _weight(oracle_mod, seed, n, k, fmt):
    bits = W.gaussian_weight(70, seed, n, k, outlier_rows=fmt != "mx", heavy_tail=fmt == "mx")
    return oracle_mod.quantize_format(bits, fmt)


def _case(rng):
    n = int(rng.integers(1, 700))
    k = int(rng.choice(K_CHOICES))
    m = int(rng.integers(1, 33))
    return n, k, m


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("seed", range(4))
def test_random_single_calls(fp8w, oracle_mod, fmt, seed):
    rng = np.random.default_rng([71, seed, FORMATS.index(fmt)])
    for i in range(6):
        n, k, m = _case(rng)
        c, s = _weight(oracle_mod, 1000 * seed + i, n, k, fmt)
        x = W.activation(72, m, k)
        routes = [0, fp8w.ROUTE_MFMA] + ([fp8w.ROUTE_VALU] if m <= 8 else [])
        dc, ds, dx = to_dev(c), _dev_scales(fmt, s), to_dev_bf16(x)
        ys = [fp8w.fp8w_gemv(dx, dc, ds, fmt, route=r) for r in routes]
        _sync()
        y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, fmt)
        for r, y in zip(routes, ys):
            assert_within_bound(bf16_to_f64(y), y_ref, bound, f"{fmt} [{n}x{k}] m={m} route={r}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("seed", range(3))
def test_random_grouped_launches(fp8w, oracle_mod, fmt, seed):
    rng = np.random.default_rng([73, seed, FORMATS.index(fmt)])
    m = int(rng.integers(1, 33))
    shapes = [_case(rng)[:2] for _ in range(int(rng.integers(2, 7)))]
    jobs = [(n, k) + _weight(oracle_mod, 100 * seed + i, n, k, fmt) for i, (n, k) in enumerate(shapes)]
    xs = [W.activation(74, m, k) for (_, k, _, _) in jobs]
    routes = [0, fp8w.ROUTE_MFMA] + ([fp8w.ROUTE_VALU] if m <= 8 else [])
    for r in routes:
        plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs], [to_dev(c) for (_, _, c, _) in jobs],
                                           [_dev_scales(fmt, s) for (_, _, _, s) in jobs], fmt=fmt, route=r)
        ys = fp8w.fp8w_gemv_grouped(plan)
        _sync()
        for (n, k, c, s), x, y in zip(jobs, xs, ys):
            y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, fmt)
            assert_within_bound(bf16_to_f64(y), y_ref, bound, f"grouped {fmt} [{n}x{k}] m={m} route={r}")
