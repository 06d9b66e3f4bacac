"""GPU parity of the MFMA kernels' panel walk against the CPU oracle.

The streaming MFMA kernel walks a tile's panels rotated (each workgroup from
its own x segment, each wave from its own panel of it) on jobs whose K is a
multiple of 2048 with x segments of at least four panels, and in plain order
otherwise; a run of tiles ends after a whole group of pipeline slots, so a
run whose panel count is odd consumes one dead panel past its last tile.  The
direct single-call kernels rotate their panel assignment by workgroup on the
same K.  Up to 16 rows x is staged in one buffer (x whole where it fits,
else segments restaged behind barriers); above, by one-panel segments in two
buffers, the next segment (of the tile, the next tile or the next job)
prefetched while the current one is in use.  Every kernel is compiled per
scale format.  The cases below mix rotated and plain jobs in one grouped
launch, cover 16-, 8- and 5-panel segments (M = 3 / 9 / 16) and one-panel
segments (M = 17..32), jobs whose x fits one segment next to jobs that need
several, launches whose x fits whole (restaged at job changes), force every
run length,
run single calls on both kernels and on the fp8 x fp8 direct kernel, in
every scale format.
"""
import numpy as np
import pytest

from fp8_block_scaled_02_amd import workloads as W
from gpu_util import assert_within_bound, bf16_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

FORMATS = ["block", "mx", "block_bf16", "row", "tensor"]
# rotated (K = 2048, 4096, 6144, 8192) and plain (K = 2560; K = 4112: 17
# panels, the last one partial, so runs can end on an odd panel count) jobs
SHAPES = [(300, 2048), (1030, 4096), (129, 8192), (257, 2560), (200, 4112), (384, 6144)]


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


def _quantized(oracle_mod, fmt, shapes, seed):
    out = []
    for i, (n, k) in enumerate(shapes):
        bits = W.gaussian_weight(seed, i, n, k, outlier_rows=True, heavy_tail=fmt == "mx")
        c, s = oracle_mod.quantize_format(bits, fmt)
        out.append((n, k, c, s))
    return out


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("m", [3, 9, 16, 17, 32])
def test_grouped_walk_every_run_length(fp8w, oracle_mod, fmt, m):
    jobs = _quantized(oracle_mod, fmt, SHAPES, 140)
    xs = [W.activation(141, m, k) for (_, k, _, _) in jobs]
    plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs], [to_dev(c) for (_, _, c, _) in jobs],
                                       [_dev_scales(fmt, s) for (_, _, _, s) in jobs], fmt=fmt,
                                       route=fp8w.ROUTE_MFMA)
    assert plan.route == fp8w.ROUTE_MFMA and plan.plan.tiles_per_block > 0
    seg = plan.plan.seg_cols
    assert seg % 256 == 0 and seg == {3: 4096, 9: 2048, 16: 1280, 17: 256, 32: 256}[m]
    tiles = plan.plan.tiles
    refs = [oracle_mod.gemv_format_f64(x, c, s, fmt) for x, (_, _, c, s) in zip(xs, jobs)]
    for run in (1, 2, 5, tiles):
        plan.plan.tiles_per_block = run
        plan.plan.blocks = -(-tiles // run)
        for y in plan.ys:
            y.fill_(float("nan"))
        ys = fp8w.fp8w_gemv_grouped(plan)
        _sync()
        for (n, k, _, _), (y_ref, bound), y in zip(jobs, refs, ys):
            assert_within_bound(bf16_to_f64(y), y_ref, bound, f"walk {fmt} m={m} run={run} [{n}x{k}] seg={seg}")


# x of every job whole in one buffer (m * K * 2 bytes within the one-buffer
# budget): x is restaged only where a run enters the next job
ONE_BUFFER = {8: [(300, 2048), (257, 2560), (200, 1040), (129, 2048)],
              12: [(300, 1024), (130, 784), (257, 512), (64, 1024)]}


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("m", sorted(ONE_BUFFER))
def test_grouped_one_buffer_every_run_length(fp8w, oracle_mod, fmt, m):
    jobs = _quantized(oracle_mod, fmt, ONE_BUFFER[m], 148)
    xs = [W.activation(149, m, k) for (_, k, _, _) in jobs]
    plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs], [to_dev(c) for (_, _, c, _) in jobs],
                                       [_dev_scales(fmt, s) for (_, _, _, s) in jobs], fmt=fmt,
                                       route=fp8w.ROUTE_MFMA)
    seg = plan.plan.seg_cols
    kmax = max(k for (_, k, _, _) in jobs)
    assert seg == -(-kmax // 256) * 256, seg
    tiles = plan.plan.tiles
    refs = [oracle_mod.gemv_format_f64(x, c, s, fmt) for x, (_, _, c, s) in zip(xs, jobs)]
    for run in (1, 2, 3, tiles):
        plan.plan.tiles_per_block = run
        plan.plan.blocks = -(-tiles // run)
        for y in plan.ys:
            y.fill_(float("nan"))
        ys = fp8w.fp8w_gemv_grouped(plan)
        _sync()
        for (n, k, _, _), (y_ref, bound), y in zip(jobs, refs, ys):
            assert_within_bound(bf16_to_f64(y), y_ref, bound, f"one buffer {fmt} m={m} run={run} [{n}x{k}]")


# above 16 rows: jobs of one panel (nothing to prefetch inside the job, the
# next job's x prefetched at its tile ends), K below one panel and ragged
SHORT_K = [(300, 256), (129, 16), (257, 512), (64, 272), (200, 256), (17, 784)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("m", [17, 32])
def test_grouped_short_k_above_16_rows(fp8w, oracle_mod, fmt, m):
    jobs = _quantized(oracle_mod, fmt, SHORT_K, 150)
    xs = [W.activation(151, m, k) for (_, k, _, _) in jobs]
    plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs], [to_dev(c) for (_, _, c, _) in jobs],
                                       [_dev_scales(fmt, s) for (_, _, _, s) in jobs], fmt=fmt,
                                       route=fp8w.ROUTE_MFMA)
    assert plan.plan.seg_cols == 256
    tiles = plan.plan.tiles
    refs = [oracle_mod.gemv_format_f64(x, c, s, fmt) for x, (_, _, c, s) in zip(xs, jobs)]
    for run in (1, 2, 3, tiles):
        plan.plan.tiles_per_block = run
        plan.plan.blocks = -(-tiles // run)
        for y in plan.ys:
            y.fill_(float("nan"))
        ys = fp8w.fp8w_gemv_grouped(plan)
        _sync()
        for (n, k, _, _), (y_ref, bound), y in zip(jobs, refs, ys):
            assert_within_bound(bf16_to_f64(y), y_ref, bound, f"short K {fmt} m={m} run={run} [{n}x{k}]")


@pytest.mark.parametrize("fmt", FORMATS)
def test_direct_single_calls_rotated(fp8w, oracle_mod, fmt):
    # the direct kernel: 8 waves per tile up to 4096 rows, 4 above, one or
    # two 16-row tiles per workgroup; K = 4096 / 8192 / 2048 rotated, 4112 not.  Rows
    # 7 apart sample every 16-row tile twice, and a wrongly walked panel
    # changes every row of its tile.
    jobs = _quantized(oracle_mod, fmt, [(4096, 4096), (4200, 8192), (1000, 4112), (8192, 2048)], 142)
    for n, k, c, s in jobs:
        cd, sd = to_dev(c), _dev_scales(fmt, s)
        rows = np.unique(np.concatenate([np.arange(0, n, 7), [n - 1]]))
        for m in (3, 5, 8, 9, 16, 17, 32):
            x = W.activation(143, m, k)
            y = bf16_to_f64(fp8w.fp8w_gemv(to_dev_bf16(x), cd, sd, fmt, route=fp8w.ROUTE_MFMA))
            y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, fmt, rows=rows)
            assert_within_bound(y[:, rows], y_ref, bound, f"direct {fmt} m={m} [{n}x{k}]")


@pytest.mark.parametrize("fmt", FORMATS)
def test_streaming_single_calls_rotated(fp8w, oracle_mod, fmt):
    # single calls on 32768 rows stream with the job by value, one tile per
    # workgroup; rows 61 apart, the last row of every 128-row block and the
    # rows of the ragged last tile
    n, k = 32768 + 200, 4096
    (_, _, c, s), = _quantized(oracle_mod, fmt, [(n, k)], 144)
    cd, sd = to_dev(c), _dev_scales(fmt, s)
    rows = np.unique(np.concatenate([np.arange(0, n, 61), np.arange(127, n, 128), np.arange(n - 200, n)]))
    for m in (4, 16, 32):
        x = W.activation(145, m, k)
        y = bf16_to_f64(fp8w.fp8w_gemv(to_dev_bf16(x), cd, sd, fmt, route=fp8w.ROUTE_MFMA))
        y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, fmt, rows=rows)
        assert_within_bound(y[:, rows], y_ref, bound, f"streaming single {fmt} m={m}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_w8a8_direct_rotated(fp8w, oracle_mod, fmt):
    # fp8 x fp8 direct kernel, per scale format; K = 4096 / 8192 rotated,
    # 4112 not.  The dequantized activation codes are exact in bf16, so the
    # bf16 GEMV bound applies to them, times the activation scale.
    # 8 waves per tile up to 4096 rows, 4 above; rows sampled as above.
    jobs = _quantized(oracle_mod, fmt, [(1000, 4096), (600, 8192), (300, 4112), (4200, 4096)], 146)
    for n, k, c, s in jobs:
        cd, sd = to_dev(c), _dev_scales(fmt, s)
        rows = np.unique(np.concatenate([np.arange(0, n, 7), [n - 1]]))
        for m in (5, 16, 17, 32):
            x = W.activation(147, m, k)
            xc, xs = oracle_mod.quantize_act_tensor(x)
            y = bf16_to_f64(fp8w.fp8w_gemv_w8a8(to_dev(xc), to_dev(np.array([xs], np.float32)), cd, sd, fmt))
            xb = (oracle_mod.e4m3_decode(xc).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            y_ref, bound = oracle_mod.gemv_format_f64(xb, c, s, fmt, rows=rows)
            assert_within_bound(y[:, rows], xs * y_ref, xs * bound, f"w8a8 {fmt} m={m} [{n}x{k}]")


@pytest.mark.parametrize("fmt", FORMATS)
def test_single_calls_x_in_registers(fp8w, oracle_mod, fmt):
    # single calls on many rows whose K spans eight panels keep each wave's
    # x^T fragments in registers for a run of 16-row tiles: K = 2048 and a
    # partial last panel (K = 1808), a ragged last tile; rows 53 apart, the
    # last row of every 16-row tile near both ends and the last rows
    for n, k in [(32768 + 37, 2048), (32768 + 200, 1808)]:
        (_, _, c, s), = _quantized(oracle_mod, fmt, [(n, k)], 152)
        cd, sd = to_dev(c), _dev_scales(fmt, s)
        rows = np.unique(np.concatenate([np.arange(0, n, 53), np.arange(15, 4096, 16), np.arange(n - 300, n)]))
        for m in (4, 9, 16, 17, 32):
            x = W.activation(153, m, k)
            y = bf16_to_f64(fp8w.fp8w_gemv(to_dev_bf16(x), cd, sd, fmt, route=fp8w.ROUTE_MFMA))
            y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, fmt, rows=rows)
            assert_within_bound(y[:, rows], y_ref, bound, f"x in registers {fmt} m={m} [{n}x{k}]")
