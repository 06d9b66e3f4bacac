"""GPU parity of the grouped GEMV (many independent GEMVs in one launch)
against the CPU oracle, its argument checks, and HIP-graph replays."""
import numpy as np
import pytest

from fp8_block_scaled_02_amd import workloads as W
from gpu_util import assert_within_bound, bf16_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

# ragged N, K multiples of 16 that are not multiples of 128, several jobs per K
SHAPES = [(300, 1008), (130, 272), (1024, 1024), (257, 2560), (129, 4112), (64, 16), (2560, 3072)]


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


def _jobs(oracle_mod, fmt, seed):
    out = []
    for i, (n, k) in enumerate(SHAPES):
        bits = W.gaussian_weight(30 + seed, i, n, k, outlier_rows=fmt == "block", heavy_tail=fmt == "mx")
        codes, sc = oracle_mod.quantize_block(bits) if fmt == "block" else oracle_mod.quantize_mx(bits)
        out.append((n, k, codes, sc))
    return out


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("m", [1, 2, 5, 8, 9, 16, 17, 32])
def test_grouped_matches_oracle(fp8w, oracle_mod, fmt, m):
    jobs = _jobs(oracle_mod, fmt, 0)
    xs_h = [W.activation(31, m, k) for (_, k, _, _) in jobs]
    plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs_h],
                                       [to_dev(c) for (_, _, c, _) in jobs],
                                       [to_dev(s) for (_, _, _, s) in jobs], fmt=fmt)
    assert plan.route == (fp8w.ROUTE_VALU if m == 1 or (m == 2 and fmt != "mx") else fp8w.ROUTE_MFMA)
    if plan.route == fp8w.ROUTE_MFMA:   # streaming kernel, x staged by K segments
        assert plan.plan.tiles_per_block > 0 and plan.plan.seg_cols % 256 == 0 and plan.plan.seg_cols > 0
    ys = fp8w.fp8w_gemv_grouped(plan)
    _sync()
    ref = oracle_mod.gemv_block_f64 if fmt == "block" else oracle_mod.gemv_mx_f64
    for (n, k, c, s), x, y in zip(jobs, xs_h, ys):
        y_ref, bound = ref(x, c, s)
        assert_within_bound(bf16_to_f64(y), y_ref, bound, f"grouped {fmt} m={m} [{n}x{k}]")


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("route,ms", [("mfma", (1,)), ("valu", (2, 3, 4, 6, 8))])
def test_grouped_explicit_route_where_auto_picks_the_other(fp8w, oracle_mod, fmt, route, ms):
    jobs = _jobs(oracle_mod, fmt, 1)
    r = {"valu": fp8w.ROUTE_VALU, "mfma": fp8w.ROUTE_MFMA}[route]
    ref = oracle_mod.gemv_block_f64 if fmt == "block" else oracle_mod.gemv_mx_f64
    for m in ms:
        xs_h = [W.activation(32, m, k) for (_, k, _, _) in jobs]
        plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs_h],
                                           [to_dev(c) for (_, _, c, _) in jobs],
                                           [to_dev(s) for (_, _, _, s) in jobs], fmt=fmt, route=r)
        assert plan.route == r
        ys = fp8w.fp8w_gemv_grouped(plan)
        _sync()
        for (n, k, c, s), x, y in zip(jobs, xs_h, ys):
            y_ref, bound = ref(x, c, s)
            assert_within_bound(bf16_to_f64(y), y_ref, bound, f"grouped {route} {fmt} m={m} [{n}x{k}]")


def test_grouped_rejects_overlapping_outputs(fp8w, oracle_mod):
    import torch
    jobs = _jobs(oracle_mod, "block", 2)[:2]
    xs = [to_dev_bf16(W.activation(33, 1, k)) for (_, k, _, _) in jobs]
    cs = [to_dev(c) for (_, _, c, _) in jobs]
    ss = [to_dev(s) for (_, _, _, s) in jobs]
    big = torch.empty((1, 4096), dtype=torch.bfloat16, device="cuda")
    ys = [big[:, :jobs[0][0]], big[:, 100:100 + jobs[1][0]]]        # overlapping views
    with pytest.raises(fp8w.Fp8wError) as e:
        fp8w.fp8w_grouped_plan_init(xs, cs, ss, ys=ys)
    assert e.value.status == fp8w.ERR_OVERLAP


def test_grouped_and_single_calls_replay_in_a_graph(fp8w, oracle_mod):
    """Capture single and grouped calls in one HIP graph; replay it several
    times with eager work and synchronizations in between; every replay must
    equal the eager result bit for bit."""
    import torch
    jobs = _jobs(oracle_mod, "block", 3)
    m = 3
    xs = [to_dev_bf16(W.activation(34, m, k)) for (_, k, _, _) in jobs]
    cs = [to_dev(c) for (_, _, c, _) in jobs]
    ss = [to_dev(s) for (_, _, _, s) in jobs]
    plan = fp8w.fp8w_grouped_plan_init(xs, cs, ss)
    ys_single = [torch.empty((m, c.shape[0]), dtype=torch.bfloat16, device="cuda") for c in cs]

    def run():
        fp8w.fp8w_gemv_grouped(plan)
        for x, c, s, y in zip(xs, cs, ss, ys_single):
            fp8w.fp8w_gemv_block(x, c, s, y=y)

    run()
    _sync()
    eager_g = [y.clone() for y in plan.ys]
    eager_s = [y.clone() for y in ys_single]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    _sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        for y in plan.ys + ys_single:
            y.fill_(float(rep + 7))                       # eager work between replays
        _sync()
        g.replay()
        _sync()
        for a, b in zip(plan.ys + ys_single, eager_g + eager_s):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"replay {rep}"


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("case", ["projection_like", "many_small_jobs"])
def test_grouped_streaming_kernel_matches_oracle(fp8w, oracle_mod, fmt, case):
    """m = 1 with every K <= 3072 takes the streaming kernel (runs of tiles
    per workgroup that cross job boundaries).  MX weights stream when every
    exponent array is a whole number of dwords: their N is rounded up to a
    multiple of 4 here (still ragged against the 16-row tiles)."""
    rng = np.random.default_rng(40)
    if case == "projection_like":
        shapes = [(300, 1008), (130, 272), (8192, 2560), (257, 2560), (64, 16), (2560, 3072), (17, 3072)]
    else:
        shapes = [(int(rng.integers(1, 300)), int(rng.integers(1, 193)) * 16) for _ in range(60)]
    if fmt == "mx":
        shapes = [((n + 3) // 4 * 4, k) for n, k in shapes]
    jobs = []
    for i, (n, k) in enumerate(shapes):
        bits = W.gaussian_weight(41, i, n, k, outlier_rows=fmt == "block", heavy_tail=fmt == "mx")
        c, s = oracle_mod.quantize_block(bits) if fmt == "block" else oracle_mod.quantize_mx(bits)
        jobs.append((n, k, c, s))
    xs_h = [W.activation(42, 1, k) for (_, k, _, _) in jobs]
    plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs_h],
                                       [to_dev(c) for (_, _, c, _) in jobs],
                                       [to_dev(s) for (_, _, _, s) in jobs], fmt=fmt)
    assert plan.plan.tiles_per_block > 0 and plan.plan.blocks * plan.plan.tiles_per_block >= plan.plan.tiles
    ys = fp8w.fp8w_gemv_grouped(plan)
    _sync()
    ref = oracle_mod.gemv_block_f64 if fmt == "block" else oracle_mod.gemv_mx_f64
    for (n, k, c, s), x, y in zip(jobs, xs_h, ys):
        y_ref, bound = ref(x, c, s)
        assert_within_bound(bf16_to_f64(y), y_ref, bound, f"stream {fmt} [{n}x{k}]")


def _offset_dev(a: np.ndarray, off: int):
    """Device copy of a uint8 array starting `off` bytes past an aligned
    allocation (torch allocations are 256-byte aligned)."""
    import torch
    buf = torch.zeros(a.size + off, dtype=torch.uint8, device="cuda")
    buf[off:].copy_(to_dev(np.ascontiguousarray(a).reshape(-1)))
    return buf[off:].view(a.shape)


@pytest.mark.parametrize("long_k", [False, True])
@pytest.mark.parametrize("off", [0, 1, 4])
@pytest.mark.parametrize("m", [1, 2, 8, 17])
def test_mx_exponent_alignment_paths(fp8w, oracle_mod, off, m, long_k):
    """MX exponents at every alignment: the streaming VALU kernel reads them
    as dwords only from a 4-byte aligned array of whole dwords; the MFMA
    panels read 8 bytes at once only when 8-byte aligned with groups % 8 == 0
    (K = 240 and 496 have groups % 8 == 0 without K % 256 == 0).  Grouped
    plans, single calls and forced-VALU single calls."""
    shapes = [(37, 240), (130, 496), (300, 2048), (61, 2064), (129, 1040), (7, 3056)]
    if long_k:   # several K segments in the per-call VALU kernel; no streaming plan
        shapes.append((19, 4240))
    jobs = []
    for i, (n, k) in enumerate(shapes):
        bits = W.gaussian_weight(43, i, n, k, heavy_tail=True)
        c, e = oracle_mod.quantize_mx(bits)
        jobs.append((n, k, c, e))
    xs_h = [W.activation(44, m, k) for (_, k, _, _) in jobs]
    xs = [to_dev_bf16(x) for x in xs_h]
    codes = [to_dev(c) for (_, _, c, _) in jobs]
    exps = [_offset_dev(e, off) for (_, _, _, e) in jobs]
    plan = fp8w.fp8w_grouped_plan_init(xs, codes, exps, fmt="mx")
    if m == 1:   # streaming only with aligned exponent arrays of whole dwords and every K <= 3072
        dwords = all(n * ((k + 31) // 32) % 4 == 0 for n, k in shapes)
        assert (plan.plan.tiles_per_block > 0) == (off % 4 == 0 and dwords and max(k for _, k in shapes) <= 3072)
    ys = fp8w.fp8w_gemv_grouped(plan)
    ys_single = [fp8w.fp8w_gemv_mx(x, c, e) for x, c, e in zip(xs, codes, exps)]
    ys_valu = [fp8w.fp8w_gemv_mx(x, c, e, route=fp8w.ROUTE_VALU) if m <= 8 else None
               for x, c, e in zip(xs, codes, exps)]
    _sync()
    for (n, k, c, e), x, yg, ysg, ysv in zip(jobs, xs_h, ys, ys_single, ys_valu):
        y_ref, bound = oracle_mod.gemv_mx_f64(x, c, e)
        assert_within_bound(bf16_to_f64(yg), y_ref, bound, f"grouped mx off={off} m={m} [{n}x{k}]")
        assert_within_bound(bf16_to_f64(ysg), y_ref, bound, f"single mx off={off} m={m} [{n}x{k}]")
        if ysv is not None:
            assert_within_bound(bf16_to_f64(ysv), y_ref, bound, f"single valu mx off={off} m={m} [{n}x{k}]")


# Grouped M = 1 plans above the streaming K limit run the wide per-tile
# tiles, with 4096-column K segments when that takes fewer segment rounds
# over the group (seg_cols = 4096) and 3072-column ones otherwise.
@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("shapes,seg", [([(300, 4096), (130, 3584), (257, 8176)], 4096),
                                        ([(300, 4160), (129, 6144)], 0)])
def test_grouped_wide_tiles_segment_width(fp8w, oracle_mod, fmt, shapes, seg):
    jobs = []
    for i, (n, k) in enumerate(shapes):
        bits = W.gaussian_weight(37, i, n, k, outlier_rows=fmt == "block", heavy_tail=fmt == "mx")
        codes, sc = oracle_mod.quantize_block(bits) if fmt == "block" else oracle_mod.quantize_mx(bits)
        jobs.append((n, k, codes, sc))
    xs_h = [W.activation(38, 1, k) for (_, k, _, _) in jobs]
    plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs_h], [to_dev(c) for (_, _, c, _) in jobs],
                                       [to_dev(s) for (_, _, _, s) in jobs], fmt=fmt)
    assert plan.route == fp8w.ROUTE_VALU and plan.plan.tiles_per_block == 0 and plan.plan.seg_cols == seg
    ys = fp8w.fp8w_gemv_grouped(plan)
    _sync()
    ref = oracle_mod.gemv_block_f64 if fmt == "block" else oracle_mod.gemv_mx_f64
    for (n, k, c, s), x, y in zip(jobs, xs_h, ys):
        y_ref, bound = ref(x, c, s)
        assert_within_bound(bf16_to_f64(y), y_ref, bound, f"grouped wide {fmt} seg={seg} [{n}x{k}]")


# MFMA plans over MX weights read 8 exponents per load when every GEMV's
# exponent rows start 8-byte aligned (ceil(k/32) % 8 == 0 and an aligned
# array: mx_packed8 = 1), one per chunk otherwise; ragged N and K.
@pytest.mark.parametrize("off", [0, 4])
@pytest.mark.parametrize("m", [2, 9, 17, 32])
def test_mx_packed_exponents_grouped(fp8w, oracle_mod, off, m):
    shapes = [(37, 240), (130, 496), (300, 2048), (7, 3056), (129, 4352)]
    jobs = []
    for i, (n, k) in enumerate(shapes):
        bits = W.gaussian_weight(45, i, n, k, heavy_tail=True)
        c, e = oracle_mod.quantize_mx(bits)
        jobs.append((n, k, c, e))
    xs_h = [W.activation(46, m, k) for (_, k, _, _) in jobs]
    plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs_h], [to_dev(c) for (_, _, c, _) in jobs],
                                       [_offset_dev(e, off) for (_, _, _, e) in jobs], fmt="mx")
    assert plan.route == fp8w.ROUTE_MFMA and plan.plan.mx_packed8 == (1 if off == 0 else 0)
    ys = fp8w.fp8w_gemv_grouped(plan)
    _sync()
    for (n, k, c, e), x, y in zip(jobs, xs_h, ys):
        y_ref, bound = oracle_mod.gemv_mx_f64(x, c, e)
        assert_within_bound(bf16_to_f64(y), y_ref, bound, f"grouped mx packed={off == 0} m={m} [{n}x{k}]")


# Streaming MX plans at M = 1 with ragged N: exponent arrays of whole dwords
# (groups % 4 == 0, so any n) stream, the span of the last tile reaching past
# row n - 1; one array of n * groups % 4 != 0 in the group keeps the plan on
# the per-tile kernel.
@pytest.mark.parametrize("odd", [False, True])
def test_mx_streaming_ragged_rows(fp8w, oracle_mod, odd):
    shapes = [(37, 256), (130, 2048), (301, 3072), (5, 128)] + ([(61, 2064)] if odd else [])
    jobs = []
    for i, (n, k) in enumerate(shapes):
        bits = W.gaussian_weight(47, i, n, k, heavy_tail=True)
        c, e = oracle_mod.quantize_mx(bits)
        jobs.append((n, k, c, e))
    xs_h = [W.activation(48, 1, k) for (_, k, _, _) in jobs]
    plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs_h], [to_dev(c) for (_, _, c, _) in jobs],
                                       [to_dev(e) for (_, _, _, e) in jobs], fmt="mx")
    assert (plan.plan.tiles_per_block > 0) == (not odd)
    ys = fp8w.fp8w_gemv_grouped(plan)
    _sync()
    for (n, k, c, e), x, y in zip(jobs, xs_h, ys):
        y_ref, bound = oracle_mod.gemv_mx_f64(x, c, e)
        assert_within_bound(bf16_to_f64(y), y_ref, bound, f"streaming mx odd={odd} [{n}x{k}]")


# Grouped MFMA plans run several 128-row tiles per workgroup when the group
# has more tiles than eight per resident workgroup slot; every run length is
# exercised here by rewriting the plan's run length (a valid plan: blocks *
# tiles_per_block >= tiles), runs that cross job boundaries included. Outputs are poisoned first so a
# tile that no workgroup sums shows.
@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("m", [4, 17])
def test_grouped_mfma_run_lengths(fp8w, oracle_mod, fmt, m):
    jobs = _jobs(oracle_mod, fmt, 2)
    xs_h = [W.activation(50, m, k) for (_, k, _, _) in jobs]
    plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs_h], [to_dev(c) for (_, _, c, _) in jobs],
                                       [to_dev(s) for (_, _, _, s) in jobs], fmt=fmt, route=fp8w.ROUTE_MFMA)
    tiles = plan.plan.tiles
    assert tiles == sum(-(-n // 128) for n, _, _, _ in jobs)
    ref = oracle_mod.gemv_block_f64 if fmt == "block" else oracle_mod.gemv_mx_f64
    refs = [ref(x, c, s) for x, (_, _, c, s) in zip(xs_h, jobs)]
    for run in (2, 3, 7, tiles):
        plan.plan.tiles_per_block = run
        plan.plan.blocks = -(-tiles // run)
        for y in plan.ys:
            y.fill_(float("nan"))
        ys = fp8w.fp8w_gemv_grouped(plan)
        _sync()
        for (n, k, _, _), (y_ref, bound), y in zip(jobs, refs, ys):
            assert_within_bound(bf16_to_f64(y), y_ref, bound, f"mfma runs {fmt} m={m} run={run} [{n}x{k}]")
