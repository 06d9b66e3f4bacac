"""GPU parity: libfp8w (HIP, through the C ABI) against the CPU oracle.

Codes and scales must be bit-exact; GEMV outputs must satisfy
|y - y_ref| <= 2^-7 * (|x| . |deq W|^T) + 1e-6 with y_ref in fp64 from the
oracle's own quantization of the same seeded weights.  Every expected value
comes from the oracle; nothing computed on the GPU is fed back to it.
"""
import numpy as np
import pytest

from cases import edge_case_weight
from fp8_block_scaled_02_amd import workloads as W
from gpu_util import assert_within_bound, bf16_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8w():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import fp8_block_scaled_02_amd as F
    F.lib()
    return F


def _ids(shape):
    return "x".join(map(str, shape))


def _sync():
    import torch
    torch.cuda.synchronize()


# ---------------------------------------------------------------- block ----

BLOCK_SHAPES = [(1, 1), (1, 127), (127, 129), (130, 260), (1000, 1000), (129, 4100),
                (1024, 1024), (2560, 3072), (6656, 2560)]


@pytest.mark.parametrize("shape", BLOCK_SHAPES, ids=_ids)
def test_quantize_block_bit_exact(fp8w, oracle_mod, shape):
    bits = W.gaussian_weight(11, shape[0] * 31 + shape[1], *shape, outlier_rows=shape[0] >= 100)
    codes, scales = fp8w.fp8w_quantize_block(to_dev_bf16(bits))
    _sync()
    ref_c, ref_s = oracle_mod.quantize_block(bits)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def test_quantize_block_edge_tiles(fp8w, oracle_mod):
    bits = edge_case_weight()
    codes, scales = fp8w.fp8w_quantize_block(to_dev_bf16(bits))
    _sync()
    ref_c, ref_s = oracle_mod.quantize_block(bits)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def test_quantize_block_config1(fp8w, oracle_mod):
    bits = W.WORKLOADS[1].weights[0].bits(1)
    codes, scales = fp8w.fp8w_quantize_block(to_dev_bf16(bits))
    _sync()
    ref_c, ref_s = oracle_mod.quantize_block(bits)
    assert np.array_equal(scales.cpu().numpy(), ref_s) and np.array_equal(codes.cpu().numpy(), ref_c)


@pytest.mark.parametrize("shape", [(200, 256), (130, 300)], ids=_ids)
def test_quantize_block_unaligned_source(fp8w, oracle_mod, shape):
    """A source that is not 16-byte aligned takes the any-alignment kernel."""
    n, k = shape
    bits = W.gaussian_weight(12, n + k, n, k)
    flat = to_dev_bf16(np.concatenate([np.zeros(1, np.uint16), bits.ravel()]))
    w = flat[1:].view(n, k)
    assert w.data_ptr() % 16 != 0
    codes, scales = fp8w.fp8w_quantize_block(w)
    _sync()
    ref_c, ref_s = oracle_mod.quantize_block(bits)
    assert np.array_equal(scales.cpu().numpy(), ref_s) and np.array_equal(codes.cpu().numpy(), ref_c)


def test_quantize_block_guard_bands_untouched(fp8w):
    import torch
    n, k = 257, 300
    bits = W.gaussian_weight(13, 0, n, k)
    tn, tk = fp8w.block_scale_shape(n, k)
    cbuf = torch.full((n * k + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((tn * tk + 1024,), -7.0, dtype=torch.float32, device="cuda")
    fp8w.fp8w_quantize_block(to_dev_bf16(bits), cbuf[:n * k].view(n, k), sbuf[:tn * tk].view(tn, tk))
    _sync()
    assert (cbuf[n * k:] == 0xA5).all() and (sbuf[tn * tk:] == -7.0).all()


# ------------------------------------------------------------------- MX ----

MX_SHAPES = [(1, 1), (3, 31), (5, 1008), (64, 2560), (129, 4100), (2560, 3072), (8192, 2560)]


@pytest.mark.parametrize("shape", MX_SHAPES, ids=_ids)
def test_quantize_mx_bit_exact(fp8w, oracle_mod, shape):
    bits = W.gaussian_weight(14, shape[0] * 31 + shape[1], *shape, heavy_tail=True)
    codes, e8m0 = fp8w.fp8w_quantize_mx(to_dev_bf16(bits))
    _sync()
    ref_c, ref_e = oracle_mod.quantize_mx(bits)
    assert np.array_equal(e8m0.cpu().numpy(), ref_e)
    assert np.array_equal(codes.cpu().numpy(), ref_c)


def test_quantize_mx_edge_groups_and_unaligned(fp8w, oracle_mod):
    bits = edge_case_weight()
    ref_c, ref_e = oracle_mod.quantize_mx(bits)
    codes, e8m0 = fp8w.fp8w_quantize_mx(to_dev_bf16(bits))
    _sync()
    assert np.array_equal(e8m0.cpu().numpy(), ref_e) and np.array_equal(codes.cpu().numpy(), ref_c)
    n, k = bits.shape
    flat = to_dev_bf16(np.concatenate([np.zeros(1, np.uint16), bits.ravel()]))
    codes2, e8m02 = fp8w.fp8w_quantize_mx(flat[1:].view(n, k))
    _sync()
    assert np.array_equal(e8m02.cpu().numpy(), ref_e) and np.array_equal(codes2.cpu().numpy(), ref_c)


# ----------------------------------------------------------------- GEMV ----

GEMV_SHAPES = [(130, 272), (300, 1008), (1024, 1024), (257, 2560)]


def _block_case(oracle_mod, n, k, seed):
    bits = W.gaussian_weight(15, seed, n, k, outlier_rows=True)
    return oracle_mod.quantize_block(bits)


@pytest.mark.parametrize("m", list(range(1, 33)))
def test_gemv_block_every_m(fp8w, oracle_mod, m):
    for (n, k) in GEMV_SHAPES:
        codes, scales = _block_case(oracle_mod, n, k, n + k)
        x = W.activation(15, m, k)
        y = fp8w.fp8w_gemv_block(to_dev_bf16(x), to_dev(codes), to_dev(scales))
        _sync()
        y_ref, bound = oracle_mod.gemv_block_f64(x, codes, scales)
        assert_within_bound(bf16_to_f64(y), y_ref, bound, f"block m={m} [{n}x{k}]")


@pytest.mark.parametrize("route", ["valu", "mfma"])
def test_gemv_block_each_route(fp8w, oracle_mod, route):
    r = {"valu": fp8w.ROUTE_VALU, "mfma": fp8w.ROUTE_MFMA}[route]
    ms = range(1, 9) if route == "valu" else range(1, 33)
    n, k = 300, 1008
    codes, scales = _block_case(oracle_mod, n, k, 1)
    for m in ms:
        x = W.activation(16, m, k)
        y = fp8w.fp8w_gemv_block(to_dev_bf16(x), to_dev(codes), to_dev(scales), route=r)
        _sync()
        y_ref, bound = oracle_mod.gemv_block_f64(x, codes, scales)
        assert_within_bound(bf16_to_f64(y), y_ref, bound, f"{route} m={m}")


@pytest.mark.parametrize("m", list(range(1, 33)))
def test_gemv_mx_every_m(fp8w, oracle_mod, m):
    for (n, k) in [(130, 272), (257, 2560)]:
        bits = W.gaussian_weight(17, n + k, n, k, heavy_tail=True)
        codes, e8m0 = oracle_mod.quantize_mx(bits)
        x = W.activation(17, m, k)
        y = fp8w.fp8w_gemv_mx(to_dev_bf16(x), to_dev(codes), to_dev(e8m0))
        _sync()
        y_ref, bound = oracle_mod.gemv_mx_f64(x, codes, e8m0)
        assert_within_bound(bf16_to_f64(y), y_ref, bound, f"mx m={m} [{n}x{k}]")


@pytest.mark.parametrize("route", ["valu", "mfma"])
def test_gemv_decodes_every_code_exactly(fp8w, oracle_mod, route):
    """One-hot x against a weight whose row r holds code r: y[r] = dec(r)."""
    r = {"valu": fp8w.ROUTE_VALU, "mfma": fp8w.ROUTE_MFMA}[route]
    n, k = 256, 256
    codes = np.tile(np.arange(256, dtype=np.uint8)[:, None], (1, k))
    codes[(codes & 0x7F) == 0x7F] = 0
    scales = np.ones((2, 2), np.float32)
    for col in (0, 17, 255):
        x = np.zeros((1, k), np.uint16)
        x[0, col] = 0x3F80
        y = fp8w.fp8w_gemv_block(to_dev_bf16(x), to_dev(codes), to_dev(scales), route=r)
        _sync()
        y_ref, _ = oracle_mod.gemv_block_f64(x, codes, scales)
        assert np.array_equal(bf16_to_f64(y), y_ref)


@pytest.mark.parametrize("route", ["valu", "mfma"])
def test_gemv_mx_every_code_times_every_scale_byte(fp8w, oracle_mod, route):
    """Exhaustive over the 254 finite codes x e8m0 bytes 0..246: row r holds
    one (code, byte) pair in column 0, x is one-hot on column 0, so
    y[r] = dec(code) * 2^(byte-127).  Exact whenever that is a normal bf16.
    Bytes >= 247 are excluded: with them the largest codes dequantize to
    2^128 or more, which is not finite in fp32 (outside the contract)."""
    r = {"valu": fp8w.ROUTE_VALU, "mfma": fp8w.ROUTE_MFMA}[route]
    code_vals = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    e_vals = np.arange(0, 247, dtype=np.uint8)
    cc, ee = np.meshgrid(code_vals, e_vals, indexing="ij")
    n, k = cc.size, 64
    rng = np.random.default_rng(6)
    codes = rng.integers(0, 0x70, size=(n, k), dtype=np.uint8)   # finite filler
    codes[:, 0] = cc.ravel()
    e8m0 = np.stack([ee.ravel(), ee.ravel()], axis=1).astype(np.uint8)
    x = np.zeros((1, k), np.uint16)
    x[0, 0] = 0x3F80
    y = fp8w.fp8w_gemv_mx(to_dev_bf16(x), to_dev(codes), to_dev(e8m0), route=r)
    _sync()
    y_ref, bound = oracle_mod.gemv_mx_f64(x, codes, e8m0)
    got = bf16_to_f64(y)
    assert_within_bound(got, y_ref, bound, f"mx code x byte {route}")
    normal = np.abs(y_ref) >= 2.0 ** -126
    assert np.array_equal(got[normal], y_ref[normal])


def test_gemv_is_bitwise_deterministic(fp8w, oracle_mod):
    import torch
    n, k = 2560, 3072
    codes, scales = _block_case(oracle_mod, n, k, 3)
    cd, sd = to_dev(codes), to_dev(scales)
    for m in (1, 8, 16, 32):
        xd = to_dev_bf16(W.activation(18, m, k))
        a = fp8w.fp8w_gemv_block(xd, cd, sd)
        b = fp8w.fp8w_gemv_block(xd, cd, sd)
        _sync()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_gemv_guard_bands_and_no_write_on_error(fp8w, oracle_mod):
    import torch
    n, k, m = 300, 1008, 5
    codes, scales = _block_case(oracle_mod, n, k, 4)
    x = to_dev_bf16(W.activation(19, m, k))
    ybuf = torch.full((m * n + 512,), 1234.0, dtype=torch.bfloat16, device="cuda")
    fp8w.fp8w_gemv_block(x, to_dev(codes), to_dev(scales), y=ybuf[:m * n].view(m, n))
    _sync()
    assert (ybuf[m * n:] == 1234.0).all()
    # an invalid call (m = 33) returns an error and writes nothing
    yb2 = torch.full((33 * n,), 77.0, dtype=torch.bfloat16, device="cuda")
    st = fp8w.lib().fp8w_gemv_block(x.data_ptr(), 33, to_dev(codes).data_ptr(),
                                    to_dev(scales).data_ptr(), n, k, yb2.data_ptr(), None)
    _sync()
    assert st == fp8w.ERR_SHAPE and (yb2 == 77.0).all()


# ------------------------------------------------ minimal and long-K shapes --

EDGE_GEMV = [(1, 16), (17, 16), (1, 65552), (3, 32784), (33, 4112)]


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("m", [1, 2, 8, 9, 16, 17, 32])
def test_gemv_minimal_and_long_k_on_every_route(fp8w, oracle_mod, fmt, m):
    """N = 1 and K = 16 (one 16-byte chunk, a tile and panel almost all
    padding), and K up to 65552 (dozens of K segments on the VALU kernels,
    many x segments on the streaming MFMA kernel): single calls on AUTO and
    on both routes, and the same GEMVs as one grouped plan."""
    routes = [fp8w.ROUTE_AUTO, fp8w.ROUTE_MFMA] + ([fp8w.ROUTE_VALU] if m <= 8 else [])
    quant = oracle_mod.quantize_block if fmt == "block" else oracle_mod.quantize_mx
    ref = oracle_mod.gemv_block_f64 if fmt == "block" else oracle_mod.gemv_mx_f64
    jobs = []
    for i, (n, k) in enumerate(EDGE_GEMV):
        c, s = quant(W.gaussian_weight(17, i, n, k, outlier_rows=fmt == "block", heavy_tail=fmt == "mx"))
        x = W.activation(17, m, k)
        jobs.append((n, k, c, s, x, ref(x, c, s)))
    dev = [(to_dev_bf16(x), to_dev(c), to_dev(s)) for (_, _, c, s, x, _) in jobs]
    for r in routes:
        for (n, k, _, _, _, (y_ref, bound)), (xd, cd, sd) in zip(jobs, dev):
            y = fp8w.fp8w_gemv(xd, cd, sd, fmt, route=r)
            _sync()
            assert_within_bound(bf16_to_f64(y), y_ref, bound, f"{fmt} m={m} route={r} [{n}x{k}]")
    for r in routes:
        plan = fp8w.fp8w_grouped_plan_init([d[0] for d in dev], [d[1] for d in dev], [d[2] for d in dev],
                                           fmt=fmt, route=r)
        ys = fp8w.fp8w_gemv_grouped(plan)
        _sync()
        for (n, k, _, _, _, (y_ref, bound)), y in zip(jobs, ys):
            assert_within_bound(bf16_to_f64(y), y_ref, bound, f"grouped {fmt} m={m} route={r} [{n}x{k}]")
