"""GPU parity of the dequantizers and of the large-M GEMM route.

Dequantized weights are compared bit for bit with the oracle's bf16
dequantizers (fp32 product of the decoded value and the scale, rounded to
nearest even bf16), on both kernel paths (16-byte chunks, and any k or
alignment), on every code against scales over the whole fp32 range, on
every (code, e8m0 byte) pair, and on full-size weights.  The GEMM route is
compared with the oracle's fp64 product on sampled outputs within the GEMV
bound.
"""
import numpy as np
import pytest

from cases import edge_case_weight
from fp8_block_scaled_02_amd import workloads as W
from gpu_util import assert_within_bound, bf16_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

NON_NAN = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)


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


def _bits(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _misaligned_u8(a: np.ndarray):
    """Device copy of a uint8 [n, k] array whose data pointer is odd."""
    import torch
    n, k = a.shape
    buf = torch.empty(n * k + 1, dtype=torch.uint8, device="cuda")
    buf[1:].copy_(torch.from_numpy(a.reshape(-1)))
    return buf[1:].view(n, k)


@pytest.mark.parametrize("n,k", [(300, 1008), (129, 4112), (1, 16), (127, 129), (1, 1), (1000, 1000), (130, 24)])
@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_dequantize_matches_oracle_on_ragged_shapes(fp8w, oracle_mod, n, k, fmt):
    rng = np.random.default_rng(n * 7 + k)
    codes = rng.choice(NON_NAN, size=(n, k)).astype(np.uint8)
    if fmt == "block":
        s = np.ldexp(rng.uniform(1, 2, oracle_mod.block_scale_shape(n, k)),
                     rng.integers(-30, 10, oracle_mod.block_scale_shape(n, k))).astype(np.float32)
        got = fp8w.fp8w_dequantize_block(to_dev(codes), to_dev(s))
        want = oracle_mod.dequant_block_bf16(codes, s)
    else:
        e = rng.integers(90, 140, oracle_mod.mx_scale_shape(n, k)).astype(np.uint8)
        got = fp8w.fp8w_dequantize_mx(to_dev(codes), to_dev(e))
        want = oracle_mod.dequant_mx_bf16(codes, e)
    _sync()
    assert np.array_equal(_bits(got), want)


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_dequantize_vector_path_on_8_byte_aligned_codes(fp8w, oracle_mod, fmt):
    """Codes 8 bytes past an aligned allocation: the vector path's 8-byte
    unit loads, with k % 16 == 8."""
    import torch
    n, k = 77, 1032
    rng = np.random.default_rng(6)
    codes = rng.choice(NON_NAN, size=(n, k)).astype(np.uint8)
    buf = torch.empty(n * k + 8, dtype=torch.uint8, device="cuda")
    buf[8:].copy_(torch.from_numpy(codes.reshape(-1)))
    c = buf[8:].view(n, k)
    if fmt == "block":
        s = rng.uniform(1e-4, 1e-2, oracle_mod.block_scale_shape(n, k)).astype(np.float32)
        got, want = fp8w.fp8w_dequantize_block(c, to_dev(s)), oracle_mod.dequant_block_bf16(codes, s)
    else:
        e = rng.integers(100, 130, oracle_mod.mx_scale_shape(n, k)).astype(np.uint8)
        got, want = fp8w.fp8w_dequantize_mx(c, to_dev(e)), oracle_mod.dequant_mx_bf16(codes, e)
    _sync()
    assert np.array_equal(_bits(got), want)


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_dequantize_scalar_path_on_misaligned_codes(fp8w, oracle_mod, fmt):
    n, k = 256, 512                     # k % 16 == 0, but the codes pointer is odd
    rng = np.random.default_rng(5)
    codes = rng.choice(NON_NAN, size=(n, k)).astype(np.uint8)
    c = _misaligned_u8(codes)
    if fmt == "block":
        s = rng.uniform(1e-4, 1e-2, oracle_mod.block_scale_shape(n, k)).astype(np.float32)
        got, want = fp8w.fp8w_dequantize_block(c, to_dev(s)), oracle_mod.dequant_block_bf16(codes, s)
    else:
        e = rng.integers(100, 130, oracle_mod.mx_scale_shape(n, k)).astype(np.uint8)
        got, want = fp8w.fp8w_dequantize_mx(c, to_dev(e)), oracle_mod.dequant_mx_bf16(codes, e)
    _sync()
    assert np.array_equal(_bits(got), want)


def test_dequantize_block_every_code_against_scales_over_the_fp32_range(fp8w, oracle_mod):
    # one 128 x 128 tile per scale; rows of the tile cycle through the 254 codes
    rng = np.random.default_rng(6)
    scales = np.concatenate([
        np.ldexp(rng.uniform(1, 2, 400), rng.integers(-149, 120, 400)),     # every binade, subnormals too
        [1.0, 2.0 ** -149, 2.0 ** -126, 3.4e38 / 448, 1.0 / 448],
    ]).astype(np.float32)
    t = scales.size
    codes = np.resize(np.tile(NON_NAN, 65), (t * 128, 128)).astype(np.uint8)
    s = scales.reshape(t, 1)
    got = fp8w.fp8w_dequantize_block(to_dev(codes), to_dev(s))
    _sync()
    assert np.array_equal(_bits(got), oracle_mod.dequant_block_bf16(codes, s))


def test_dequantize_mx_every_code_times_every_scale_byte(fp8w, oracle_mod):
    codes = np.repeat(np.tile(NON_NAN, (255, 1)), 32, axis=1)            # [255, 254*32]
    e8m0 = np.repeat(np.arange(255, dtype=np.uint8)[:, None], codes.shape[1] // 32, axis=1)
    got = fp8w.fp8w_dequantize_mx(to_dev(codes), to_dev(e8m0))
    _sync()
    assert np.array_equal(_bits(got), oracle_mod.dequant_mx_bf16(codes, e8m0))   # incl. overflow to inf


@pytest.mark.parametrize("misaligned", [False, True])
def test_dequantize_mx_exponent_positions(fp8w, oracle_mod, misaligned):
    """Exponent rows of 80 bytes (k = 2560) whose bytes run through every
    value 0..254 at each of the four byte positions of a dword, on an
    aligned and on an odd exponent pointer: each group takes its own
    exponent."""
    n, k = 97, 2560
    rng = np.random.default_rng(8)
    codes = rng.choice(NON_NAN, size=(n, k)).astype(np.uint8)
    e8m0 = (np.arange(n * (k // 32)) % 255).astype(np.uint8).reshape(n, k // 32)
    e = _misaligned_u8(e8m0) if misaligned else to_dev(e8m0)
    got = fp8w.fp8w_dequantize_mx(to_dev(codes), e)
    _sync()
    assert np.array_equal(_bits(got), oracle_mod.dequant_mx_bf16(codes, e8m0))


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_dequantize_nan_codes_give_nan(fp8w, fmt):
    import torch
    codes = np.array([[0x7F, 0xFF] * 8], dtype=np.uint8)
    if fmt == "block":
        w = fp8w.fp8w_dequantize_block(to_dev(codes), to_dev(np.ones((1, 1), np.float32)))
    else:
        w = fp8w.fp8w_dequantize_mx(to_dev(codes), to_dev(np.full((1, 1), 127, np.uint8)))
    _sync()
    assert torch.isnan(w.float()).all()


def test_dequantize_edge_tiles_after_gpu_quantize(fp8w, oracle_mod):
    bits = edge_case_weight()
    for q, d, od in ((fp8w.fp8w_quantize_block, fp8w.fp8w_dequantize_block, oracle_mod.dequant_block_bf16),
                     (fp8w.fp8w_quantize_mx, fp8w.fp8w_dequantize_mx, oracle_mod.dequant_mx_bf16)):
        c, s = q(to_dev_bf16(bits))
        w = d(c, s)
        _sync()
        assert np.array_equal(_bits(w), od(c.cpu().numpy(), s.cpu().numpy()))


def test_dequantize_dense_layer_full_size_and_round_trip(fp8w, oracle_mod):
    """The 8B dense layer's four weights: bit-exact against the oracle, and
    the quantize -> dequantize round trip near the pages' 2.25 % (lm_head QAT
    page, Validation)."""
    for w in W.WORKLOADS[4].weights:
        bits = w.bits(4)
        c, s = fp8w.fp8w_quantize_block(to_dev_bf16(bits))
        deq = fp8w.fp8w_dequantize_block(c, s)
        _sync()
        got = _bits(deq)
        assert np.array_equal(got, oracle_mod.dequant_block_bf16(c.cpu().numpy(), s.cpu().numpy())), w.name
        ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        back = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        nz = ref != 0
        rel = float(np.mean(np.abs(back[nz] - ref[nz]) / np.abs(ref[nz])))
        assert 0.020 < rel < 0.025, (w.name, rel)


# ------------------------------------------------------------ GEMM route --

def _check_gemm(fp8w, oracle_mod, fmt, n, k, m, seed, x_rows=None, w_rows=None):
    import torch
    rng = np.random.default_rng(seed)
    bits = W.gaussian_weight(40, seed, n, k, outlier_rows=fmt == "block", heavy_tail=fmt == "mx")
    x = W.activation(40, m, k)
    if fmt == "block":
        codes, s = oracle_mod.quantize_block(bits)
        y = fp8w.fp8w_gemm_block(to_dev_bf16(x), to_dev(codes), to_dev(s))
        ref = oracle_mod.gemv_block_f64
    else:
        codes, s = oracle_mod.quantize_mx(bits)
        y = fp8w.fp8w_gemm_mx(to_dev_bf16(x), to_dev(codes), to_dev(s))
        ref = oracle_mod.gemv_mx_f64
    _sync()
    yg = bf16_to_f64(y)
    mi = np.arange(m) if x_rows is None else np.unique(np.r_[0, m - 1, rng.choice(m, x_rows)])
    nj = np.arange(n) if w_rows is None else np.unique(np.r_[0, n - 1, rng.choice(n, w_rows)])
    y_ref, bound = ref(x[mi], codes, s, rows=nj)
    assert_within_bound(yg[np.ix_(mi, nj)], y_ref, bound, f"gemm {fmt} m={m} [{n}x{k}]")
    del torch


@pytest.mark.parametrize("fmt", ["block", "mx"])
@pytest.mark.parametrize("m", [1, 33, 64, 300])
def test_gemm_route_ragged(fp8w, oracle_mod, fmt, m):
    _check_gemm(fp8w, oracle_mod, fmt, 300, 1000, m, 1)     # k not a multiple of 16: scalar dequantize


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_gemm_route_dense_layer_shapes(fp8w, oracle_mod, fmt):
    for (n, k), m in (((4096, 4096), 1024), ((6144, 4096), 300), ((4096, 12288), 96)):
        _check_gemm(fp8w, oracle_mod, fmt, n, k, m, n + k, x_rows=6, w_rows=24)


def test_gemm_workspace_holds_the_dequantized_weight(fp8w, oracle_mod):
    import torch
    n, k, m = 384, 512, 48
    bits = W.gaussian_weight(41, 0, n, k, outlier_rows=True, heavy_tail=False)
    codes, s = oracle_mod.quantize_block(bits)
    ws = torch.empty(fp8w.lib().fp8w_gemm_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    fp8w.fp8w_gemm_block(to_dev_bf16(W.activation(41, m, k)), to_dev(codes), to_dev(s), workspace=ws)
    _sync()
    assert np.array_equal(ws.cpu().numpy().view(np.uint16).reshape(n, k),
                          oracle_mod.dequant_block_bf16(codes, s))


def test_fp8weight_matmul_routes_on_m(fp8w, oracle_mod):
    n, k = 512, 1024
    bits = W.gaussian_weight(42, 0, n, k, outlier_rows=False, heavy_tail=False)
    for fmt in (fp8w.BLOCK128, fp8w.MX32):
        wt = fp8w.Fp8Weight.quantize(to_dev_bf16(bits), fmt)
        c, s = wt.codes.cpu().numpy(), wt.scales.cpu().numpy()
        ref = oracle_mod.gemv_block_f64 if fmt == fp8w.BLOCK128 else oracle_mod.gemv_mx_f64
        for m in (8, 32, 33, 200):
            x = W.activation(42, m, k)
            y = bf16_to_f64(wt.matmul(to_dev_bf16(x)))
            y_ref, bound = ref(x, c, s)
            assert_within_bound(y, y_ref, bound, f"matmul {fmt} m={m}")
