"""GPU parity of the other scale formats (bf16 128x128 block scales,
per-row and per-tensor fp32 scales) through the generic calls: quantize and
dequantize bit for bit against the oracle, and the GEMV (both routes, single
calls and grouped), the W8A8 GEMV and the large-M route within the bound."""
import numpy as np
import pytest

from cases import edge_case_weight
from fp8_block_scaled_02_amd import workloads as W
from gpu_util import assert_within_bound, bf16_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

NEW = ("block_bf16", "row", "tensor")
ALL = ("block", "mx") + NEW
SHAPES = [(300, 1008), (130, 272), (257, 2560), (129, 4112), (64, 16), (2560, 3072)]


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


def _np_scales(t):
    """Device scale tensor -> the numpy array the oracle takes (bf16 as bits)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _dev_scales(fmt, s):
    import torch
    t = to_dev(np.ascontiguousarray(s))
    return t.view(torch.bfloat16) if fmt == "block_bf16" else t


@pytest.mark.parametrize("fmt", ALL)
@pytest.mark.parametrize("n,k", [(300, 1000), (127, 129), (1, 16), (2560, 3072), (96, 200)])
def test_quantize_and_dequantize_bit_exact(fp8w, oracle_mod, fmt, n, k):
    import torch
    bits = W.gaussian_weight(80, n + k, n, k, outlier_rows=True, heavy_tail=fmt == "mx")
    codes, scales = fp8w.fp8w_quantize(to_dev_bf16(bits), fmt)
    deq = fp8w.fp8w_dequantize(codes, scales, fmt)
    _sync()
    rc, rs = oracle_mod.quantize_format(bits, fmt)
    assert np.array_equal(_np_scales(scales).reshape(rs.shape).view(rs.dtype), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(deq.view(torch.int16).cpu().numpy().view(np.uint16),
                          oracle_mod.dequant_format_bf16(rc, rs, fmt))


@pytest.mark.parametrize("fmt", NEW)
def test_edge_tiles(fp8w, oracle_mod, fmt):
    bits = edge_case_weight()                # all-zero, subnormal-amax, +-448, huge and -0 tiles
    codes, scales = fp8w.fp8w_quantize(to_dev_bf16(bits), fmt)
    _sync()
    rc, rs = oracle_mod.quantize_format(bits, fmt)
    assert np.array_equal(_np_scales(scales).reshape(rs.shape).view(rs.dtype), rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def _jobs(oracle_mod, fmt, seed):
    out = []
    for i, (n, k) in enumerate(SHAPES):
        bits = W.gaussian_weight(81 + seed, i, n, k, outlier_rows=True, heavy_tail=False)
        c, s = oracle_mod.quantize_format(bits, fmt)
        out.append((n, k, c, s))
    return out


@pytest.mark.parametrize("fmt", NEW)
def test_gemv_single_both_routes(fp8w, oracle_mod, fmt):
    jobs = _jobs(oracle_mod, fmt, 0)
    for route, ms in ((fp8w.ROUTE_VALU, (1, 2, 5, 8)), (fp8w.ROUTE_MFMA, (1, 3, 9, 16, 17, 32))):
        for m in ms:
            for n, k, c, s in jobs:
                x = W.activation(82, m, k)
                y = bf16_to_f64(fp8w.fp8w_gemv(to_dev_bf16(x), to_dev(c), _dev_scales(fmt, s), fmt, route=route))
                y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, fmt)
                assert_within_bound(y, y_ref, bound, f"{fmt} route={route} m={m} [{n}x{k}]")


@pytest.mark.parametrize("fmt", NEW)
@pytest.mark.parametrize("m", [1, 2, 8, 16, 32])
def test_gemv_grouped(fp8w, oracle_mod, fmt, m):
    jobs = _jobs(oracle_mod, fmt, 1)
    xs = [W.activation(83, m, k) for (_, k, _, _) in jobs]
    plan = fp8w.fp8w_grouped_plan_init([to_dev_bf16(x) for x in xs], [to_dev(c) for (_, _, c, _) in jobs],
                                       [_dev_scales(fmt, s) for (_, _, _, s) in jobs], fmt=fmt)
    ys = fp8w.fp8w_gemv_grouped(plan)
    _sync()
    for (n, k, c, s), x, y in zip(jobs, xs, ys):
        y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, fmt)
        assert_within_bound(bf16_to_f64(y), y_ref, bound, f"grouped {fmt} m={m} [{n}x{k}]")


@pytest.mark.parametrize("fmt", NEW)
def test_w8a8_and_large_m_routes(fp8w, oracle_mod, fmt):
    n, k = 1030, 2048
    bits = W.gaussian_weight(84, 0, n, k, outlier_rows=True, heavy_tail=False)
    c, s = oracle_mod.quantize_format(bits, fmt)
    cd, sd = to_dev(c), _dev_scales(fmt, s)
    for m in (1, 7, 16, 32):
        x = W.activation(84, m, k)
        xc, xs = oracle_mod.quantize_act_tensor(x)
        y = bf16_to_f64(fp8w.fp8w_gemv_w8a8(to_dev(xc), to_dev(np.array([xs], np.float32)), cd, sd, fmt))
        # the dequantized activation codes are exact in bf16, so the bf16 reference applies, times xs
        xb = (oracle_mod.e4m3_decode(xc).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        y_ref, bound = oracle_mod.gemv_format_f64(xb, c, s, fmt)
        assert_within_bound(y, xs * y_ref, xs * bound, f"w8a8 {fmt} m={m}")
    for m in (33, 200):
        x = W.activation(85, m, k)
        y = bf16_to_f64(fp8w.fp8w_gemm(to_dev_bf16(x), cd, sd, fmt))
        rows = np.array([0, 5, 128, 513, n - 1])
        y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, fmt, rows=rows)
        assert_within_bound(y[:, rows], y_ref, bound, f"gemm {fmt} m={m}")


@pytest.mark.parametrize("fmt", ALL)
def test_fp8weight_formats_end_to_end(fp8w, oracle_mod, fmt):
    name = {"block": fp8w.BLOCK128, "mx": fp8w.MX32, "block_bf16": fp8w.BLOCK128_BF16, "row": fp8w.ROW,
            "tensor": fp8w.TENSOR}[fmt]
    bits = W.gaussian_weight(86, 0, 512, 768, outlier_rows=False, heavy_tail=False)
    wt = fp8w.Fp8Weight.quantize(to_dev_bf16(bits), name)
    c, s = wt.codes.cpu().numpy(), _np_scales(wt.scales)
    for m in (4, 64):
        x = W.activation(86, m, 768)
        y = bf16_to_f64(wt.matmul(to_dev_bf16(x)))
        y_ref, bound = oracle_mod.gemv_format_f64(x, c, s, fmt)
        assert_within_bound(y, y_ref, bound, f"Fp8Weight {fmt} m={m}")
