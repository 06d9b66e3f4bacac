"""GPU parity of the W8A8 route: per-tensor activation quantization (bit
exact against the oracle on both the one-launch and the block-parallel path)
and the fp8 x fp8 GEMV (within the GEMV bound of the fp64 product of the
same quantized operands; end to end within that plus the activation's own
quantization error)."""
import numpy as np
import pytest

from fp8_block_scaled_02_amd import workloads as W
from gpu_util import assert_within_bound, bf16_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

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


@pytest.mark.parametrize("m,k", [(1, 16), (8, 128), (32, 512), (32, 520), (32, 12288), (7, 1001), (33, 1001),
                                 (300, 3072)])
def test_quantize_act_bit_exact(fp8w, oracle_mod, m, k):
    """(32, 512) is exactly 16384 elements (one launch); (32, 520) the first
    block-parallel size; odd counts take the scalar path."""
    x = W.activation(60, m, k)
    codes, scale = fp8w.fp8w_quantize_act(to_dev_bf16(x))
    _sync()
    rc, rs = oracle_mod.quantize_act_tensor(x)
    assert np.float32(scale.item()) == np.float32(rs)
    assert np.array_equal(codes.cpu().numpy(), rc)


def test_quantize_act_zero_outlier_and_misaligned(fp8w, oracle_mod):
    import torch
    z = np.zeros((16, 2048), dtype=np.uint16)
    z[3, 5] = 0x8000                                   # -0.0
    c, s = fp8w.fp8w_quantize_act(to_dev_bf16(z))
    _sync()
    assert s.item() == 1.0 and c.cpu().numpy()[3, 5] == 0x80 and np.count_nonzero(c.cpu().numpy()) == 1
    x = W.activation(61, 24, 2048)
    x[7, 100] = 0x4F00                                 # one large outlier sets the scale for all rows
    x[2, 3] = 0x0001                                   # a bf16 subnormal
    c, s = fp8w.fp8w_quantize_act(to_dev_bf16(x))
    _sync()
    rc, rs = oracle_mod.quantize_act_tensor(x)
    assert np.float32(s.item()) == np.float32(rs) and np.array_equal(c.cpu().numpy(), rc)
    # x at an odd element offset: 2-byte aligned only, the scalar path
    buf = torch.empty(24 * 2048 + 1, dtype=torch.bfloat16, device="cuda")
    buf[1:].copy_(to_dev_bf16(x).reshape(-1))
    c, s = fp8w.fp8w_quantize_act(buf[1:].view(24, 2048))
    _sync()
    assert np.float32(s.item()) == np.float32(rs) and np.array_equal(c.cpu().numpy(), rc)


def _jobs(oracle_mod, fmt, seed):
    out = []
    for i, (n, k) in enumerate(SHAPES):
        bits = W.gaussian_weight(62 + seed, i, n, k, outlier_rows=fmt == "block", heavy_tail=fmt == "mx")
        codes, sc = oracle_mod.quantize_block(bits) if fmt == "block" else oracle_mod.quantize_mx(bits)
        out.append((n, k, codes, sc))
    return out


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_w8a8_gemv_every_m_within_bound(fp8w, oracle_mod, fmt):
    jobs = _jobs(oracle_mod, fmt, 0)
    gemv = fp8w.fp8w_gemv_block_w8a8 if fmt == "block" else fp8w.fp8w_gemv_mx_w8a8
    ref = oracle_mod.gemv_w8a8_block_f64 if fmt == "block" else oracle_mod.gemv_w8a8_mx_f64
    for m in range(1, 33):
        for idx, (n, k, c, s) in enumerate(jobs):
            if (m + idx) % 3:          # every M, each against a rotating third of the shapes
                continue
            x = W.activation(63, m, k)
            xc, xs = oracle_mod.quantize_act_tensor(x)
            xs_dev = to_dev(np.array([xs], dtype=np.float32))
            y = bf16_to_f64(gemv(to_dev(xc), xs_dev, to_dev(c), to_dev(s)))
            y_ref, bound = ref(xc, xs, c, s)
            assert_within_bound(y, y_ref, bound, f"w8a8 {fmt} m={m} [{n}x{k}]")


def test_w8a8_mx_scale_mapping_every_code_and_scale_byte(fp8w, oracle_mod):
    """Row r of the weight uses e8m0 byte r in every group; column c holds
    code NON_NAN[c % 254].  Each activation row is one-hot at a column in a
    different 32-column group and 128-column block, so each output is one
    exact product and a scale from the wrong group or lane would show."""
    non_nan = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    n, k = 246, 4096                                   # bytes 0..245: every product (|code| * |x| <= 672) finite in fp32
    codes = np.resize(non_nan, (n, k)).astype(np.uint8)
    for r in range(n):
        codes[r] = np.roll(codes[r], r)
    e8m0 = np.repeat(np.arange(n, dtype=np.uint8)[:, None], k // 32, axis=1)
    m = 32
    cols = np.array([(i * 37 + 5) % k for i in range(m)])
    xc = np.zeros((m, k), dtype=np.uint8)
    xc[np.arange(m), cols] = 0x38 + (np.arange(m) % 5)   # 1.0 .. 1.5
    xs = np.float32(0.5)
    y = bf16_to_f64(fp8w.fp8w_gemv_mx_w8a8(to_dev(xc), to_dev(np.array([xs], np.float32)), to_dev(codes),
                                           to_dev(e8m0)))
    y_ref, bound = oracle_mod.gemv_w8a8_mx_f64(xc, xs, codes, e8m0)
    assert_within_bound(y, y_ref, bound, "mx scale mapping")
    assert len({c // 32 % 4 for c in cols}) == 4 and len({c // 128 for c in cols}) > 8


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_w8a8_end_to_end_against_bf16_reference(fp8w, oracle_mod, fmt):
    """GPU activation quantization + GPU W8A8 GEMV against the bf16 oracle
    GEMV y_ref.  With y_q the oracle's fp64 product of the quantized operands
    (its own activation codes, bit-equal to the GPU's), the triangle
    inequality gives |y - y_ref| <= |y - y_q| + |y_q - y_ref|: the first term
    is the W8A8 GEMV bound 2^-7 * sum |x_q| |deq| + 1e-6 on the quantized
    operands, the second the activation's own e4m3 error carried through
    the weight, exact in fp64 and itself at most sum (2^-4 |x| + 2^-10
    x_scale) |deq| (half an ulp of a normal code relative to |x|, half the
    subnormal step 2^-9 x_scale).  No other slack than the fp64 rounding of
    the references themselves."""
    n, k = 2560, 3072
    bits = W.gaussian_weight(64, 0, n, k, outlier_rows=False, heavy_tail=fmt == "mx")
    c, s = oracle_mod.quantize_block(bits) if fmt == "block" else oracle_mod.quantize_mx(bits)
    deq = oracle_mod.dequant_block(c, s) if fmt == "block" else oracle_mod.dequant_mx(c, s)
    for m in (1, 8, 16, 32):
        x = W.activation(64, m, k)
        xc, xs = fp8w.fp8w_quantize_act(to_dev_bf16(x))
        xc_ref, xs_ref = oracle_mod.quantize_act_tensor(x)
        assert np.array_equal(xc.cpu().numpy(), xc_ref) and float(xs.item()) == xs_ref, f"{fmt} m={m}"
        gemv = fp8w.fp8w_gemv_block_w8a8 if fmt == "block" else fp8w.fp8w_gemv_mx_w8a8
        y = bf16_to_f64(gemv(xc, xs, to_dev(c), to_dev(s)))
        y_ref, bound = (oracle_mod.gemv_block_f64 if fmt == "block" else oracle_mod.gemv_mx_f64)(x, c, s)
        y_q, bound_q = (oracle_mod.gemv_w8a8_block_f64 if fmt == "block"
                        else oracle_mod.gemv_w8a8_mx_f64)(xc_ref, xs_ref, c, s)
        xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        act_err = (np.ldexp(np.abs(xf), -4) + np.ldexp(xs_ref, -10)) @ np.abs(deq).T
        act_dev = np.abs(y_q - y_ref)
        # rounding of the two fp64 reference sums (k terms each): at most
        # k * 2^-53 of each sum of magnitudes, doubled for safety
        fp64 = k * 2.0 ** -52 * (bound + bound_q)
        assert np.all(act_dev <= act_err + fp64), f"{fmt} m={m}: activation error bound"
        err = np.abs(y - y_ref)
        assert np.all(err <= np.ldexp(bound_q, -7) + 1e-6 + act_dev + fp64), f"{fmt} m={m}"
