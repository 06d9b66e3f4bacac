"""GPU parity of the grouped quantizer (many weights in one launch): codes
and scales bit-exact against the CPU oracle in every grouped format, on
shapes that take the 16-byte body and shapes (or offsets) that take the
any-shape body in the same launch; bit-identical to the single calls on
full-size weights; and HIP-graph replays."""
import numpy as np
import pytest

from fp8_block_scaled_02_amd import workloads as W
from gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu

# ragged tiles and groups; k % 8 != 0 and k % 32 != 0 take the any-shape
# bodies (block / MX), the rest the 16-byte ones
SHAPES = [(300, 1008), (130, 272), (257, 2560), (129, 4112), (64, 16), (5, 40), (1000, 784), (131, 96),
          (1, 1), (3, 129)]


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


def _weights(seed, fmt):
    return [W.gaussian_weight(60 + seed, i, n, k, outlier_rows=fmt != "mx", heavy_tail=fmt == "mx")
            for i, (n, k) in enumerate(SHAPES)]


def _offset_bf16(bits, offset):
    """A device bf16 tensor whose data starts `offset` elements into its
    storage (2-byte aligned, not 16-byte aligned for odd offsets)."""
    import torch
    n, k = bits.shape
    flat = to_dev_bf16(np.concatenate([np.zeros(offset, np.uint16), bits.reshape(-1)]))
    return torch.as_strided(flat, (n, k), (k, 1), offset)


@pytest.mark.parametrize("fmt", ["block", "block_bf16", "mx"])
def test_grouped_quantize_matches_oracle(fp8w, oracle_mod, fmt):
    bits = _weights(0, fmt)
    ws = [to_dev_bf16(b) for b in bits]
    ws[1] = _offset_bf16(bits[1], 3)     # not 16-byte aligned: the any-shape body
    plan = fp8w.fp8w_quant_plan_init(ws, fmt=fmt)
    codes, scales = fp8w.fp8w_quantize_grouped(plan)
    _sync()
    for (n, k), b, c, s in zip(SHAPES, bits, codes, scales):
        ref_c, ref_s = oracle_mod.quantize_format(b, fmt)
        assert np.array_equal(c.cpu().numpy(), ref_c), f"{fmt} [{n}x{k}] codes"
        assert np.array_equal(_bytes(s), np.ascontiguousarray(ref_s).view(np.uint8)), f"{fmt} [{n}x{k}] scales"


def _bytes(t) -> np.ndarray:
    """The raw bytes of a device tensor (bit-exact compare, NaN-safe)."""
    import torch
    return t.contiguous().cpu().view(torch.uint8).numpy()


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_grouped_quantize_equals_single_calls_on_projection_weights(fp8w, fmt):
    """Full-size projection and dense-layer weights: the grouped launch
    writes the same bytes as one fp8w_quantize call per weight."""
    import torch
    shapes = [(6656, 2560), (8192, 2560), (2560, 3072), (4096, 4096), (4096, 12288)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    ws = [(torch.randn((n, k), device="cuda", generator=gen) * 0.02).to(torch.bfloat16) for n, k in shapes]
    ws[0][17, 5:300] = 0                                   # zero groups and near-zero tiles
    ws[1][:128, :128] = 1e-30
    plan = fp8w.fp8w_quant_plan_init(ws, fmt=fmt)
    codes, scales = fp8w.fp8w_quantize_grouped(plan)
    for w, c, s in zip(ws, codes, scales):
        c1, s1 = fp8w.fp8w_quantize(w, fmt)
        _sync()
        assert torch.equal(c, c1) and torch.equal(s, s1), f"{fmt} {tuple(w.shape)}"


def test_grouped_quantize_replays_in_a_graph(fp8w):
    """Captured on a side stream, replayed four times with the outputs
    cleared by eager work between replays: every replay rewrites them."""
    import torch
    bits = _weights(1, "mx")
    ws = [to_dev_bf16(b) for b in bits]
    plan = fp8w.fp8w_quant_plan_init(ws, fmt="mx")
    codes, scales = fp8w.fp8w_quantize_grouped(plan)
    _sync()
    want = [(c.clone(), s.clone()) for c, s in zip(codes, scales)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fp8w.fp8w_quantize_grouped(plan)
    for rep in range(4):
        for c, s in zip(codes, scales):
            c.fill_(0x7F)
            s.fill_(0)
        _sync()
        g.replay()
        _sync()
        for (c, s), (wc, wsc) in zip(zip(codes, scales), want):
            assert torch.equal(c, wc) and torch.equal(s, wsc), f"replay {rep}"


def test_grouped_quantize_rejects_bad_groups(fp8w):
    import torch
    w = torch.zeros((16, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fp8w.fp8w_quant_plan_init([])
    with pytest.raises(fp8w.Fp8wError, match="UNSUPPORTED"):
        fp8w.fp8w_quant_plan_init([w], fmt="row")
    c = torch.empty((16, 16), dtype=torch.uint8, device="cuda")
    s = torch.empty((1, 1), dtype=torch.float32, device="cuda")
    with pytest.raises(fp8w.Fp8wError, match="OVERLAP"):   # two weights write the same codes
        fp8w.fp8w_quant_plan_init([w, w.clone()], codes=[c, c], scales=[s, s.clone()])


@pytest.mark.parametrize("fmt", ["block", "mx"])
def test_grouped_quantize_many_small_weights(fp8w, fmt):
    """300 weights of mixed tiny and ragged shapes in one launch: every
    workgroup finds its weight by the table search, including weights of a
    single workgroup next to each other."""
    import torch
    rng = np.random.default_rng(17)
    shapes = [(int(rng.integers(1, 300)), int(rng.choice([1, 7, 16, 32, 40, 96, 130, 256, 272]))) for _ in range(300)]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    ws = [(torch.randn((n, k), device="cuda", generator=gen) * 0.05).to(torch.bfloat16) for n, k in shapes]
    plan = fp8w.fp8w_quant_plan_init(ws, fmt=fmt)
    codes, scales = fp8w.fp8w_quantize_grouped(plan)
    _sync()
    for i, (w, c, s) in enumerate(zip(ws, codes, scales)):
        c1, s1 = fp8w.fp8w_quantize(w, fmt)
        _sync()
        assert torch.equal(c, c1) and torch.equal(s, s1), f"{fmt} weight {i} {tuple(w.shape)}"
