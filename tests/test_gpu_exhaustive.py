"""Exhaustive GPU parity of the quantizers' per-element arithmetic.

A block code depends only on the element w and its tile's amax A (through
scale = fl(A/448) and fl(w/scale)); an MX code depends only on w and the
group's exponent.  Both spaces are small enough to cover completely for
bf16 inputs: every (|w|, A) pair with |w| <= A, and every (|w|, exponent)
pair with |w| at most the exponent's largest amax, compared bit for bit with
the oracle.
"""
import numpy as np
import pytest

from gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu

TILE = 128
PER_TILE = TILE * TILE


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


def _tiles_for(amax_bits):
    """Tiles of 16384 elements: element 0 is the amax A, the rest run over
    every magnitude 0..A (one sign each, alternating with the pattern), zero
    padded.  Returns bf16 bits [tiles, 16384]."""
    a = np.asarray(amax_bits, dtype=np.int32)
    per = PER_TILE - 1
    counts = (a + 1 + per - 1) // per                 # tiles for each A
    owner = np.repeat(a, counts)                      # A of each tile
    first = (np.concatenate([np.arange(c) for c in counts]) * per).astype(np.int32)
    vals = first[:, None] + np.arange(per, dtype=np.int32)[None, :]
    valid = vals <= owner[:, None]
    mags = np.where(valid, vals, 0)
    sign = ((mags + owner[:, None]) & 1) << 15
    body = (mags | np.where(valid, sign, 0)).astype(np.uint16)
    return np.concatenate([owner[:, None].astype(np.uint16), body], axis=1)


def _misaligned_bf16(bits):
    """Device copy of bf16 bits whose data pointer is only 2-byte aligned,
    which sends the quantizer down its any-shape path."""
    import torch
    n, k = bits.shape
    buf = torch.empty(n * k + 1, dtype=torch.bfloat16, device="cuda")
    buf[1:].copy_(to_dev_bf16(bits).reshape(-1))
    return buf[1:].view(n, k)


@pytest.mark.parametrize("path", ["vector", "any"])
@pytest.mark.parametrize("part", range(4))
def test_block_quantizer_every_w_amax_pair(fp8w, oracle_mod, part, path):
    """All positive finite bf16 amax values (subnormals included) split in 4
    parts; each part is one [128*T, 128] weight, one tile column, through
    the 16-byte kernel and through the any-shape kernel."""
    amax_all = np.arange(1, 0x7F80, dtype=np.int64)
    amax = amax_all[part::4]
    tiles = _tiles_for(amax)
    t = tiles.shape[0]
    bits = tiles.reshape(t, TILE, TILE).reshape(t * TILE, TILE)
    w = to_dev_bf16(bits) if path == "vector" else _misaligned_bf16(bits)
    codes, scales = fp8w.fp8w_quantize_block(w)
    _sync()
    rc, rs = oracle_mod.quantize_block(bits)
    gs = scales.cpu().numpy()
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32))
    gc = codes.cpu().numpy()
    bad = np.flatnonzero((gc != rc).any(axis=1))
    assert bad.size == 0, f"first mismatching row {bad[:5]}"


@pytest.mark.parametrize("part", range(4))
def test_block_bf16_scale_quantizer_every_w_amax_pair(fp8w, oracle_mod, part):
    """The same pairs with the scale stored as bf16: the codes divide by the
    rounded scale, a different set of divisors."""
    import torch
    amax = np.arange(1, 0x7F80, dtype=np.int64)[part::4]
    tiles = _tiles_for(amax)
    t = tiles.shape[0]
    bits = tiles.reshape(t, TILE, TILE).reshape(t * TILE, TILE)
    codes, scales = fp8w.fp8w_quantize(to_dev_bf16(bits), "block_bf16")
    _sync()
    rc, rs = oracle_mod.quantize_block_bf16(bits)
    assert np.array_equal(scales.view(torch.int16).cpu().numpy().view(np.uint16), rs)
    gc = codes.cpu().numpy()
    bad = np.flatnonzero((gc != rc).any(axis=1))
    assert bad.size == 0, f"first mismatching row {bad[:5]}"


def test_mx_quantizer_every_w_exponent_pair_and_every_amax(fp8w, oracle_mod):
    # largest bf16 amax of each exponent e (amax <= 448 * 2^e), e = -127..120
    f32 = lambda b: (np.asarray(b, np.uint32) << 16).view(np.float32)
    all_bits = np.arange(1, 0x7F80, dtype=np.int64)
    e_all = oracle_mod.e8m0_exponent(f32(all_bits))
    leaders = np.array([all_bits[e_all == e].max() for e in np.unique(e_all)], dtype=np.int64)
    rows = []
    for lead in leaders:
        mags = np.arange(lead + 1, dtype=np.int64)
        pad = (-len(mags)) % 31
        mags = np.concatenate([mags, np.zeros(pad, np.int64)]).reshape(-1, 31)
        sign = ((mags + lead) & 1) << 15
        grp = np.concatenate([np.full((mags.shape[0], 1), lead), mags | sign], axis=1)
        rows.append(grp)
    # every amax once: [A, 0, ..., 0]
    one = np.zeros((all_bits.size, 32), np.int64)
    one[:, 0] = all_bits
    rows.append(one)
    bits = np.concatenate(rows).astype(np.uint16)
    codes, e8m0 = fp8w.fp8w_quantize_mx(to_dev_bf16(bits))
    _sync()
    rc, re_ = oracle_mod.quantize_mx(bits)
    assert np.array_equal(e8m0.cpu().numpy(), re_)
    assert np.array_equal(codes.cpu().numpy(), rc)
