"""The read-ceiling pass reads every 16-byte word of its buffer once: the
XOR of its per-workgroup words equals the XOR of all of the buffer's
dwords, computed on the host."""
import numpy as np
import pytest

from gpu_util import to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,words", [(16, 2048), (1 << 20, 2048), ((64 << 20) + 48, 2048), ((8 << 20) + 16, 7)])
def test_read_ceiling_reads_every_word(nbytes, words):
    import torch
    import fp8_block_scaled_02_amd as F
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    buf = to_dev(host.view(np.int32))
    out = torch.full((words,), -1, dtype=torch.int32, device="cuda")
    F.fp8w_read_ceiling(buf, out)
    torch.cuda.synchronize()
    blocks = min(words, -(-nbytes // 32768))
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)[:blocks])
    assert got == np.bitwise_xor.reduce(host)
    assert (out.cpu().numpy()[blocks:] == -1).all()   # nothing written past the grid
