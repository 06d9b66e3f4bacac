"""Hand-made test inputs shared by the oracle pins and the GPU parity tests."""
import numpy as np

from fp8_block_scaled_02_amd import workloads as W


def f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def edge_case_weight() -> np.ndarray:
    """[384 x 300] bf16 with hand-made tiles: all zero, a single nonzero,
    a subnormal amax, an exact +-448, huge values, negative zeros."""
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((384, 300)) * 0.02).astype(np.float32)
    w[0:128, 0:128] = 0.0                                   # all-zero tile
    w[0:128, 128:256] = 0.0
    w[5, 130] = -0.75                                       # single nonzero
    w[128:256, 0:128] = rng.standard_normal((128, 128)) * 1e-39   # subnormal amax
    w[128:256, 128:256] = np.clip(rng.standard_normal((128, 128)) * 200, -448, 448)
    w[130, 140], w[131, 141] = 448.0, -448.0
    w[256:384, 0:128] *= 1e36                               # huge values
    w[256:300, 256:300] = -0.0                              # negative zeros in the tail tile
    bits = W._to_bf16(w)
    assert np.isfinite(f32(bits)).all()
    return bits


