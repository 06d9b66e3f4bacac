"""Seeded synthetic inputs and the workload shapes they are drawn for.

This module holds no arithmetic of the method (no scales, no codes, no
products): it only draws weights and activations and rounds them to bf16, so
that the HIP path, the CPU oracle, the tests and the benchmark all see the
same inputs.

Recipe (every tensor is independent and reproducible):

* generator: ``numpy.random.default_rng(SeedSequence([workload, tensor_id,
  stream, ...]))``; stream 0 draws values, stream 1 the outlier or
  heavy-tail selection, stream 2 activations; weights are drawn in chunks of
  256 rows, chunk c seeded with ``[workload, tensor_id, stream, c]``;
* weights: fp32 samples of N(0, 0.02) (0.02 is the standard deviation);
  fp32 is then rounded to bf16 with round-to-nearest-even (torch's cast);
* "outlier rows": ``round(1% of N)`` distinct rows chosen without
  replacement are multiplied by 50 before rounding;
* "heavy tail": each entry independently (probability 0.005) is replaced by
  0.02 * Student-t(3) before rounding;
* activations: x ~ N(0, 1) of shape [M, K], rounded to bf16, seeded by
  ``[workload, 1000 + M, 2, K]``.

The shapes are those of the pages' decode projections and heads: the
per-rank 48-layer projection set of "feat(qwen4_exp): load-time per-tensor
FP8 dense projections" (Why: 12 x [6656x2560], 36 x [8192x2560], and one
[2560x3072] per layer), a vocab 151936 x hidden 2048 lm_head ("feat(quant):
opt-in fp8-block QAT for the lm_head", Summary), a hidden-4096 /
intermediate-12288 dense layer (the 8B model of "feat: add FP8 blockwise
weight quantization and FP8(E4M3) KV cache support", Motivation), and the
MXFP8 requantization targets ("Load-time MXFP8 requantization ..." issue).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

VALUES, SELECT, ACTIVATIONS = 0, 1, 2
SIGMA = 0.02


def _rng(workload: int, tensor_id: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([workload, tensor_id, stream, *extra]))


ROW_CHUNK = 256   # rows drawn per generator; chunks are drawn on a thread pool
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _to_bf16(vals: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits with round-to-nearest-even (torch's cast is RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def gaussian_weight(workload: int, tensor_id: int, n: int, k: int,
                    outlier_rows: bool = False, heavy_tail: bool = False) -> np.ndarray:
    """bf16 bits [n, k] of N(0, 0.02) with the optional outlier structure.

    Rows are drawn in chunks of ``ROW_CHUNK``; chunk c uses the seed
    ``[workload, tensor_id, stream, c]``, so the result does not depend on
    the number of threads.
    """
    vals = np.empty((n, k), dtype=np.float32)

    def fill(c: int) -> None:
        r0, r1 = c * ROW_CHUNK, min(n, (c + 1) * ROW_CHUNK)
        block = vals[r0:r1]
        _rng(workload, tensor_id, VALUES, c).standard_normal(block.shape, dtype=np.float32, out=block)
        block *= np.float32(SIGMA)
        if heavy_tail:
            sel = _rng(workload, tensor_id, SELECT, c)
            mask = sel.random(block.shape) < 0.005
            t = sel.standard_t(3, size=int(mask.sum())).astype(np.float32)
            block[mask] = np.float32(SIGMA) * t

    chunks = range((n + ROW_CHUNK - 1) // ROW_CHUNK)
    if len(chunks) > 1 and _THREADS > 1:
        with ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(fill, chunks))
    else:
        for c in chunks:
            fill(c)
    if outlier_rows:
        count = int(round(0.01 * n))
        rows = _rng(workload, tensor_id, SELECT).choice(n, size=count, replace=False)
        vals[rows] *= np.float32(50.0)
    return _to_bf16(vals)


def activation(workload: int, m: int, k: int) -> np.ndarray:
    """bf16 bits [m, k] of N(0, 1)."""
    vals = _rng(workload, 1000 + m, ACTIVATIONS, k).standard_normal((m, k), dtype=np.float32)
    return _to_bf16(vals)


@dataclass(frozen=True)
class Weight:
    tensor_id: int
    n: int
    k: int
    outlier_rows: bool = False
    heavy_tail: bool = False
    name: str = ""

    def bits(self, workload: int) -> np.ndarray:
        return gaussian_weight(workload, self.tensor_id, self.n, self.k,
                               self.outlier_rows, self.heavy_tail)


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    weights: Tuple[Weight, ...]
    ms: Tuple[int, ...]
    fmt: str = "block"            # "block" (128x128 fp32) or "mx" (32 x e8m0)
    notes: str = ""
    extra: dict = field(default_factory=dict)


def _projection_set() -> Tuple[Weight, ...]:
    out: List[Weight] = []
    for layer in range(48):
        n_first = 6656 if layer % 4 == 3 else 8192   # 12 of the 48 layers are 6656 wide
        out.append(Weight(2 * layer, n_first, 2560, name=f"layer{layer}.in"))
        out.append(Weight(2 * layer + 1, 2560, 3072, name=f"layer{layer}.out"))
    return tuple(out)


WORKLOADS = {
    1: Workload(1, "single_1024x1024_outlier_rows",
                (Weight(0, 1024, 1024, outlier_rows=True, name="w"),), (1,),
                notes="1% of rows x50"),
    2: Workload(2, "projection_set_48_layers",
                _projection_set(), (1, 8, 16),
                notes="12x[6656x2560] + 36x[8192x2560] + 48x[2560x3072]"),
    3: Workload(3, "lm_head_151936x2048",
                (Weight(0, 151936, 2048, name="lm_head"),), (1, 4, 16, 32)),
    4: Workload(4, "dense_layer_h4096_i12288",
                (Weight(0, 6144, 4096, name="qkv"), Weight(1, 4096, 4096, name="o"),
                 Weight(2, 24576, 4096, name="gate_up"), Weight(3, 4096, 12288, name="down")),
                (1, 4, 8, 9, 16, 32)),
    5: Workload(5, "mxfp8_8192x2560_2560x3072",
                (Weight(0, 8192, 2560, heavy_tail=True, name="a"),
                 Weight(1, 2560, 3072, heavy_tail=True, name="b")),
                (1, 8, 16), fmt="mx"),
}
