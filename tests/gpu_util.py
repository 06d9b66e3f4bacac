"""Helpers for the GPU parity tests: host <-> device copies of bf16 bit
patterns and the GEMV acceptance bound."""
import numpy as np


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev_bf16(bits: np.ndarray):
    """uint16 bf16 bit patterns -> a torch.bfloat16 tensor on the GPU."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(dev()).view(torch.bfloat16)


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_to_f64(y) -> np.ndarray:
    """GPU bf16 tensor -> float64 numpy (exact)."""
    return y.float().cpu().numpy().astype(np.float64)


def assert_within_bound(y_gpu: np.ndarray, y_ref: np.ndarray, bound: np.ndarray, what: str = ""):
    """|y - y_ref| <= 2^-7 * (|x| . |deq W|^T) + 1e-6, elementwise."""
    err = np.abs(y_gpu - y_ref)
    tol = np.ldexp(bound, -7) + 1e-6
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} outputs outside the bound; first at {tuple(i)}: "
            f"gpu={y_gpu[tuple(i)]!r} ref={y_ref[tuple(i)]!r} tol={tol[tuple(i)]!r}")
