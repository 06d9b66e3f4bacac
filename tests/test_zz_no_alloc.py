"""fp8w_quantize_act_noalloc (the activation quantizer for callers that
cannot allocate) against fp8w_quantize_act, the entry point it varies,
through the C ABI: two calls in a row on the same device array, the second
on a smaller input, then one below the single-launch size.  Codes and scale
must be bit-identical to the workspace call's, and to the oracle's."""
import ctypes

import numpy as np
import pytest

from fp8_block_scaled_02_amd import workloads as W
from gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def F():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import fp8_block_scaled_02_amd as fp8w
    fp8w.lib()
    return fp8w


def _noalloc(F, x, codes, scale):
    import torch
    L = F.lib()
    m, k = x.shape
    st = L.fp8w_quantize_act_noalloc(ctypes.c_void_p(x.data_ptr()), m, k, ctypes.c_void_p(codes.data_ptr()),
                                     ctypes.c_void_p(scale.data_ptr()),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == F.OK, F.status_string(st)


def test_noalloc_matches_workspace_call_on_consecutive_calls(F, oracle_mod):
    import torch
    # The first input has the larger magnitudes, so a partial maximum left
    # in the array by the first call would raise the second call's scale.
    shapes = [(32, 12288, 4.0), (8, 4096, 1.0), (4, 2048, 1.0)]   # 192, 16 partials, then one launch
    codes = torch.empty(32 * 12288, dtype=torch.uint8, device="cuda")
    scale = torch.empty(1, dtype=torch.float32, device="cuda")
    for i, (m, k, mag) in enumerate(shapes):
        xh = W.activation(90 + i, m, k)
        if mag != 1.0:
            xh = W._to_bf16(((xh.astype(np.uint32) << 16).view(np.float32) * mag))
        x = to_dev_bf16(xh)
        c_na = codes[: m * k].view(m, k)
        print(f"noalloc call {i}: m={m} k={k}", flush=True)
        _noalloc(F, x, c_na, scale)
        c_ws, s_ws = F.fp8w_quantize_act(x)
        torch.cuda.synchronize()
        assert torch.equal(c_na, c_ws), f"call {i}: codes differ from fp8w_quantize_act"
        assert scale.view(torch.int32).item() == s_ws.view(torch.int32).item(), f"call {i}: scale"
        rc, rs = oracle_mod.quantize_act_tensor(xh)
        assert np.array_equal(c_na.cpu().numpy(), rc) and float(scale.item()) == rs, f"call {i}: oracle"


def test_noalloc_rejects_bad_arguments(F):
    import torch
    L = F.lib()
    x = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((2, 64), dtype=torch.uint8, device="cuda")
    s = torch.empty(1, dtype=torch.float32, device="cuda")
    P = ctypes.c_void_p
    assert L.fp8w_quantize_act_noalloc(None, 2, 64, P(c.data_ptr()), P(s.data_ptr()), None) == F.ERR_NULL
    assert L.fp8w_quantize_act_noalloc(P(x.data_ptr()), 0, 64, P(c.data_ptr()), P(s.data_ptr()), None) == F.ERR_SHAPE
    assert L.fp8w_quantize_act_noalloc(P(x.data_ptr()), 2, 64, P(x.data_ptr()), P(s.data_ptr()), None) == F.ERR_OVERLAP
