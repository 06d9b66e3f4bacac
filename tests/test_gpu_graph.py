"""A decode step of library calls captured in one HIP graph: activation
quantization and W8A8 GEMVs, W8A16 single calls on the streaming kernels
(one job passed by value), MX single and grouped calls and dequantization.
The graph is replayed several times, with eager work and synchronizations
between replays, and every replay must reproduce the eager results bit for
bit; the eager results themselves are checked against the oracle.  The
large-M route (dequantize + rocBLAS) is captured on its own once its
rocBLAS handle exists, and refuses to create one under capture."""
import os
import subprocess
import sys

import numpy as np
import pytest

from fp8_block_scaled_02_amd import workloads as W
from gpu_util import assert_within_bound, bf16_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


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


def test_decode_step_replays_in_a_graph(fp8w, oracle_mod):
    import torch
    big_n, small_n, k = 33000, 1030, 2048
    wb = W.gaussian_weight(95, 0, big_n, k, outlier_rows=True)
    ws = W.gaussian_weight(95, 1, small_n, k, heavy_tail=True)
    cb, sb = oracle_mod.quantize_block(wb)
    cm, em = oracle_mod.quantize_mx(ws)
    cbd, sbd, cmd, emd = to_dev(cb), to_dev(sb), to_dev(cm), to_dev(em)
    x1, x16, x17 = (W.activation(95, m, k) for m in (1, 16, 17))
    x1d, x16d, x17d = to_dev_bf16(x1), to_dev_bf16(x16), to_dev_bf16(x17)
    ws_act = torch.empty(int(fp8w.lib().fp8w_quantize_act_workspace_bytes()), dtype=torch.uint8, device="cuda")
    xc1 = torch.empty((1, k), dtype=torch.uint8, device="cuda")
    xs1 = torch.empty(1, dtype=torch.float32, device="cuda")
    xc16 = torch.empty((16, k), dtype=torch.uint8, device="cuda")
    xs16 = torch.empty(1, dtype=torch.float32, device="cuda")
    out = {name: torch.empty(shape, dtype=torch.bfloat16, device="cuda") for name, shape in {
        "w16_m1": (1, big_n), "w16_m17": (17, big_n), "w8_m1": (1, big_n), "w8_m16": (16, big_n),
        "mx_m1": (1, small_n), "mx_m16": (16, small_n)}.items()}
    deq = torch.empty((small_n, k), dtype=torch.bfloat16, device="cuda")
    plan = fp8w.fp8w_grouped_plan_init([x1d], [cmd], [emd], fmt="mx")
    codes_out = [xc1, xs1, xc16, xs16]

    def step():
        fp8w.fp8w_quantize_act(x1d, xc1, xs1, ws_act)
        fp8w.fp8w_quantize_act(x16d, xc16, xs16, ws_act)
        fp8w.fp8w_gemv_w8a8(xc1, xs1, cbd, sbd, "block", y=out["w8_m1"])
        fp8w.fp8w_gemv_w8a8(xc16, xs16, cbd, sbd, "block", y=out["w8_m16"])
        fp8w.fp8w_gemv_block(x1d, cbd, sbd, y=out["w16_m1"])
        fp8w.fp8w_gemv_block(x17d, cbd, sbd, y=out["w16_m17"])
        fp8w.fp8w_gemv_mx(x1d, cmd, emd, y=out["mx_m1"])
        fp8w.fp8w_gemv_mx(x16d, cmd, emd, y=out["mx_m16"])
        fp8w.fp8w_gemv_grouped(plan)
        fp8w.fp8w_dequantize(cmd, emd, "mx", w=deq)

    step()
    _sync()
    results = list(out.values()) + plan.ys + [deq] + codes_out
    eager = [t.clone() for t in results]

    # the eager step against the oracle
    for name, x, c, s, ref in (("w16_m1", x1, cb, sb, oracle_mod.gemv_block_f64),
                               ("w16_m17", x17, cb, sb, oracle_mod.gemv_block_f64),
                               ("mx_m1", x1, cm, em, oracle_mod.gemv_mx_f64),
                               ("mx_m16", x16, cm, em, oracle_mod.gemv_mx_f64)):
        rows = np.array([0, 1, 127, 128, 5000, c.shape[0] - 1]) if c.shape[0] > 5000 else None
        y_ref, bound = ref(x, c, s, rows=rows)
        y = bf16_to_f64(out[name])
        assert_within_bound(y if rows is None else y[:, rows], y_ref, bound, name)
    assert torch.equal(plan.ys[0].view(torch.int16), out["mx_m1"].view(torch.int16))
    for x, xcd, xsd, name in ((x1, xc1, xs1, "w8_m1"), (x16, xc16, xs16, "w8_m16")):
        rc, rs = oracle_mod.quantize_act_tensor(x)
        assert np.array_equal(xcd.cpu().numpy(), rc) and np.float32(xsd.item()) == np.float32(rs)
        rows = np.array([0, 1, 127, 128, 5000, big_n - 1])
        y_ref, bound = oracle_mod.gemv_w8a8_block_f64(rc, rs, cb, sb, rows=rows)
        assert_within_bound(bf16_to_f64(out[name])[:, rows], y_ref, bound, name)
    assert np.array_equal(deq.view(torch.int16).cpu().numpy().view(np.uint16), oracle_mod.dequant_mx_bf16(cm, em))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    _sync()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in results:
            t.fill_(rep + 3)                  # eager work between replays
        _sync()
        g.replay()
        _sync()
        for a, b in zip(results, eager):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                               b.view(torch.uint8) if b.dtype != torch.uint8 else b), f"replay {rep}"


def test_calls_on_concurrent_streams(fp8w, oracle_mod):
    """GEMVs of every kernel family on four streams at once, each stream
    with its own outputs (and its own activation-quantization workspace):
    the library keeps no per-call device state, so every result equals the
    one computed alone."""
    import torch
    k = 2048
    wts = [(33000, "block", 0), (1030, "mx", 1), (16500, "block", 2), (700, "block", 3)]
    dev = []
    for n, fmt, tid in wts:
        bits = W.gaussian_weight(96, tid, n, k, outlier_rows=fmt == "block", heavy_tail=fmt == "mx")
        c, s = oracle_mod.quantize_block(bits) if fmt == "block" else oracle_mod.quantize_mx(bits)
        dev.append((to_dev(c), to_dev(s), fmt))
    ms = (1, 17, 4, 32)
    xs = [to_dev_bf16(W.activation(96, m, k)) for m in ms]

    def work(i, y):
        c, s, fmt = dev[i]
        fp8w.fp8w_gemv(xs[i], c, s, fmt, y=y)
        if fmt == "block":
            xc, xsc = fp8w.fp8w_quantize_act(xs[i])
            return fp8w.fp8w_gemv_w8a8(xc, xsc, c, s, fmt)
        return None

    alone = []
    for i in range(4):
        y = torch.empty((ms[i], dev[i][0].shape[0]), dtype=torch.bfloat16, device="cuda")
        y8 = work(i, y)
        _sync()
        alone.append((y.clone(), None if y8 is None else y8.clone()))
    streams = [torch.cuda.Stream() for _ in range(4)]
    for rep in range(3):
        outs = [torch.full((ms[i], dev[i][0].shape[0]), 1.0, dtype=torch.bfloat16, device="cuda") for i in range(4)]
        _sync()
        res = []
        for i, st in enumerate(streams):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                res.append(work(i, outs[i]))
        for st in streams:
            torch.cuda.current_stream().wait_stream(st)
        _sync()
        for i in range(4):
            assert torch.equal(outs[i].view(torch.int16), alone[i][0].view(torch.int16)), f"stream {i} rep {rep}"
            if res[i] is not None:
                assert torch.equal(res[i].view(torch.int16), alone[i][1].view(torch.int16)), f"w8a8 {i} rep {rep}"


_FIRST_GEMM_UNDER_CAPTURE = r"""
import torch, fp8_block_scaled_02_amd as F
L = F.lib()
m, n, k = 64, 256, 512
x = torch.zeros((m, k), dtype=torch.bfloat16, device="cuda")
c = torch.zeros((n, k), dtype=torch.uint8, device="cuda")
s = torch.ones((2, 4), dtype=torch.float32, device="cuda")
y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
ws = torch.empty(n * k * 2, dtype=torch.uint8, device="cuda")
torch.cuda.synchronize()
side = torch.cuda.Stream()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=side):
    y.fill_(1.0)
    st = L.fp8w_gemm_block(x.data_ptr(), m, c.data_ptr(), s.data_ptr(), n, k, y.data_ptr(),
                           ws.data_ptr(), ws.numel(), side.cuda_stream)
torch.cuda.synchronize()
print("status", st, flush=True)
"""


def test_first_gemm_call_under_capture_is_refused():
    """In a fresh process (no rocBLAS handle yet), a GEMM call on a capturing
    stream returns FP8W_ERR_CAPTURE and enqueues nothing, instead of letting
    rocBLAS allocate inside the capture."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    print("fresh process: first fp8w_gemm_block under capture", flush=True)
    r = subprocess.run([sys.executable, "-c", _FIRST_GEMM_UNDER_CAPTURE], cwd=root, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert "status 7" in r.stdout, r.stdout[-2000:]


def test_gemm_route_replays_in_a_graph(fp8w, oracle_mod):
    import torch
    fp8w.fp8w_gemm_prepare()
    m, n, k = 96, 1280, 1024
    bits = W.gaussian_weight(96, 0, n, k, outlier_rows=True)
    c, s = oracle_mod.quantize_block(bits)
    x = W.activation(96, m, k)
    cd, sd, xd = to_dev(c), to_dev(s), to_dev_bf16(x)
    y = torch.empty((m, n), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(int(fp8w.lib().fp8w_gemm_workspace_bytes(n, k)), dtype=torch.uint8, device="cuda")
    fp8w.fp8w_gemm_block(xd, cd, sd, y=y, workspace=ws)
    _sync()
    eager = y.clone()
    rows = np.array([0, 1, 127, 128, 700, n - 1])
    y_ref, bound = oracle_mod.gemv_block_f64(x, c, s, rows=rows)
    assert_within_bound(bf16_to_f64(eager)[:, rows], y_ref, bound, "gemm eager")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        fp8w.fp8w_gemm_block(xd, cd, sd, y=y, workspace=ws, stream=side)
    for rep in range(4):
        y.fill_(rep + 3)
        ws.fill_(rep + 1)                     # eager work between replays
        _sync()
        g.replay()
        _sync()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
