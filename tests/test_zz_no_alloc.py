"""muon_ns_batched_noalloc (no workspace argument; the library's fixed
per-GPU scratch array) against muon_ns_batched with a caller workspace, called
through the C ABI: bitwise equal outputs (the same kernels on the same
inputs) and parity with the float64 oracle, on two calls in a row, the second
with a smaller input; sizes beyond the array are refused before anything is
enqueued; a captured call replays like eager calls."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, rel_fro, storage_f64, to_dev, to_f64, torch_cuda

import newton_schulz_ns5_amd as ns

pytestmark = pytest.mark.gpu


def noalloc_call(torch, x3, y3, cfg):
    L = ns.lib()
    return L.muon_ns_batched_noalloc(
        ctypes.c_void_p(x3.data_ptr()), ns._dt(x3), x3.stride(0), x3.stride(1),
        ctypes.c_void_p(y3.data_ptr()), ns._dt(y3), y3.stride(0), y3.stride(1),
        x3.shape[0], x3.shape[1], x3.shape[2], ctypes.byref(cfg),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("compute", ["bf16", "f32"])
def test_noalloc_equals_workspace_entry_point(compute):
    torch = torch_cuda()
    cfg = ns.ns_config(compute_dtype=compute)
    # Two calls in a row on the same array, the second smaller (its buffers
    # lie in what the first call left behind); then the first shape again.
    for k, shape in enumerate([(3, 300, 520), (2, 130, 200), (3, 300, 520)]):
        x = synth.gaussian(shape, (50, k, 0, 1, 0), compute)
        xt = to_dev(x, compute)
        y_no = torch.empty_like(xt)
        y_ws = torch.empty_like(xt)
        rc = noalloc_call(torch, xt, y_no, cfg)
        assert rc == 0, ns.lib().muon_last_error()
        ns.ns_batched(xt, y_ws, cfg=cfg)
        torch.cuda.synchronize()
        assert torch.equal(y_no, y_ws), (compute, shape)
        got, xin = to_f64(y_no), storage_f64(x, compute)
        err = max(rel_fro(got[i], oracle.newton_schulz5(xin[i])) for i in range(shape[0]))
        assert err <= TOL[compute], (compute, shape, err)


def test_noalloc_per_head_views_and_binding():
    # Strided per-head views of q [32, 128, 4096] (the split-K Gram path) through
    # the Python binding, bitwise equal to the workspace entry point.
    torch = torch_cuda()
    q = to_dev(synth.gaussian((4096, 4096), (50, 9, 0, 1, 0), "bf16"), "bf16")
    heads = ns.per_head_view(q, 32)
    a = ns.ns_batched_noalloc(heads)
    b = ns.ns_batched(heads)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_noalloc_refuses_problems_beyond_the_array():
    torch = torch_cuda()
    cfg = ns.ns_config()
    need = ns.ns_workspace_bytes(1, 4096, 14336, cfg)
    assert need > ns.NOALLOC_WORKSPACE_BYTES
    x = torch.zeros((1, 4096, 14336), dtype=torch.bfloat16, device="cuda")
    y = torch.full_like(x, 7.0)
    assert noalloc_call(torch, x, y, cfg) == -3
    assert b"scratch" in ns.lib().muon_last_error()
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())      # nothing was enqueued


def test_noalloc_graph_replay_matches_eager():
    torch = torch_cuda()
    shape = (4, 256, 640)
    cfg = ns.ns_config()
    static_x = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(static_x)
    ns.lib()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            rc = noalloc_call(torch, static_x, out, cfg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert rc == 0, ns.lib().muon_last_error()
    for step in (1, 2, 3):
        x = to_dev(synth.gaussian(shape, (51, 0, 0, step, 0), "bf16"), "bf16")
        static_x.copy_(x)
        eager = ns.ns_batched(x)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), step
