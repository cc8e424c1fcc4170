"""Helpers for the GPU parity tests: moving seeded inputs to the device and
exact float64 views of device results.  No arithmetic of the method here."""
import numpy as np
import pytest

import synth


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to_dev(arr, dtype):
    """numpy storage array (float32, or uint16 bf16 bits) -> CUDA tensor."""
    torch = torch_cuda()
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def to_f64(t):
    """Exact float64 copy of a CUDA float32 / bfloat16 tensor."""
    torch = torch_cuda()
    c = t.detach().cpu().contiguous()
    if c.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f64(c.view(torch.int16).numpy().view(np.uint16))
    return c.numpy().astype(np.float64)


def storage_f64(arr, dtype):
    return synth.bf16_bits_to_f64(arr) if dtype == "bf16" else np.asarray(arr, dtype=np.float64)


def rel_fro(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / d) if d > 0 else float(np.linalg.norm(x))


def max_rel_fro(xs, refs):
    return max(rel_fro(a, b) for a, b in zip(xs, refs))


def bf16_ulp_diff(a, b):
    """Elementwise distance in bf16 units in the last place between two bf16 arrays (as float64)."""
    ba = synth.f64_to_bf16_bits(a).astype(np.int32)
    bb = synth.f64_to_bf16_bits(b).astype(np.int32)
    # map sign-magnitude to a monotone integer line
    ma = np.where(ba & 0x8000, -(ba & 0x7FFF), ba)
    mb = np.where(bb & 0x8000, -(bb & 0x7FFF), bb)
    return np.abs(ma - mb)


TOL = {"bf16": 2e-2, "f32": 1e-4}
