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


def check_step_against_oracle(tag, w_after, m_after, v_after, wm_after, w_before, g_f64, ostate, hp, tol):
    """One parameter after one GPU step against one oracle step taken from the
    oracle's own state ``ostate`` (dict with w, m, v; advanced in place).

    w_after / m_after / v_after: exact float64 copies of the GPU's fp32 master,
    momentum and NorMuon variance (v_after None without NorMuon); wm_after: the
    bf16 model copy as uint16 bits, or None; w_before: the master before the
    step.  Checks the weight change (relative Frobenius error <= tol), the
    momentum (within 1 bf16 ulp, or 2^-20 (|mu m| + |g|) where the update
    cancels; fp32 momentum within max(tol, 1e-6) relative), the variance
    (<= 2 tol) and the model copy (bitwise RNE of the GPU master)."""
    import oracle
    r = oracle.muon_step(ostate["w"], g_f64, ostate["m"], ostate["v"], hp)
    err = rel_fro(w_after - w_before, r["w"] - ostate["w"])
    assert err <= tol, (tag, "dW", err)
    if hp.mom_dtype == "bf16":
        diff = bf16_ulp_diff(m_after, r["m"])
        scale = hp.momentum * np.abs(ostate["m"]) + np.abs(g_f64)
        off = (diff > 1) & (np.abs(m_after - r["m"]) > 2.0 ** -20 * scale)
        assert not off.any(), (tag, "momentum", int(off.sum()))
    else:
        assert rel_fro(m_after, r["m"]) <= max(tol, 1e-6), (tag, "momentum")
    if hp.normuon:
        assert rel_fro(v_after, r["v"]) <= 2 * tol, (tag, "variance")
    if wm_after is not None:
        assert np.array_equal(wm_after, synth.f64_to_bf16_bits(w_after)), (tag, "model copy")
    ostate.update(w=r["w"], m=r["m"], v=r["v"])
    return err
