"""Full-size parity of the optimizer step in the launch configuration bench.py
times (one Llama-3-8B-shaped layer, c2) and for the whole 32-layer model (c5).

Both run ``step_groups`` (muon_step_groups: one call over the four shape
groups) in bf16 compute with NorMuon (beta2 0.95, eps 1e-8), bf16 momentum,
fp32 master weights and a bf16 model copy, for two steps.  Gradients follow
the power-law recipe (U diag(i^-0.7) V^T + 0.1 N(0,1)); U, V and s are drawn
once per shape.

Checks: sampled matrices against the oracle (k and v on both steps, q and
gate on step 1); every other matrix bitwise
against the same parameters stepped by per-group calls (c2) or by the
single-layer configuration (c5), since a matrix's result does not depend on
the batch it is stepped in.
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, bf16_ulp_diff, rel_fro, storage_f64, to_dev, to_f64, torch_cuda

import newton_schulz_ns5_amd as ns

pytestmark = pytest.mark.gpu

LAYER = synth.LLAMA3_8B_LAYER
WORKLOAD = 2        # key prefix of the layer workload's inputs
INDEX = {name: i for i, (name, _) in enumerate(LAYER)}
LR = 0.05


def shape_groups():
    """[(shape, [names])] in first-appearance order, as bench.py groups them."""
    out, by = [], {}
    for name, shape in LAYER:
        if shape not in by:
            by[shape] = []
            out.append((shape, by[shape]))
        by[shape].append(name)
    return out


@functools.lru_cache(maxsize=None)
def signal(shape):
    """Low-rank part of the shape's gradients (float64, host), keyed by the
    first matrix of that shape in the layer."""
    first = next(INDEX[n] for s, names in shape_groups() if s == shape for n in names)
    return synth.power_law_signal(shape, (WORKLOAD, 0, first))


def hparams():
    return dict(lr=LR, momentum=0.95, nesterov=True, normuon=True, beta2=0.95, norm_eps=1e-8,
                ns=ns.ns_config(compute_dtype="bf16"))


def new_state(torch, shape, w0):
    return {
        "w_master": w0.clone(),
        "moms": torch.zeros(shape, dtype=torch.bfloat16, device="cuda"),
        "variances": torch.zeros(shape[0], dtype=torch.float32, device="cuda"),
        "w_model": w0.to(torch.bfloat16),
    }


def groups_of(states, grads, names_by_shape):
    """step_groups arguments from per-matrix states keyed by name."""
    out = []
    for shape, names in names_by_shape:
        out.append({
            "w_master": [states[n]["w_master"] for n in names],
            "grads": [grads[n] for n in names],
            "moms": [states[n]["moms"] for n in names],
            "variances": [states[n]["variances"] for n in names],
            "w_model": [states[n]["w_model"] for n in names],
        })
    return out


def check_against_oracle(torch, name, st, before, g_bits, ostate, step):
    """One matrix after one step vs the oracle step from the oracle's own state."""
    hp = oracle.MuonHParams(lr=LR, normuon=True, mom_dtype="bf16")
    r = oracle.muon_step(ostate["w"], storage_f64(g_bits, "bf16"), ostate["m"], ostate["v"], hp)
    tol = TOL["bf16"]
    w_gpu = to_f64(st["w_master"])
    err = rel_fro(w_gpu - before, r["w"] - ostate["w"])
    assert err <= tol, (name, step, "dW", err)
    m_gpu = to_f64(st["moms"])
    diff = bf16_ulp_diff(m_gpu, r["m"])
    scale = 0.95 * np.abs(ostate["m"]) + np.abs(storage_f64(g_bits, "bf16"))
    assert not ((diff > 1) & (np.abs(m_gpu - r["m"]) > 2.0 ** -20 * scale)).any(), (name, step, "momentum")
    assert rel_fro(to_f64(st["variances"]), r["v"]) <= 2 * tol, (name, step, "variance")
    got = st["w_model"].cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, synth.f64_to_bf16_bits(w_gpu)), (name, step, "model copy")
    ostate.update(w=r["w"], m=r["m"], v=r["v"])


def test_c2_layer_grouped_step_parity():
    torch = torch_cuda()
    groups = shape_groups()
    w0 = {n: to_dev(synth.gaussian(s, (WORKLOAD, 0, INDEX[n], 0, synth.ROLE_WEIGHT), "f32", std=0.02), "f32")
          for n, s in LAYER}
    grouped = {n: new_state(torch, s, w0[n]) for n, s in LAYER}
    single = {n: new_state(torch, s, w0[n]) for n, s in LAYER}
    # name -> oracle-checked steps; gate (14336 x 4096) is the tall class whose
    # last update writes the transposed output, about 11 TFLOP of float64 work
    sampled = {"k": (1, 2), "v": (1, 2), "q": (1,), "gate": (1,)}
    ostate = {n: {"w": to_f64(w0[n]), "m": np.zeros(dict(LAYER)[n]), "v": np.zeros(dict(LAYER)[n][0])}
              for n in sampled}
    for step in (1, 2):
        bits = {n: synth.power_law_from_signal(signal(s), (WORKLOAD, 0, INDEX[n], step)) for n, s in LAYER}
        grads = {n: to_dev(bits[n], "bf16") for n in bits}
        before = {n: to_f64(grouped[n]["w_master"]) for n in sampled}
        ns.step_groups(groups_of(grouped, grads, groups), **hparams())
        for shape, names in groups:
            ns.step_groups(groups_of(single, grads, [(shape, names)]), **hparams())
        torch.cuda.synchronize()
        for n, _ in LAYER:
            for key in ("w_master", "moms", "variances", "w_model"):
                assert torch.equal(grouped[n][key], single[n][key]), (n, step, key)
        for n, steps in sampled.items():
            if step <= max(steps):
                if step in steps:
                    check_against_oracle(torch, n, grouped[n], before[n], bits[n], ostate[n], step)
                else:
                    hp = oracle.MuonHParams(lr=LR, normuon=True, mom_dtype="bf16")
                    r = oracle.muon_step(ostate[n]["w"], storage_f64(bits[n], "bf16"), ostate[n]["m"],
                                         ostate[n]["v"], hp)
                    ostate[n].update(w=r["w"], m=r["m"], v=r["v"])


def test_c5_model_step_batch_invariance_and_parity():
    """32 layers, 224 matrices (6,979,321,856 parameters) in four groups of
    64, 64, 64 and 32 matrices; per-layer noise drawn on the GPU."""
    torch = torch_cuda()
    L = 32
    groups = shape_groups()
    sig_dev = {s: torch.from_numpy(signal(s).astype(np.float32)).cuda() for s, _ in groups}
    order = [(s, [(l, n) for l in range(L) for n in names]) for s, names in groups]

    def w_init(l, n):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(synth.key_seed((5, l, INDEX[n], 0, synth.ROLE_WEIGHT)))
        return 0.02 * torch.randn(dict(LAYER)[n], generator=gen, device="cuda", dtype=torch.float32)

    def grad(l, n, step):
        return synth.power_law_device(sig_dev[dict(LAYER)[n]], (5, l, INDEX[n], step))

    state = {}
    for s, members in order:
        for l, n in members:
            state[(l, n)] = new_state(torch, s, w_init(l, n))
    picks = sorted(int(x) for x in synth.generator(5, 99).choice(L, size=2, replace=False))
    alone = {(l, n): new_state(torch, s, state[(l, n)]["w_master"]) for l in picks for n, s in LAYER}
    ostate = {(l, n): {"w": to_f64(state[(l, n)]["w_master"]), "m": np.zeros(dict(LAYER)[n]),
                       "v": np.zeros(dict(LAYER)[n][0])} for l in picks for n in ("k", "v")}
    for step in (1, 2):
        grads = {key: grad(*key, step) for key in state}
        before = {key: to_f64(state[key]["w_master"]) for key in ostate}
        args = []
        for s, members in order:
            args.append({
                "w_master": [state[k]["w_master"] for k in members],
                "grads": [grads[k] for k in members],
                "moms": [state[k]["moms"] for k in members],
                "variances": [state[k]["variances"] for k in members],
                "w_model": [state[k]["w_model"] for k in members],
            })
        ns.step_groups(args, **hparams())
        for l in picks:
            ns.step_groups(groups_of({n: alone[(l, n)] for n, _ in LAYER}, {n: grads[(l, n)] for n, _ in LAYER},
                                     groups), **hparams())
        torch.cuda.synchronize()
        for l in picks:
            for n, _ in LAYER:
                for key in ("w_master", "moms", "variances", "w_model"):
                    assert torch.equal(state[(l, n)][key], alone[(l, n)][key]), (l, n, step, key)
        for (l, n), os_ in ostate.items():
            bits = grads[(l, n)].cpu().view(torch.int16).numpy().view(np.uint16)
            check_against_oracle(torch, f"{n}{l}", state[(l, n)], before[(l, n)], bits, os_, step)
        del grads
