"""Full-size parity of the optimizer step in the launch configuration bench.py
times (one Llama-3-8B-shaped layer, c2) and for the whole 32-layer model (c5).

Both run ``step_groups`` (muon_step_groups: one call over the four shape
groups) in bf16 compute with NorMuon (beta2 0.95, eps 1e-8), bf16 momentum,
fp32 master weights and a bf16 model copy, for two steps.  Gradients follow
the power-law recipe (U diag(i^-0.7) V^T + 0.1 N(0,1)); U, V and s are drawn
once per shape.

The GPU work of each workload runs once, in a module fixture that keeps host
copies of what the checks need; every matrix is then checked against the
oracle in a test of its own (the oracle takes tens of seconds per 4096 x
14336 matrix-step):

* c2: all seven matrices on both steps; every matrix also bitwise equal to
  the same parameters stepped by per-group calls;
* c5: all seven matrices of one seeded layer on both steps, k and v of a
  second one; both layers bitwise equal to the same layer stepped alone
  (a matrix's result does not depend on the batch it is stepped in).
"""
import functools

import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, check_step_against_oracle, to_dev, torch_cuda

import newton_schulz_ns5_amd as ns

pytestmark = pytest.mark.gpu

LAYER = synth.LLAMA3_8B_LAYER
NAMES = [n for n, _ in LAYER]
SHAPE = dict(LAYER)
WORKLOAD = 2        # key prefix of the layer workload's inputs
INDEX = {name: i for i, (name, _) in enumerate(LAYER)}
LR = 0.05
KEYS = ("w_master", "moms", "variances", "w_model")
C5_LAYERS = 32


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


def oracle_hp():
    return oracle.MuonHParams(lr=LR, normuon=True, mom_dtype="bf16")


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


def bits16(torch, t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def snapshot(torch, st):
    """Host copies of one parameter's state: fp32 master and variance, bf16
    momentum and model copy as bit patterns."""
    return {"w": st["w_master"].cpu().numpy(), "m": bits16(torch, st["moms"]),
            "v": st["variances"].cpu().numpy(), "wm": bits16(torch, st["w_model"])}


def check_two_steps(tag, w0, snaps, gbits):
    """One matrix's two GPU steps (host snapshots) against two oracle steps."""
    shape = w0.shape
    ostate = {"w": w0.astype(np.float64), "m": np.zeros(shape), "v": np.zeros(shape[0])}
    before = w0.astype(np.float64)
    errs = []
    for step in (1, 2):
        sn = snaps[step]
        w_after = sn["w"].astype(np.float64)
        errs.append(check_step_against_oracle(
            f"{tag} step {step}", w_after, synth.bf16_bits_to_f64(sn["m"]), sn["v"].astype(np.float64), sn["wm"],
            before, synth.bf16_bits_to_f64(gbits[step]), ostate, oracle_hp(), TOL["bf16"]))
        before = w_after
    print(f"{tag}: relative error of the weight change vs the oracle, steps 1-2: "
          f"{errs[0]:.3e} {errs[1]:.3e}", flush=True)


# ---- c2: one layer ---------------------------------------------------------------

@pytest.fixture(scope="module")
def c2_run():
    torch = torch_cuda()
    groups = shape_groups()
    w0 = {n: synth.gaussian(s, (WORKLOAD, 0, INDEX[n], 0, synth.ROLE_WEIGHT), "f32", std=0.02) for n, s in LAYER}
    grouped = {n: new_state(torch, s, to_dev(w0[n], "f32")) for n, s in LAYER}
    single = {n: new_state(torch, s, to_dev(w0[n], "f32")) for n, s in LAYER}
    out = {"w0": w0, "bits": {}, "snaps": {n: {} for n in NAMES}, "mismatch": []}
    for step in (1, 2):
        bits = {n: synth.power_law_from_signal(signal(s), (WORKLOAD, 0, INDEX[n], step)) for n, s in LAYER}
        grads = {n: to_dev(bits[n], "bf16") for n in bits}
        ns.step_groups(groups_of(grouped, grads, groups), **hparams())
        for shape, names in groups:
            ns.step_groups(groups_of(single, grads, [(shape, names)]), **hparams())
        torch.cuda.synchronize()
        out["mismatch"] += [(n, step, k) for n in NAMES for k in KEYS if not torch.equal(grouped[n][k], single[n][k])]
        for n in NAMES:
            out["snaps"][n][step] = snapshot(torch, grouped[n])
        out["bits"][step] = bits
        del grads
    del grouped, single
    torch.cuda.empty_cache()
    return out


@pytest.mark.timeout(600)
def test_c2_grouped_step_bitwise_equals_per_group_calls(c2_run):
    assert not c2_run["mismatch"], c2_run["mismatch"][:8]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", NAMES)
def test_c2_matrix_two_steps_against_oracle(c2_run, name):
    check_two_steps(f"c2 {name}", c2_run["w0"][name], c2_run["snaps"][name],
                    {s: c2_run["bits"][s][name] for s in (1, 2)})


# ---- c5: the 32-layer model --------------------------------------------------------

C5_PICKS = sorted(int(x) for x in synth.generator(5, 99).choice(C5_LAYERS, size=2, replace=False))
C5_ORACLE = [(C5_PICKS[0], n) for n in NAMES] + [(C5_PICKS[1], "k"), (C5_PICKS[1], "v")]


@pytest.fixture(scope="module")
def c5_run():
    """32 layers, 224 matrices (6,979,321,856 parameters) in four groups of
    64, 64, 64 and 32 matrices; per-layer noise drawn on the GPU."""
    torch = torch_cuda()
    groups = shape_groups()
    sig_dev = {s: torch.from_numpy(signal(s).astype(np.float32)).cuda() for s, _ in groups}
    order = [(s, [(l, n) for l in range(C5_LAYERS) for n in names]) for s, names in groups]

    def w_init(l, n):
        gen = torch.Generator(device="cuda")
        gen.manual_seed(synth.key_seed((5, l, INDEX[n], 0, synth.ROLE_WEIGHT)))
        return 0.02 * torch.randn(SHAPE[n], generator=gen, device="cuda", dtype=torch.float32)

    def grad(l, n, step):
        return synth.power_law_device(sig_dev[SHAPE[n]], (5, l, INDEX[n], step))

    state = {}
    for s, members in order:
        for l, n in members:
            state[(l, n)] = new_state(torch, s, w_init(l, n))
    alone = {(l, n): new_state(torch, s, state[(l, n)]["w_master"]) for l in C5_PICKS for n, s in LAYER}
    out = {"w0": {k: state[k]["w_master"].cpu().numpy() for k in C5_ORACLE}, "bits": {k: {} for k in C5_ORACLE},
           "snaps": {k: {} for k in C5_ORACLE}, "mismatch": []}
    for step in (1, 2):
        grads = {key: grad(*key, step) for key in state}
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
        for l in C5_PICKS:
            ns.step_groups(groups_of({n: alone[(l, n)] for n in NAMES}, {n: grads[(l, n)] for n in NAMES}, groups),
                           **hparams())
        torch.cuda.synchronize()
        out["mismatch"] += [(l, n, step, k) for l in C5_PICKS for n in NAMES for k in KEYS
                            if not torch.equal(state[(l, n)][k], alone[(l, n)][k])]
        for key in C5_ORACLE:
            out["snaps"][key][step] = snapshot(torch, state[key])
            out["bits"][key][step] = bits16(torch, grads[key])
        del grads, args
    del state, alone, sig_dev
    torch.cuda.empty_cache()
    return out


@pytest.mark.timeout(600)
def test_c5_sampled_layers_bitwise_equal_single_layer_steps(c5_run):
    assert not c5_run["mismatch"], c5_run["mismatch"][:8]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layer,name", C5_ORACLE)
def test_c5_matrix_two_steps_against_oracle(c5_run, layer, name):
    key = (layer, name)
    check_two_steps(f"c5 layer {layer} {name}", c5_run["w0"][key], c5_run["snaps"][key], c5_run["bits"][key])
