"""A whole optimizer step captured in a HIP graph.

The library only enqueues kernels on the caller's stream (no allocation, no
memset, no synchronization while launch timing is off), so a
``muon_step_groups`` call can be captured once and replayed.  The graph is
replayed three times, each time after new gradients are written into its
static input tensors and after eager steps of an identical copy of the state,
and every replay is compared bitwise with the eager result; a second captured
step is replayed twice and each replay is checked against the float64 oracle.
"""
import numpy as np
import pytest

import synth
from gpu_util import to_dev, torch_cuda

import newton_schulz_ns5_amd as ns

pytestmark = pytest.mark.gpu

SHAPES = [((256, 512), 2, 1), ((384, 128), 1, 1), ((512, 256), 2, 4)]   # (shape, n, heads)


def make_states(torch, seed):
    out = []
    for k, (shape, n, heads) in enumerate(SHAPES):
        w = [to_dev(synth.gaussian(shape, (seed, k, i, 0, synth.ROLE_WEIGHT), "f32", std=0.02), "f32")
             for i in range(n)]
        out.append({
            "w_master": w,
            "moms": [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)],
            "variances": [torch.zeros(shape[0], device="cuda") for _ in range(n)],
            "w_model": [t.to(torch.bfloat16) for t in w],
            "heads": heads,
        })
    return out


def grads(seed, step):
    return [[synth.power_law(shape, (seed, k, 0), (seed, k, i, step)) for i in range(n)]
            for k, (shape, n, _) in enumerate(SHAPES)]


def test_step_groups_graph_replay_matches_eager():
    torch = torch_cuda()
    hp = ns.hparams(normuon=True, ns=ns.ns_config(compute_dtype="bf16"))
    eager = make_states(torch, 31)
    graphed = make_states(torch, 31)
    static_g = [[torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
                for shape, n, _ in SHAPES]
    for st, g in zip(graphed, static_g):
        st["grads"] = g
    need = ns.step_groups_workspace_bytes([ns._make_group(st["w_master"], st["grads"], st["moms"],
                                                          st["variances"], st["w_model"], st["heads"])[0]
                                           for st in graphed], hp)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    # The captured call must not be the first use of the library in the process.
    ns.lib()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            ns.step_groups(graphed, hp=hp, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # Capture enqueues nothing: the graphed state is still the initial one.
    for a, b in zip(eager, graphed):
        for x, y in zip(a["w_master"], b["w_master"]):
            assert torch.equal(x, y)
    for step in (1, 2, 3):
        gs = grads(31, step)
        for k in range(len(SHAPES)):
            for i, g in enumerate(gs[k]):
                static_g[k][i].copy_(to_dev(g, "bf16"))
            eager[k]["grads"] = [to_dev(g, "bf16") for g in gs[k]]
        ns.step_groups(eager, hp=hp)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(eager, graphed)):
            for key in ("w_master", "moms", "variances", "w_model"):
                for x, y in zip(a[key], b[key]):
                    assert torch.equal(x, y), (step, k, key)


def test_ns_groups_graph_replay_matches_eager():
    # muon_ns_groups over per-head views of two projections (the fused
    # sum-and-polynomial path) and a ragged matrix, captured once; each replay
    # after new inputs are written equals an eager call bitwise.
    torch = torch_cuda()
    shapes = [(8, 128, 2048), (2, 128, 2048), (2, 300, 520)]
    static_x = [torch.empty(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    outs = [torch.empty_like(x) for x in static_x]
    cfg = ns.ns_config()
    need = ns.ns_groups_workspace_bytes(shapes, cfg)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    ns.lib()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            ns.ns_groups(static_x, outs, cfg=cfg, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for step in (1, 2, 3):
        xs = [to_dev(synth.gaussian(s, (35, k, 0, step, 0), "bf16"), "bf16") for k, s in enumerate(shapes)]
        for sx, x in zip(static_x, xs):
            sx.copy_(x)
        eager = ns.ns_groups(xs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o, e), step


def test_step_groups_graph_replay_matches_oracle():
    # The captured step against the float64 oracle: two replays (new
    # gradients written into the captured input tensors before each), every
    # parameter's weight change, momentum, NorMuon variance and model copy
    # checked after each replay (the head-split group per head, as the
    # oracle's per-head step).
    import oracle
    from gpu_util import TOL, check_step_against_oracle, to_f64
    torch = torch_cuda()
    hp = ns.hparams(normuon=True, ns=ns.ns_config(compute_dtype="bf16"))
    graphed = make_states(torch, 37)
    static_g = [[torch.empty(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
                for shape, n, _ in SHAPES]
    for st, g in zip(graphed, static_g):
        st["grads"] = g
    need = ns.step_groups_workspace_bytes([ns._make_group(st["w_master"], st["grads"], st["moms"],
                                                          st["variances"], st["w_model"], st["heads"])[0]
                                           for st in graphed], hp)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    ns.lib()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            ns.step_groups(graphed, hp=hp, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ostate = [[{"w": to_f64(w), "m": np.zeros(shape), "v": np.zeros(shape[0])} for w in st["w_master"]]
              for st, (shape, n, _) in zip(graphed, SHAPES)]
    for step in (1, 2):
        gs = grads(37, step)
        for k in range(len(SHAPES)):
            for i, g in enumerate(gs[k]):
                static_g[k][i].copy_(to_dev(g, "bf16"))
        before = [[to_f64(w) for w in st["w_master"]] for st in graphed]
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (shape, n, heads) in enumerate(SHAPES):
            ohp = oracle.MuonHParams(lr=0.05, normuon=True, heads=heads, mom_dtype="bf16")
            st = graphed[k]
            for i in range(n):
                wm = st["w_model"][i].cpu().view(torch.int16).numpy().view(np.uint16)
                check_step_against_oracle(
                    f"replay {step} group {k} param {i}", to_f64(st["w_master"][i]), to_f64(st["moms"][i]),
                    to_f64(st["variances"][i]), wm, before[k][i], synth.bf16_bits_to_f64(gs[k][i]), ostate[k][i],
                    ohp, TOL["bf16"])
