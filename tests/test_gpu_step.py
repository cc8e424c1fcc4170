"""GPU parity of muon_step_group and normuon_normalize against the oracle.

Compared after each step (per parameter, max over the group):
* the weight change W_after - W_before: relative Frobenius error <= tol;
* the momentum: elementwise within 1 bf16 ulp, or within 2^-20 (|mu m_prev| + |g|)
  where the update cancels (the ABI carries mu as the float 0.95f, so an exact
  fp64 zero comes out as ~1e-8 on the GPU); fp32 momentum: rel <= tol;
* the NorMuon variance: relative Frobenius error <= 2 tol (it is quadratic in O);
* the bf16 model copy: bitwise equal to RNE(GPU fp32 master).
tol = 2e-2 in bf16 compute mode, 1e-4 in fp32 compute mode.
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, bf16_ulp_diff, rel_fro, storage_f64, to_dev, to_f64, torch_cuda

import newton_schulz_ns5_amd as ns

pytestmark = pytest.mark.gpu


def make_state(cfg, n, shape, gdt, mdt, key_layer=0):
    ws = [synth.gaussian(shape, (cfg, key_layer, i, 0, synth.ROLE_WEIGHT), "f32", std=0.02) for i in range(n)]
    return ws


def grads_for(cfg, n, shape, gdt, step, power=False, gscale=1.0):
    out = []
    for i in range(n):
        if power:
            r = shape[0]
            c = int(np.prod(shape[1:]))
            g = synth.power_law((r, c), (cfg, 0, i), (cfg, 0, i, step), gdt).reshape(shape)
        else:
            g = synth.gaussian(shape, (cfg, 0, i, step, synth.ROLE_GRAD), gdt, std=gscale)
        out.append(g)
    return out


def run_steps(shape, n, gdt, mdt, compute, steps=2, normuon=False, heads=1, model_copy=False, power=False,
              cfg_id=7, lr=0.05, wd=0.0, check=None, split_rows=None, gscale=1.0):
    torch = torch_cuda()
    w0 = make_state(cfg_id, n, shape, gdt, mdt)
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
    W = [to_dev(w, "f32") for w in w0]
    M = [torch.zeros(shape, dtype=tdt[mdt], device="cuda") for _ in range(n)]
    V = [torch.zeros(shape[0], dtype=torch.float32, device="cuda") for _ in range(n)] if normuon else None
    WM = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)] if model_copy else None
    # oracle state
    ow = [w.astype(np.float64) for w in w0]
    om = [np.zeros(shape) for _ in range(n)]
    ov = [np.zeros(shape[0]) for _ in range(n)]
    hp = oracle.MuonHParams(lr=lr, weight_decay=wd, heads=heads, normuon=normuon, mom_dtype=mdt,
                            split_rows=tuple(split_rows) if split_rows else None)
    tol = TOL[compute]
    check = list(range(n)) if check is None else check
    for step in range(1, steps + 1):
        g = grads_for(cfg_id, n, shape, gdt, step, power, gscale)
        G = [to_dev(x, gdt) for x in g]
        before = [to_f64(w) for w in W]
        ns.step_group(W, G, M, V, WM, heads=heads, split_rows=split_rows, lr=lr, weight_decay=wd,
                      normuon=normuon, ns=ns.ns_config(compute_dtype=compute))
        torch.cuda.synchronize()
        for i in check:
            r = oracle.muon_step(ow[i], storage_f64(g[i], gdt), om[i], ov[i], hp)
            w_gpu = to_f64(W[i])
            dw_err = rel_fro(w_gpu - before[i], r["w"] - ow[i])
            assert dw_err <= tol, (step, i, dw_err)
            m_gpu = to_f64(M[i])
            if mdt == "bf16":
                diff = bf16_ulp_diff(m_gpu, r["m"])
                gin = storage_f64(g[i], gdt)
                scale = 0.95 * np.abs(om[i]) + np.abs(gin)
                off = (diff > 1) & (np.abs(m_gpu - r["m"]) > 2.0 ** -20 * scale)
                if off.any():
                    bad = np.argwhere(off)
                    info = [(tuple(int(t) for t in ix), m_gpu[tuple(ix)], r["m"][tuple(ix)], om[i][tuple(ix)],
                             gin[tuple(ix)]) for ix in bad[:6]]
                    raise AssertionError(f"momentum step {step} param {i}: {len(bad)} elements off by >1 ulp; "
                                         f"(index, gpu, oracle, previous m, grad): {info}")
            else:
                assert rel_fro(m_gpu, r["m"]) <= max(tol, 1e-6), (step, i)
            if normuon:
                assert rel_fro(to_f64(V[i]), r["v"]) <= 2 * tol, (step, i)
            if model_copy:
                want = synth.f64_to_bf16_bits(w_gpu)
                got = WM[i].cpu().view(torch.int16).numpy().view(np.uint16)
                assert np.array_equal(got, want), (step, i)
            ow[i], om[i] = r["w"], r["m"]
            if normuon:
                ov[i] = r["v"]
    return W, M, V


def test_c1_fp32_two_steps():
    # 256 x 256 fp32 gradient, momentum 0.95 Nesterov, lr 0.05, fp32 compute.
    run_steps((256, 256), 1, "f32", "f32", "f32", steps=2)


def test_c1_bf16_compute_two_steps():
    run_steps((256, 256), 1, "f32", "f32", "bf16", steps=2)


@pytest.mark.parametrize("compute", ["bf16", "f32"])
def test_ragged_group_normuon(compute):
    run_steps((300, 130), 3, "bf16" if compute == "bf16" else "f32", "bf16" if compute == "bf16" else "f32",
              compute, steps=2, normuon=True, model_copy=True)


def test_tall_and_wide_groups():
    run_steps((520, 200), 2, "bf16", "bf16", "bf16", steps=2)
    run_steps((200, 520), 2, "bf16", "bf16", "bf16", steps=2, normuon=True)


def test_conv_p1_shapes_tail():
    # Two (8, 4, 3, 3) convolutions, the megabatch of the flattening fix.
    run_steps((8, 4, 3, 3), 2, "bf16", "bf16", "bf16", steps=2, normuon=True, model_copy=True)


def test_per_head_step():
    run_steps((256, 384), 2, "bf16", "bf16", "bf16", steps=2, heads=4)


def test_per_head_split_gram_step():
    # Heads of 128 x 2048 (a 512 x 2048 parameter, heads=4): the 128-row path
    # with a split Gram, where the norm of the momentum update comes from the
    # first Gram's chunk sums of squares of its bf16 rounding, the fused
    # update / Gram kernel and its update-only last iteration; NorMuon and the
    # bf16 model copy on the whole parameter.
    run_steps((512, 2048), 2, "bf16", "bf16", "bf16", steps=2, heads=4, normuon=True, model_copy=True)


@pytest.mark.parametrize("normuon", [False, True])
def test_split_qkv_step(normuon):
    # A fused [q; k; v] weight of 384 x 256 split into 256 + 64 + 64 rows (the
    # 4:1:1 grouped-query ratio of the Llama-3-8B attention), two steps; the
    # scale sqrt(384 / 256) comes from the whole parameter.
    run_steps((384, 256), 2, "bf16", "bf16", "bf16", steps=2, normuon=normuon, power=True, model_copy=True,
              split_rows=[256, 64, 64])


def test_split_ragged_blocks_f32():
    # Blocks of 100, 37 and 3 rows (wide, wide, wide; the last a 3 x 96 sliver)
    # in fp32 compute.
    run_steps((140, 96), 2, "f32", "f32", "f32", steps=2, normuon=True, split_rows=[100, 37, 3])


def test_split_tall_blocks():
    # Blocks taller than wide take the transposed orientation inside the split.
    run_steps((448, 128), 1, "bf16", "bf16", "bf16", steps=2, split_rows=[320, 128])


def test_split_blocks_step_like_their_own_groups_bitwise():
    # Without NorMuon a row block of a split parameter steps bitwise like the
    # same rows stepped as a parameter of their own, given the same lr scale
    # (fan_out / fan_in pinned to the whole parameter's).
    torch = torch_cuda()
    shape, hs, n = (384, 512), [256, 64, 64], 2
    g = [to_dev(x, "bf16") for x in grads_for(9, n, shape, "bf16", 1, power=True)]
    w = [to_dev(x, "f32") for x in make_state(9, n, shape, "bf16", "bf16")]
    m = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    hp = dict(fan_out=shape[0], fan_in=shape[1])
    parts = []
    r0 = 0
    for h in hs:
        parts.append({"w_master": [x[r0:r0 + h].clone() for x in w], "grads": [x[r0:r0 + h].contiguous() for x in g],
                      "moms": [x[r0:r0 + h].clone() for x in m]})
        r0 += h
    ns.step_groups([{"w_master": w, "grads": g, "moms": m, "split_rows": hs}], **hp)
    ns.step_groups(parts, **hp)
    torch.cuda.synchronize()
    r0 = 0
    for k, h in enumerate(hs):
        for i in range(n):
            assert torch.equal(w[i][r0:r0 + h], parts[k]["w_master"][i]), (k, i)
            assert torch.equal(m[i][r0:r0 + h], parts[k]["moms"][i]), (k, i)
        r0 += h


def test_split_step_is_independent_of_max_batch_bitwise():
    # Three fused [q; k; v] weights stepped in passes of 2 (max_batch) or all at
    # once, with NorMuon: bitwise the same.
    torch = torch_cuda()
    shape, hs, n = (384, 256), [256, 64, 64], 3
    g = [to_dev(x, "bf16") for x in grads_for(10, n, shape, "bf16", 1, power=True)]

    def state():
        return {"w_master": [to_dev(x, "f32") for x in make_state(10, n, shape, "bf16", "bf16")],
                "grads": g, "moms": [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)],
                "variances": [torch.zeros(shape[0], device="cuda") for _ in range(n)], "split_rows": hs}

    a, b = state(), state()
    ns.step_groups([a], normuon=True)
    ns.step_groups([b], normuon=True, ns=ns.ns_config(max_batch=2))
    torch.cuda.synchronize()
    for key in ("w_master", "moms", "variances"):
        for x, y in zip(a[key], b[key]):
            assert torch.equal(x, y), key


def test_weight_decay_and_gate_shape_lr():
    # fan_out / fan_in = 3.5 > 1 scales lr by sqrt(3.5).
    run_steps((448, 128), 1, "bf16", "bf16", "bf16", steps=1, wd=0.1)


def test_c4_conv_megabatches_normuon_two_steps():
    # Conv2d [64, 256, 128, 3, 3] and Conv1d [32, 512, 512, 5], bf16 power-law
    # gradients, bf16 momentum, fp32 master, NorMuon beta2 0.95 eps 1e-8.
    for name, n, shape in synth.conv_megabatches():
        run_steps(shape, n, "bf16", "bf16", "bf16", steps=2, normuon=True, power=True, cfg_id=4,
                  check=[0, n // 2, n - 1], model_copy=True)


# A convolution weight [out, *rest] steps bitwise like the [out, prod(rest)]
# weight it flattens to: Conv1d, Conv2d and Conv3d shapes, megabatches of 1, 2,
# 3 and 5, with and without NorMuon, over two steps.
@pytest.mark.parametrize("shape,n", [((6, 5, 7), 1), ((8, 4, 3, 3), 2), ((4, 3, 2, 3, 3), 3), ((5, 6, 4), 5)])
@pytest.mark.parametrize("normuon", [True, False])
def test_conv_equals_reshaped_linear_bitwise(shape, n, normuon):
    torch = torch_cuda()
    rows, cols = shape[0], int(np.prod(shape[1:]))
    w = [to_dev(x, "f32") for x in make_state(5, n, shape, "bf16", "bf16")]
    w2 = [t.clone().reshape(rows, cols) for t in w]
    m = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    m2 = [torch.zeros((rows, cols), dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    v = [torch.zeros(rows, device="cuda") for _ in range(n)]
    v2 = [torch.zeros(rows, device="cuda") for _ in range(n)]
    for step in (1, 2):
        g = [to_dev(x, "bf16") for x in grads_for(5, n, shape, "bf16", step)]
        ns.step_group(w, g, m, v if normuon else None, normuon=normuon)
        ns.step_group(w2, [t.reshape(rows, cols) for t in g], m2, v2 if normuon else None, normuon=normuon)
    torch.cuda.synchronize()
    for a, b in zip(w, w2):
        assert torch.equal(a.reshape(rows, cols), b)
    for a, b in zip(m, m2):
        assert torch.equal(a.reshape(rows, cols), b)
    if normuon:
        for a, b in zip(v, v2):
            assert torch.equal(a, b)


def test_group_size_invariance_bitwise():
    # A parameter steps identically alone and inside a group of 5.
    torch = torch_cuda()
    shape = (256, 512)
    g = [to_dev(x, "bf16") for x in grads_for(6, 5, shape, "bf16", 1)]
    w = [to_dev(x, "f32") for x in make_state(6, 5, shape, "bf16", "bf16")]
    wa = [t.clone() for t in w]
    m = [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(5)]
    ma = [t.clone() for t in m]
    ns.step_group(w, g, m)
    ns.step_group([wa[3]], [g[3]], [ma[3]])
    torch.cuda.synchronize()
    assert torch.equal(w[3], wa[3]) and torch.equal(m[3], ma[3])


def test_grouped_step_equals_per_group_bitwise():
    # muon_step_groups over six shape groups (a wide, a tall, a per-head, a
    # ragged, a 128-row split-Gram and a small one, each a different GEMM tile
    # edge or orientation; more problems than one launch of the load, row
    # statistics and update kernels holds) gives every parameter exactly the
    # result of its own group's muon_step_group call, over two steps, with
    # NorMuon and the bf16 model copy.
    torch = torch_cuda()
    specs = [((256, 512), 2, 1), ((640, 256), 1, 1), ((512, 384), 2, 4), ((300, 130), 3, 1), ((128, 4096), 2, 1),
             ((96, 200), 5, 1)]

    def state(seed):
        out = []
        for k, (shape, n, h) in enumerate(specs):
            w = [to_dev(x, "f32") for x in make_state(seed + k, n, shape, "bf16", "bf16")]
            out.append({
                "w_master": w,
                "moms": [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)],
                "variances": [torch.zeros(shape[0], device="cuda") for _ in range(n)],
                "w_model": [torch.zeros(shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)],
                "heads": h,
            })
        return out

    a, b = state(20), state(20)
    for step in (1, 2):
        for k, (shape, n, h) in enumerate(specs):
            g = [to_dev(x, "bf16") for x in grads_for(20 + k, n, shape, "bf16", step, power=True)]
            a[k]["grads"] = g
            b[k]["grads"] = g
        ns.step_groups(a, normuon=True)
        for d in b:
            ns.step_group(d["w_master"], d["grads"], d["moms"], d["variances"], d["w_model"], heads=d["heads"],
                          normuon=True)
        torch.cuda.synchronize()
        for k in range(len(specs)):
            for key in ("w_master", "moms", "variances", "w_model"):
                for x, y in zip(a[k][key], b[k][key]):
                    assert torch.equal(x, y), (step, k, key)


def test_normuon_normalize_parity():
    torch = torch_cuda()
    n, rows, cols = 3, 96, 200
    o = synth.gaussian((n, rows, cols), (8, 0, 0, 1, 0), "f32") * np.linspace(0.5, 2, rows)[None, :, None]
    o = o.astype(np.float32)
    v0 = np.abs(synth.gaussian((n, rows), (8, 0, 1, 1, 0), "f32")).astype(np.float32) * 0.01
    ot = to_dev(o, "f32")
    vt = to_dev(v0, "f32")
    ns.normuon_normalize(ot, vt, beta2=0.95, eps=1e-8)
    torch.cuda.synchronize()
    got, gv = to_f64(ot), to_f64(vt)
    for i in range(n):
        ref, rv = oracle.normuon(o[i].astype(np.float64), v0[i].astype(np.float64), 0.95, 1e-8)
        assert rel_fro(got[i], ref) <= 1e-5
        assert rel_fro(gv[i], rv) <= 1e-5


@pytest.mark.parametrize("gscale", [1e-12, 1e12])
@pytest.mark.parametrize("compute", ["bf16", "f32"])
def test_step_gradient_scale(gscale, compute):
    # Momentum, the folded normalization and NorMuon at gradient scales far
    # from 1 (two steps, so the momentum term enters).
    dt = compute
    run_steps((192, 320), 2, dt, dt, compute, steps=2, normuon=True, model_copy=True, cfg_id=42, gscale=gscale)


def test_normuon_normalize_bf16_in_place():
    # bf16 o normalized in place: each element within one bf16 ulp of the
    # oracle's value rounded to bf16 (the kernel forms rho d_r o in fp32 and
    # rounds once); the fp32 variance within 1e-5.  cols = 37 leaves a ragged
    # row end.
    torch = torch_cuda()
    for n, rows, cols in ((3, 96, 200), (2, 40, 37)):
        o64 = synth.gaussian((n, rows, cols), (43, rows, 0, 1, 0), "f32").astype(np.float64)
        o64 *= np.linspace(0.25, 4.0, rows)[None, :, None]
        ob = synth.store(o64, "bf16")
        v0 = (np.abs(synth.gaussian((n, rows), (43, rows, 1, 1, 0), "f32")) * 0.01).astype(np.float32)
        ot = to_dev(ob, "bf16")
        vt = to_dev(v0, "f32")
        ns.normuon_normalize(ot, vt, beta2=0.95, eps=1e-8)
        torch.cuda.synchronize()
        got = to_f64(ot)
        gv = to_f64(vt)
        for i in range(n):
            ref, rv = oracle.normuon(synth.bf16_bits_to_f64(ob[i]), v0[i].astype(np.float64), 0.95, 1e-8)
            assert bf16_ulp_diff(got[i], ref).max() <= 1, (n, rows, cols, i)
            assert rel_fro(gv[i], rv) <= 1e-5


def test_muon_ns5_channels_last_conv_weights():
    # Conv weights stored channels_last (not row-major contiguous), fp32 and
    # bf16: MuonNS5 steps them through contiguous buffers and writes the
    # results back into the parameters; bitwise equal to the same weights
    # stored contiguous, and the update against the oracle.
    torch = torch_cuda()
    shape = (64, 32, 3, 3)
    for dt in (torch.float32, torch.bfloat16):
        w0 = synth.gaussian(shape, (44, 0, 0, 0, synth.ROLE_WEIGHT), "f32", std=0.02)
        plain = torch.nn.Parameter(to_dev(w0, "f32").to(dt))
        cl = torch.nn.Parameter(to_dev(w0, "f32").to(dt).contiguous(memory_format=torch.channels_last))
        assert not cl.is_contiguous()
        opt_p = ns.MuonNS5([plain], lr=0.05, normuon=True)
        opt_c = ns.MuonNS5([cl], lr=0.05, normuon=True)
        mdt = "bf16" if dt == torch.bfloat16 else "f32"
        master = opt_p.state[id(plain)]["master"]
        ostate = {"w": to_f64(master).reshape(64, -1), "m": np.zeros((64, 288)), "v": np.zeros(64)}
        hp = oracle.MuonHParams(lr=0.05, normuon=True, mom_dtype=mdt)
        for step in (1, 2):
            g = synth.power_law((64, 288), (44, 0, 1), (44, 0, 1, step), "bf16").reshape(shape)
            plain.grad = to_dev(g, "bf16").to(dt)
            cl.grad = plain.grad.clone().contiguous(memory_format=torch.channels_last)
            start = cl.data.clone()
            before = to_f64(master).reshape(64, -1)
            opt_p.step()
            opt_c.step()
            torch.cuda.synchronize()
            assert torch.equal(plain.data, cl.data), (dt, step)
            assert torch.equal(master, opt_c.state[id(cl)]["master"]), (dt, step)
            assert not torch.equal(cl.data, start), (dt, step)
            r = oracle.muon_step(ostate["w"], storage_f64(g, "bf16").reshape(64, -1), ostate["m"], ostate["v"], hp)
            after = to_f64(master).reshape(64, -1)
            assert rel_fro(after - before, r["w"] - ostate["w"]) <= TOL["bf16"], (dt, step)
            ostate.update(w=r["w"], m=r["m"], v=r["v"])


def test_empty_group_is_noop():
    torch = torch_cuda()
    w = [torch.zeros((0, 16), device="cuda")]
    ns.step_group(w, [torch.zeros((0, 16), dtype=torch.bfloat16, device="cuda")],
                  [torch.zeros((0, 16), dtype=torch.bfloat16, device="cuda")])
    torch.cuda.synchronize()


def test_step_with_coefficient_schedule():
    # A per-iteration schedule reaches the step through the hparams' ns config.
    torch = torch_cuda()
    sched = [oracle.QUINTIC] * 4 + [(15 / 8, -10 / 8, 3 / 8)]
    shape = (256, 384)
    g = grads_for(12, 1, shape, "bf16", 1, power=True)[0]
    w0 = make_state(12, 1, shape, "bf16", "bf16")[0]
    W, M = [to_dev(w0, "f32")], [torch.zeros(shape, dtype=torch.bfloat16, device="cuda")]
    ns.step_group(W, [to_dev(g, "bf16")], M, ns=ns.ns_config(steps=5, coeffs=sched))
    torch.cuda.synchronize()
    hp = oracle.MuonHParams(coeffs=sched, mom_dtype="bf16")
    r = oracle.muon_step(w0.astype(np.float64), storage_f64(g, "bf16"), np.zeros(shape), np.zeros(shape[0]), hp)
    assert rel_fro(to_f64(W[0]) - w0, r["w"] - w0) <= TOL["bf16"]


def test_muon_ns5_optimizer_two_steps():
    # The optimizer class end to end: bf16 and fp32 weights, a convolution, a
    # per-head weight and a fused [q; k; v] weight in one MuonNS5, NorMuon on,
    # two steps with .grad set; every parameter against its own oracle step.
    torch = torch_cuda()
    specs = [((256, 384), torch.bfloat16, 1, None), ((128, 256), torch.float32, 1, None),
             ((8, 4, 3, 3), torch.bfloat16, 1, None), ((256, 384), torch.bfloat16, 4, None),
             ((384, 256), torch.bfloat16, 1, (256, 64, 64))]
    ps, ostate, hps = [], [], []
    for k, (shape, dt, h, sp) in enumerate(specs):
        w0 = synth.gaussian(shape, (30, k, 0, 0, synth.ROLE_WEIGHT), "f32", std=0.02)
        p = torch.nn.Parameter(to_dev(w0, "f32").to(dt))
        ps.append(p)
        wq = to_f64(p.data.float())          # the master starts from the parameter's stored value
        mdt = "bf16" if dt == torch.bfloat16 else "f32"
        ostate.append({"w": wq, "m": np.zeros(shape), "v": np.zeros(shape[0])})
        hps.append(oracle.MuonHParams(lr=0.05, normuon=True, heads=h, split_rows=sp, mom_dtype=mdt))
    opt = ns.MuonNS5(ps, lr=0.05, normuon=True, heads={id(ps[3]): 4}, split_rows={id(ps[4]): [256, 64, 64]})
    for step in (1, 2):
        gbits = []
        for k, (shape, dt, h, sp) in enumerate(specs):
            r, c = shape[0], int(np.prod(shape[1:]))
            g = synth.power_law((r, c), (30, k, 1), (30, k, 1, step), "bf16").reshape(shape)
            gbits.append(g)
            ps[k].grad = to_dev(g, "bf16").to(specs[k][1])
        before = [to_f64(opt.state[id(p)]["master"]) for p in ps]
        opt.step()
        torch.cuda.synchronize()
        for k, p in enumerate(ps):
            gin = storage_f64(gbits[k], "bf16")
            r = oracle.muon_step(ostate[k]["w"], gin, ostate[k]["m"], ostate[k]["v"], hps[k])
            master = to_f64(opt.state[id(p)]["master"])
            err = rel_fro(master - before[k], r["w"] - ostate[k]["w"])
            assert err <= TOL["bf16"], (step, k, err)
            if p.dtype == torch.bfloat16:
                got = p.data.cpu().view(torch.int16).numpy().view(np.uint16)
                assert np.array_equal(got, synth.f64_to_bf16_bits(master)), (step, k)
            else:
                assert p.data.data_ptr() == opt.state[id(p)]["master"].data_ptr()
            ostate[k].update(w=r["w"], m=r["m"], v=r["v"])


def test_muon_ns5_checkpoint_resume_bitwise():
    # Two steps straight equal one step, state_dict through torch.save /
    # torch.load (weights only), a fresh optimizer on the saved parameters and
    # one more step: parameters, masters, momenta and variances bitwise.
    import io
    torch = torch_cuda()
    specs = [((256, 384), torch.bfloat16), ((128, 256), torch.float32), ((8, 4, 3, 3), torch.bfloat16)]

    def make_params():
        return [torch.nn.Parameter(to_dev(synth.gaussian(s, (36, k, 0, 0, synth.ROLE_WEIGHT), "f32", std=0.02),
                                          "f32").to(dt)) for k, (s, dt) in enumerate(specs)]

    def set_grads(ps, step):
        for k, (s, dt) in enumerate(specs):
            r, c = s[0], int(np.prod(s[1:]))
            g = synth.power_law((r, c), (36, k, 1), (36, k, 1, step), "bf16").reshape(s)
            ps[k].grad = to_dev(g, "bf16").to(dt)

    straight = make_params()
    opt = ns.MuonNS5(straight, lr=0.05, normuon=True)
    for step in (1, 2):
        set_grads(straight, step)
        opt.step()
    first = make_params()
    opt1 = ns.MuonNS5(first, lr=0.05, normuon=True)
    set_grads(first, 1)
    opt1.step()
    torch.cuda.synchronize()
    buf = io.BytesIO()
    torch.save({"params": [p.detach() for p in first], "opt": opt1.state_dict()}, buf)
    buf.seek(0)
    saved = torch.load(buf, weights_only=True, map_location="cuda")
    resumed = [torch.nn.Parameter(t.clone()) for t in saved["params"]]
    opt2 = ns.MuonNS5(resumed, lr=0.05, normuon=True)
    opt2.load_state_dict(saved["opt"])
    set_grads(resumed, 2)
    opt2.step()
    torch.cuda.synchronize()
    for a, b in zip(straight, resumed):
        assert torch.equal(a.data, b.data)
        for k in ("master", "mom", "var"):
            assert torch.equal(opt.state[id(a)][k], opt2.state[id(b)][k]), k
