"""MuonNS5 rejects bad geometry and hyperparameters when it is built, before
any step (on the CPU: the checks run the library's workspace query, which
touches no device memory)."""
import math

import pytest
import torch

import newton_schulz_ns5_amd as ns


def params(*shapes, dtype=torch.bfloat16):
    return [torch.nn.Parameter(torch.zeros(s, dtype=dtype)) for s in shapes]


def test_valid_configuration_reports_its_workspace():
    ps = params((256, 384), (384, 256), (8, 4, 3, 3))
    opt = ns.MuonNS5(ps, normuon=True, heads={id(ps[0]): 4}, split_rows={id(ps[1]): [256, 64, 64]})
    assert opt.workspace_bytes > 0
    assert len(opt.groups) == 3


@pytest.mark.parametrize("kw", [
    dict(heads=lambda ps: {id(ps[0]): 5}),                    # 256 rows do not split into 5 heads
    dict(split_rows=lambda ps: {id(ps[0]): [200, 50]}),       # heights sum to 250, not 256
    dict(split_rows=lambda ps: {id(ps[0]): [256, 0]}),        # empty block
    dict(split_rows=lambda ps: {id(ps[1]): [4, 4]}),          # row splits are for 2-D weights
    dict(heads=lambda ps: {id(ps[0]): 2}, split_rows=lambda ps: {id(ps[0]): [128, 128]}),
])
def test_bad_geometry_is_rejected_at_construction(kw):
    ps = params((256, 384), (8, 4, 3, 3))
    args = {k: v(ps) for k, v in kw.items()}
    with pytest.raises(ns.MuonError):
        ns.MuonNS5(ps, **args)


@pytest.mark.parametrize("kw", [dict(lr=math.nan), dict(momentum=math.inf), dict(normuon=True, beta2=1.5),
                                dict(normuon=True, norm_eps=-1.0), dict(ns_steps=0), dict(ns_eps=-1.0)])
def test_bad_hyperparameters_are_rejected_at_construction(kw):
    with pytest.raises(ns.MuonError):
        ns.MuonNS5(params((64, 96)), **kw)


def test_vectors_are_rejected():
    with pytest.raises(ns.MuonError):
        ns.MuonNS5(params((64,)))


def test_group_keeps_its_tensors_alive():
    # A Group holds raw pointers; the `keep` returned with it must hold the
    # tensors too, or memory freed (and possibly unmapped) behind the Group's
    # back would be written by the next step that uses it.
    import gc
    import weakref
    shape = (64, 96)

    def make():
        w = [torch.zeros(shape) for _ in range(2)]
        g = [torch.zeros(shape, dtype=torch.bfloat16) for _ in range(2)]
        m = [torch.zeros(shape, dtype=torch.bfloat16) for _ in range(2)]
        v = [torch.zeros(shape[0]) for _ in range(2)]
        wm = [torch.zeros(shape, dtype=torch.bfloat16) for _ in range(2)]
        refs = [weakref.ref(t) for t in w + g + m + v + wm]
        group, keep = ns._make_group(w, g, m, v, wm)
        return group, keep, refs, w[1].data_ptr()

    group, keep, refs, p1 = make()
    gc.collect()
    assert all(r() is not None for r in refs)
    assert group.w_master[1] == p1
    del keep
    gc.collect()
    assert all(r() is None for r in refs)


def test_state_dict_round_trip_and_checks():
    # state_dict / load_state_dict move the caller-owned state (master, momentum,
    # NorMuon variance) through torch.save / torch.load (weights only) and
    # refuse a mismatching layout version or geometry before copying anything.
    import io
    ps = params((64, 96), (8, 4, 3, 3))
    opt = ns.MuonNS5(ps, normuon=True)
    for i, p in enumerate(ps):
        st = opt.state[id(p)]
        st["master"].fill_(0.5 + i)
        st["mom"].fill_(-1.0 - i)
        st["var"].fill_(0.25 * (i + 1))
    buf = io.BytesIO()
    torch.save(opt.state_dict(), buf)
    buf.seek(0)
    sd = torch.load(buf, weights_only=True)
    assert sd["state_layout_version"] == ns.state_layout_version()
    ps2 = params((64, 96), (8, 4, 3, 3))
    opt2 = ns.MuonNS5(ps2, normuon=True)
    opt2.load_state_dict(sd)
    for p, q in zip(ps, ps2):
        for k in ("master", "mom", "var"):
            assert torch.equal(opt.state[id(p)][k], opt2.state[id(q)][k])
    before = [opt2.state[id(q)]["master"].clone() for q in ps2]
    bad_version = dict(sd, state_layout_version=sd["state_layout_version"] + 1)
    with pytest.raises(ns.MuonError):
        opt2.load_state_dict(bad_version)
    with pytest.raises(ns.MuonError):
        opt2.load_state_dict(dict(sd, state=sd["state"][:1]))
    shape_bad = dict(sd, state=[sd["state"][0], dict(sd["state"][1], mom=torch.zeros(8, 36, dtype=torch.bfloat16))])
    with pytest.raises(ns.MuonError):
        opt2.load_state_dict(shape_bad)
    no_var = ns.MuonNS5(params((64, 96), (8, 4, 3, 3)), normuon=False)
    with pytest.raises(ns.MuonError):
        no_var.load_state_dict(sd)                     # a NorMuon state into a plain Muon optimizer
    for q, b in zip(ps2, before):
        assert torch.equal(opt2.state[id(q)]["master"], b)
