"""C ABI checks that need no GPU: the library loads, exports every function
the header declares, the ctypes structures match the C layout, and every
argument error is reported before anything is enqueued."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import newton_schulz_ns5_amd as m
from newton_schulz_ns5_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "muon_mi355x.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_expected_entry_points():
    names = header_functions()
    for required in ["muon_ns_batched", "muon_ns_groups", "muon_step_group", "normuon_normalize", "muon_ns_workspace_bytes",
                     "muon_step_workspace_bytes", "normuon_workspace_bytes", "muon_last_error"]:
        assert required in names


def test_library_exports_every_header_function():
    h = m.lib()
    missing = [n for n in header_functions() if not hasattr(h, n)]
    assert not missing, missing
    assert set(header_functions()) == set(_lib.SIGNATURES), "binding signatures drifted from the header"


def _c_layout():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "muon_mi355x.h"
#define F(T, f) printf(#T "." #f " %zu\n", offsetof(T, f))
int main(void) {
  printf("muon_ns_config %zu\n", sizeof(muon_ns_config));
  printf("muon_group %zu\n", sizeof(muon_group));
  printf("muon_hparams %zu\n", sizeof(muon_hparams));
  printf("muon_ns_problem %zu\n", sizeof(muon_ns_problem));
  F(muon_ns_problem, x); F(muon_ns_problem, x_dtype); F(muon_ns_problem, x_batch_stride);
  F(muon_ns_problem, x_row_stride); F(muon_ns_problem, y); F(muon_ns_problem, y_dtype);
  F(muon_ns_problem, y_batch_stride); F(muon_ns_problem, y_row_stride); F(muon_ns_problem, n);
  F(muon_ns_problem, rows); F(muon_ns_problem, cols);
  F(muon_ns_config, steps); F(muon_ns_config, a); F(muon_ns_config, b); F(muon_ns_config, c);
  F(muon_ns_config, eps); F(muon_ns_config, compute_dtype); F(muon_ns_config, schedule); F(muon_ns_config, max_batch);
  F(muon_ns_config, coeffs);
  F(muon_group, n); F(muon_group, rows); F(muon_group, cols); F(muon_group, heads); F(muon_group, grad_dtype);
  F(muon_group, mom_dtype); F(muon_group, model_dtype); F(muon_group, reserved); F(muon_group, w_master);
  F(muon_group, w_model); F(muon_group, grad); F(muon_group, mom); F(muon_group, var);
  F(muon_group, nsplit); F(muon_group, split_rows);
  F(muon_hparams, lr); F(muon_hparams, momentum); F(muon_hparams, nesterov); F(muon_hparams, weight_decay);
  F(muon_hparams, extra_scale); F(muon_hparams, normuon); F(muon_hparams, beta2); F(muon_hparams, norm_eps);
  F(muon_hparams, fan_out); F(muon_hparams, fan_in); F(muon_hparams, ns);
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    return dict((k, int(v)) for k, v in (line.split() for line in out.splitlines()))


def test_ctypes_structs_match_c_layout():
    lay = _c_layout()
    for cname, py in [("muon_ns_config", m.NSConfig), ("muon_group", m.Group), ("muon_hparams", m.HParams),
                      ("muon_ns_problem", m.NSProblem)]:
        assert ctypes.sizeof(py) == lay[cname], cname
        for fname, _ in py._fields_:
            assert getattr(py, fname).offset == lay[f"{cname}.{fname}"], (cname, fname)


def test_one_hip_runtime_per_process():
    # The library must bind to the HIP runtime torch already holds; two
    # runtimes in one process do not see each other's streams or work.
    m.lib()
    import sys
    assert "torch" in sys.modules
    assert len(_lib._hip_runtimes_mapped()) == 1, _lib._hip_runtimes_mapped()


def test_versions_and_status_strings():
    L = m.lib()
    assert L.muon_abi_version() == 4 and L.muon_state_layout_version() == 1
    for code, word in [(0, b"ok"), (-1, b"invalid"), (-2, b"unsupported"), (-3, b"workspace"), (-4, b"HIP")]:
        assert word in L.muon_status_string(code)
    assert L.muon_kernel_class_name(4) == b"update"


def test_profile_class_mask():
    L = m.lib()
    assert L.muon_profile_classes(1 << 8) == -1          # no class 8
    assert b"mask" in L.muon_last_error()
    assert L.muon_profile_classes(1 << 4) == 0
    assert L.muon_profile_classes(0xFF) == 0             # back to every class
    m.profile_classes(["update", "gram"])
    m.profile_classes()


def test_defaults():
    c = m.ns_config()
    assert (c.steps, c.compute_dtype, c.max_batch) == (5, _lib.MUON_BF16, 0)
    assert abs(c.a - 3.4445) < 1e-6 and abs(c.b + 4.775) < 1e-6 and abs(c.c - 2.0315) < 1e-6
    h = m.hparams()
    assert abs(h.lr - 0.05) < 1e-9 and abs(h.momentum - 0.95) < 1e-7 and h.nesterov == 1
    assert abs(h.beta2 - 0.95) < 1e-7 and abs(h.norm_eps - 1e-8) < 1e-15


FAKE = 1 << 20  # a non-null, 256-aligned address that is never dereferenced


def ns_call(**over):
    a = dict(x=FAKE, xd=1, xbs=64 * 64, xrs=64, y=FAKE, yd=1, ybs=64 * 64, yrs=64, n=1, rows=64, cols=64,
             ws=FAKE, wsb=1 << 40)
    cfg_kw = over.pop("cfg_kw", {})
    a["cfg"] = over.pop("cfg") if "cfg" in over else m.ns_config(**cfg_kw)
    a.update(over)
    L = m.lib()
    return L.muon_ns_batched(ctypes.c_void_p(a["x"]), a["xd"], a["xbs"], a["xrs"], ctypes.c_void_p(a["y"]), a["yd"],
                             a["ybs"], a["yrs"], a["n"], a["rows"], a["cols"],
                             ctypes.byref(a["cfg"]) if a["cfg"] is not None else None,
                             ctypes.c_void_p(a["ws"]), a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(x=0), -1), (dict(y=0), -1), (dict(ws=0), -1), (dict(ws=FAKE + 16), -1),
    (dict(n=-1), -1), (dict(rows=-3), -1), (dict(xrs=10), -1), (dict(yrs=63), -1), (dict(xbs=-1), -1),
    (dict(xd=7), -2), (dict(yd=2), -2), (dict(cfg_kw=dict(steps=0)), -1), (dict(cfg_kw=dict(steps=65)), -1),
    (dict(cfg=None), -1), (dict(wsb=100), -3), (dict(n=2, ybs=10), -1), (dict(x=FAKE + 1), -1),
    # y overlapping x without being x, and in place with another dtype or stride
    (dict(y=FAKE + 128), -1), (dict(n=3, y=FAKE + 64 * 64 * 2 * 2), -1), (dict(yd=0), -1), (dict(yrs=72), -1),
    (dict(rows=1 << 25), -1), (dict(rows=128, cols=(1 << 22) - 127, xrs=1 << 22, yrs=1 << 22, xbs=1 << 30,
                                     ybs=1 << 30), -1),
])
def test_ns_batched_argument_errors(over, code):
    assert ns_call(**over) == code
    assert m.lib().muon_last_error()


def test_ns_batched_noalloc_refuses_before_enqueue():
    # Argument errors and a workspace beyond the scratch array are reported
    # before the device is touched.
    L = m.lib()
    cfg = m.ns_config()

    def call(x=FAKE, y=FAKE, n=1, rows=64, cols=64, c=cfg):
        return L.muon_ns_batched_noalloc(ctypes.c_void_p(x), 1, rows * cols, cols, ctypes.c_void_p(y), 1, rows * cols,
                                         cols, n, rows, cols, ctypes.byref(c) if c is not None else None, None)
    assert call(x=0) == -1
    assert call(c=None) == -1
    assert call(y=FAKE + 64) == -1
    assert call(n=0) == 0
    assert m.ns_workspace_bytes(1, 4096, 14336, cfg) > m.NOALLOC_WORKSPACE_BYTES
    assert call(rows=4096, cols=14336, y=FAKE + (1 << 30)) == -3
    assert b"scratch" in L.muon_last_error()
    assert m.NOALLOC_WORKSPACE_BYTES == 256 << 20


def test_ns_batched_unsupported_compute_dtype():
    c = m.ns_config()
    c.compute_dtype = 5
    assert ns_call(cfg=c) == -2
    c = m.ns_config()
    c.schedule = 2
    assert ns_call(cfg=c) == -1


def test_ns_config_schedule_fields():
    sched = [(3.4445, -4.775, 2.0315)] * 4 + [(1.875, -1.25, 0.375)]
    c = m.ns_config(coeffs=sched)
    assert c.schedule == 1 and c.steps == 5
    assert abs(c.coeffs[4][0] - 1.875) < 1e-7 and abs(c.coeffs[0][2] - 2.0315) < 1e-6
    d = m.ns_config()
    assert d.schedule == 0 and abs(d.coeffs[63][1] + 4.775) < 1e-6   # defaults fill every row
    c.coeffs[2][1] = float("nan")
    assert ns_call(cfg=c) == -1
    c.coeffs[2][1] = -4.775
    c.coeffs[7][0] = float("inf")                                      # past `steps`: unused
    assert m.ns_workspace_bytes(2, 64, 96, c) > 0
    with pytest.raises(m.MuonError):
        m.ns_config(coeffs=sched[:3])


@pytest.mark.parametrize("over", [dict(n=0), dict(rows=0), dict(cols=0), dict(n=0, x=0, y=0, ws=0)])
def test_ns_batched_empty_is_noop(over):
    assert ns_call(**over) == 0


def test_ns_batched_without_gpu_reports_hip_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert ns_call() == -4
    assert b"device" in m.lib().muon_last_error().lower() or m.lib().muon_last_error()


def test_ns_workspace_query():
    c = m.ns_config()
    a = m.ns_workspace_bytes(3, 300, 520, c)
    b = m.ns_workspace_bytes(6, 300, 520, c)
    assert 0 < a < b
    assert m.ns_workspace_bytes(6, 300, 520, m.ns_config(max_batch=3)) == a
    assert m.ns_workspace_bytes(1, 520, 300, c) == m.ns_workspace_bytes(1, 300, 520, c)  # orientation
    assert m.ns_workspace_bytes(0, 300, 520, c) == 0
    f = m.ns_workspace_bytes(1, 256, 256, m.ns_config(compute_dtype="f32"))
    h = m.ns_workspace_bytes(1, 256, 256, c)
    assert f > h


def ns_problem(**over):
    a = dict(x=FAKE, xd=1, xbs=64 * 64, xrs=64, y=FAKE, yd=1, ybs=64 * 64, yrs=64, n=1, rows=64, cols=64)
    a.update(over)
    return m.NSProblem(a["x"], a["xd"], a["xbs"], a["xrs"], a["y"], a["yd"], a["ybs"], a["yrs"],
                       a["n"], a["rows"], a["cols"])


def groups_call(probs, cfg=None, ws=FAKE, wsb=1 << 40, nprob=None):
    arr = (m.NSProblem * max(len(probs), 1))(*probs)
    cfg = cfg or m.ns_config()
    n = len(probs) if nprob is None else nprob
    return m.lib().muon_ns_groups(arr if probs else None, n, ctypes.byref(cfg), ctypes.c_void_p(ws), wsb, None)


def test_ns_groups_workspace_is_the_sum_of_the_problems():
    c = m.ns_config()
    shapes = [(32, 128, 4096), (8, 128, 4096), (3, 300, 520), (0, 64, 64), (2, 520, 300)]
    assert m.ns_groups_workspace_bytes(shapes, c) == sum(m.ns_workspace_bytes(*s, c) for s in shapes)
    c3 = m.ns_config(max_batch=3)
    assert m.ns_groups_workspace_bytes(shapes, c3) == sum(m.ns_workspace_bytes(*s, c3) for s in shapes)
    assert m.ns_groups_workspace_bytes([], c) == 0


@pytest.mark.parametrize("bad,code", [
    (dict(x=0), -1), (dict(y=0), -1), (dict(xrs=10), -1), (dict(xd=7), -2), (dict(n=2, ybs=10), -1),
    (dict(rows=1 << 25), -1), (dict(x=FAKE + 1), -1), (dict(n=-1), -1),
])
def test_ns_groups_reports_the_failing_problem(bad, code):
    base = 1 << 30
    good = ns_problem(x=base, y=base)
    assert groups_call([good, ns_problem(**bad)]) == code
    assert b"problem 1" in m.lib().muon_last_error()


def test_ns_groups_argument_errors():
    base = 1 << 30
    p0 = ns_problem(x=base, y=base + (1 << 20))
    p1 = ns_problem(x=base + (2 << 20), y=base + (3 << 20))
    assert groups_call([p0, p1], ws=0) == -1
    assert groups_call([p0, p1], ws=FAKE + 16) == -1
    assert groups_call([p0, p1], wsb=100) == -3
    assert groups_call([p0, p1], nprob=-1) == -1
    assert groups_call([p0, p1], nprob=4097) == -1
    assert groups_call([], nprob=2) == -1                      # NULL array
    c = m.ns_config()
    c.steps = 0
    assert groups_call([p0, p1], cfg=c) == -1
    # outputs may not meet another problem's input or output
    assert groups_call([p0, ns_problem(x=base + (1 << 20) + 4096, y=base + (3 << 20))]) == -1
    assert b"overlaps" in m.lib().muon_last_error()
    assert groups_call([p0, ns_problem(x=base + (2 << 20), y=base + (1 << 20) + 64)]) == -1
    # in place within one problem is fine; so is sharing an input between problems
    same_in = ns_problem(x=base, y=base + (4 << 20))
    assert groups_call([p0, same_in], wsb=100) == -3           # gets past the overlap check
    assert groups_call([ns_problem(x=base, y=base), p1], wsb=100) == -3


def test_ns_groups_empty_is_noop():
    assert groups_call([]) == 0
    assert groups_call([ns_problem(n=0, x=0, y=0), ns_problem(rows=0)], ws=0, wsb=0) == 0


def group_call(hp=None, **over):
    L = m.lib()
    n = over.pop("n", 2)
    arrs = {k: (ctypes.c_void_p * max(n, 1))(*([FAKE] * max(n, 1))) for k in ["w", "g", "m", "v", "wm"]}
    for k, v in over.pop("arrays", {}).items():
        arrs[k] = v
    g = m.Group()
    g.n, g.rows, g.cols, g.heads = n, over.pop("rows", 64), over.pop("cols", 96), over.pop("heads", 1)
    g.grad_dtype, g.mom_dtype, g.model_dtype = over.pop("gd", 1), over.pop("md", 1), over.pop("mdl", -1)
    g.reserved = over.pop("reserved", 0)
    split = over.pop("split", None)
    if split is not None:
        keep_split = (ctypes.c_int64 * max(len(split), 1))(*split)
        g.nsplit = over.pop("nsplit", len(split))
        g.split_rows = None if over.pop("split_null", False) else ctypes.cast(keep_split, ctypes.POINTER(ctypes.c_int64))
    P = ctypes.POINTER(ctypes.c_void_p)
    g.w_master = ctypes.cast(arrs["w"], P) if arrs["w"] is not None else None
    g.grad = ctypes.cast(arrs["g"], P) if arrs["g"] is not None else None
    g.mom = ctypes.cast(arrs["m"], P) if arrs["m"] is not None else None
    g.var = ctypes.cast(arrs["v"], P) if arrs["v"] is not None else None
    g.w_model = ctypes.cast(arrs["wm"], P) if arrs["wm"] is not None else None
    hp = hp or m.hparams()
    ws = over.pop("ws", FAKE)
    wsb = over.pop("wsb", 1 << 40)
    assert not over, over
    return L.muon_step_group(ctypes.byref(g), ctypes.byref(hp), ctypes.c_void_p(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(heads=0), -1), (dict(heads=5), -1), (dict(gd=3), -2), (dict(md=9), -2), (dict(mdl=0), -2),
    (dict(reserved=2), -1), (dict(arrays={"w": None}), -1), (dict(arrays={"g": None}), -1),
    (dict(arrays={"m": None}), -1), (dict(mdl=1, arrays={"wm": None}), -1),
    (dict(arrays={"w": (ctypes.c_void_p * 2)(FAKE, 0)}), -1),
    (dict(arrays={"g": (ctypes.c_void_p * 2)(FAKE, FAKE + 8)}), -1),
    (dict(wsb=1000), -3), (dict(ws=0), -1), (dict(rows=-1), -1),
    # row splits: heights must be positive and sum to rows; heads must be 1
    (dict(split=[32, 16]), -1), (dict(split=[64, 0]), -1), (dict(split=[80, -16]), -1),
    (dict(split=[32, 32], heads=2), -1), (dict(split=[32, 32], split_null=True), -1),
    (dict(split=[32, 32], nsplit=-1), -1), (dict(split=[32, 32], wsb=1000), -3),
])
def test_step_group_argument_errors(kw, code):
    assert group_call(**kw) == code


def test_step_group_normuon_needs_var():
    hp = m.hparams(normuon=True)
    assert group_call(hp=hp, arrays={"v": None}) == -1
    hp = m.hparams(normuon=True, beta2=1.5)
    assert group_call(hp=hp) == -1


def test_step_group_bad_hparams():
    assert group_call(hp=m.hparams(lr=float("nan"))) == -1
    assert group_call(hp=m.hparams(fan_out=-1)) == -1
    assert group_call(hp=m.hparams(ns=m.ns_config(steps=0))) == -1


@pytest.mark.parametrize("kw", [dict(n=0), dict(rows=0), dict(cols=0)])
def test_step_group_empty_is_noop(kw):
    assert group_call(**kw) == 0


def test_step_workspace_scales_with_heads_and_batch():
    hp = m.hparams()
    g = m.Group()
    g.n, g.rows, g.cols, g.heads, g.grad_dtype, g.mom_dtype, g.model_dtype = 4, 4096, 4096, 32, 1, 1, -1
    per_head = m.step_workspace_bytes(g, hp)
    g.heads = 1
    whole = m.step_workspace_bytes(g, hp)
    assert per_head < whole     # 32 Gram matrices of 128^2 instead of one 4096^2
    hp2 = m.hparams(ns=m.ns_config(max_batch=1))
    assert m.step_workspace_bytes(g, hp2) < whole


def _split_group(n, rows, cols, hs, keep):
    arr = (ctypes.c_void_p * n)(*([FAKE] * n))
    g = m.Group()
    g.n, g.rows, g.cols, g.heads = n, rows, cols, 1
    g.grad_dtype, g.mom_dtype, g.model_dtype = 1, 1, -1
    P = ctypes.POINTER(ctypes.c_void_p)
    g.w_master = g.grad = g.mom = ctypes.cast(arr, P)
    keep.append(arr)
    if hs:
        h = (ctypes.c_int64 * len(hs))(*hs)
        keep.append(h)
        g.nsplit, g.split_rows = len(hs), ctypes.cast(h, ctypes.POINTER(ctypes.c_int64))
    return g


@pytest.mark.parametrize("compute", ["bf16", "f32"])
def test_split_workspace_is_blocks_plus_output(compute):
    # A fused [q; k; v] weight (4096 + 1024 + 1024 rows): one region per row
    # block, sized as the block alone, plus the assembled output [n][rows][cols].
    hp = m.hparams(ns=m.ns_config(compute_dtype=compute))
    keep = []
    n, cols, hs = 3, 4096, [4096, 1024, 1024]
    fused = m.step_workspace_bytes(_split_group(n, sum(hs), cols, hs, keep), hp)
    blocks = sum((m.step_workspace_bytes(_split_group(n, h, cols, None, keep), hp) + 255) // 256 * 256 for h in hs)
    es = 2 if compute == "bf16" else 4
    assert fused == blocks + (n * sum(hs) * cols * es + 255) // 256 * 256


def test_split_of_one_block_matches_the_plain_group_plus_output():
    hp = m.hparams()
    keep = []
    plain = m.step_workspace_bytes(_split_group(2, 300, 130, None, keep), hp)
    one = m.step_workspace_bytes(_split_group(2, 300, 130, [300], keep), hp)
    assert one == (plain + 255) // 256 * 256 + (2 * 300 * 130 * 2 + 255) // 256 * 256


def test_normuon_argument_errors():
    L = m.lib()
    ws = ctypes.c_void_p(FAKE)
    def call(**o):
        a = dict(o=FAKE, od=1, obs=64 * 8, ors=64, n=2, rows=8, cols=64, v=FAKE, vbs=8, b2=0.95, eps=1e-8, wsb=1 << 30)
        a.update(o)
        return L.normuon_normalize(ctypes.c_void_p(a["o"]), a["od"], a["obs"], a["ors"], a["n"], a["rows"], a["cols"],
                                   ctypes.c_void_p(a["v"]), a["vbs"], a["b2"], a["eps"], ws, a["wsb"], None)
    assert call(o=0) == -1 and call(v=0) == -1 and call(od=4) == -2 and call(b2=2.0) == -1
    assert call(ors=3) == -1 and call(vbs=3) == -1 and call(wsb=10) == -3 and call(n=0) == 0


def _groups_array(specs):
    keep, gs = [], []
    for n, rows, cols, heads in specs:
        arr = (ctypes.c_void_p * max(n, 1))(*([FAKE] * max(n, 1)))
        keep.append(arr)
        g = m.Group()
        g.n, g.rows, g.cols, g.heads = n, rows, cols, heads
        g.grad_dtype, g.mom_dtype, g.model_dtype = 1, 1, -1
        P = ctypes.POINTER(ctypes.c_void_p)
        g.w_master = g.grad = g.mom = ctypes.cast(arr, P)
        gs.append(g)
    return (m.Group * max(len(gs), 1))(*gs), gs, keep


def test_step_groups_workspace_is_sum_of_groups():
    hp = m.hparams()
    specs = [(2, 4096, 4096, 1), (2, 1024, 4096, 1), (1, 300, 130, 1), (0, 64, 64, 1), (3, 512, 384, 4)]
    arr, gs, keep = _groups_array(specs)
    total = m.step_groups_workspace_bytes(gs, hp)
    each = [m.step_workspace_bytes(g, hp) for g in gs]
    assert each[3] == 0
    assert total == sum((b + 255) // 256 * 256 for b in each)
    assert m.step_groups_workspace_bytes([], hp) == 0


def test_step_groups_argument_errors():
    L = m.lib()
    hp = m.hparams()
    arr, gs, keep = _groups_array([(2, 64, 96, 1), (1, 128, 32, 1)])
    big = ctypes.c_size_t(1 << 40)
    call = lambda a, n, ws=FAKE, wsb=1 << 40: L.muon_step_groups(a, n, ctypes.byref(hp), ctypes.c_void_p(ws), wsb, None)
    assert call(arr, -1) == -1
    assert call(None, 2) == -1
    assert call(None, 0) == 0                      # nothing to do
    assert call(arr, 2, wsb=1000) == -3
    assert call(arr, 2, ws=FAKE + 16) == -1        # workspace alignment
    # An invalid second group fails the whole call before anything is enqueued.
    bad, _, keep2 = _groups_array([(2, 64, 96, 1), (1, 128, 32, 3)])
    assert call(bad, 2) == -1
    assert "heads" in m.lib().muon_last_error().decode()
    out = ctypes.c_size_t(0)
    assert L.muon_step_groups_workspace_bytes(arr, 4097, ctypes.byref(hp), ctypes.byref(out)) == -1
    del big


def test_ns_batched_largest_long_side_accepted():
    # 128 x (2^22 - 128) is the widest matrix; only the fake workspace fails.
    c = m.ns_config()
    assert m.ns_workspace_bytes(1, 128, (1 << 22) - 128, c) > 0
    with pytest.raises(m.MuonError):
        m.ns_workspace_bytes(1, 128, (1 << 22) - 127, c)
