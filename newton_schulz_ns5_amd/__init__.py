"""MI355X (gfx950) Muon / NorMuon step: quintic Newton-Schulz orthogonalization
in hand-written HIP behind a C ABI (include/muon_mi355x.h).

This module is the thin Python binding.  PyTorch supplies device memory and
the current HIP stream; tensors are passed to the library as raw pointers with
their sizes and strides, and every step of the computation runs in the
library's kernels.  Nothing here computes on tensors.

Entry points (same names as the C ABI):

* ``ns_batched(x, out=None, ...)`` -- NS5 of each matrix of a [n, rows, cols]
  (or [rows, cols]) tensor, any batch / row strides (megabatch slices, per-head
  views from ``per_head_view``);
* ``ns_batched_noalloc(x, out=None, ...)`` -- ``ns_batched`` without a
  workspace: the library's fixed per-GPU scratch array (for callers that
  cannot allocate);
* ``ns_groups(xs, outs=None, ...)`` -- ``ns_batched`` on several tensors with
  every Newton-Schulz launch shared by all of them (e.g. the per-head views of
  q_proj and k_proj of one layer);
* ``normuon_normalize(o, v, beta2, eps)`` -- NorMuon on [n, rows, cols];
* ``step_group(...)`` -- one Muon / NorMuon step of same-shape parameters;
* ``MuonNS5`` -- a small optimizer that groups parameters by flattened shape
  and calls ``step_group`` per group.
"""
import ctypes
import math
from collections import OrderedDict

from . import _lib
from ._lib import MUON_BF16, MUON_F32, MuonError, NSConfig, NSProblem, Group, HParams, KERNEL_CLASSES

__all__ = ["ns_batched", "ns_batched_noalloc", "NOALLOC_WORKSPACE_BYTES", "ns_groups", "ns_groups_workspace_bytes", "normuon_normalize", "step_group", "step_groups", "step_groups_workspace_bytes", "MuonNS5", "per_head_view", "ns_config",
           "hparams", "ns_workspace_bytes", "step_workspace_bytes", "normuon_workspace_bytes",
           "profile_enable", "profile_classes", "profile_reset", "profile_query", "MuonError", "QUINTIC", "abi_version",
           "state_layout_version", "lib"]

QUINTIC = (3.4445, -4.7750, 2.0315)
lib = _lib.lib


def _torch():
    import torch
    return torch


def _dt(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return MUON_F32
    if t.dtype == torch.bfloat16:
        return MUON_BF16
    raise MuonError(_lib.MUON_ERR_UNSUPPORTED, f"dtype {t.dtype} is not float32 or bfloat16")


def _cdt(name):
    return {"bf16": MUON_BF16, "f32": MUON_F32, "fp32": MUON_F32}[name]


def _stream(t):
    return ctypes.c_void_p(_torch().cuda.current_stream(t.device).cuda_stream)


def abi_version():
    return lib().muon_abi_version()


def state_layout_version():
    return lib().muon_state_layout_version()


def ns_config(steps=5, coeffs=QUINTIC, eps=1e-7, compute_dtype="bf16", max_batch=0):
    """Newton-Schulz configuration.  ``coeffs`` is one (a, b, c) triple for every
    iteration, or a sequence of ``steps`` triples (a per-iteration schedule)."""
    c = NSConfig()
    lib().muon_ns_default_config(ctypes.byref(c))
    c.steps = int(steps)
    rows = [tuple(float(v) for v in t) for t in coeffs] if _is_schedule(coeffs) else None
    if rows is None:
        c.a, c.b, c.c = (float(v) for v in coeffs)
    else:
        if len(rows) != c.steps or any(len(r) != 3 for r in rows) or c.steps > _lib.NS_MAX_STEPS:
            raise MuonError(_lib.MUON_ERR_INVALID_ARG, "a schedule needs one (a, b, c) per iteration")
        c.schedule = 1
        c.a, c.b, c.c = rows[0]
        for k, r in enumerate(rows):
            for j in range(3):
                c.coeffs[k][j] = r[j]
    c.eps = float(eps)
    c.compute_dtype = _cdt(compute_dtype)
    c.max_batch = int(max_batch)
    return c


def _is_schedule(coeffs):
    try:
        return len(coeffs) > 0 and hasattr(coeffs[0], "__len__")
    except TypeError:
        return False


def hparams(lr=0.05, momentum=0.95, nesterov=True, weight_decay=0.0, extra_scale=1.0, normuon=False,
            beta2=0.95, norm_eps=1e-8, fan_out=0, fan_in=0, ns=None):
    h = HParams()
    lib().muon_default_hparams(ctypes.byref(h))
    h.lr, h.momentum, h.nesterov = float(lr), float(momentum), int(bool(nesterov))
    h.weight_decay, h.extra_scale, h.normuon = float(weight_decay), float(extra_scale), int(bool(normuon))
    h.beta2, h.norm_eps, h.fan_out, h.fan_in = float(beta2), float(norm_eps), int(fan_out), int(fan_in)
    h.ns = ns if ns is not None else ns_config()
    return h


# ---- workspace (caller-owned device memory; the library never allocates) ----
# One cached buffer per (device, stream): calls enqueued on one stream run in
# order and may share it; calls on different streams may overlap, so each
# stream gets its own.  A buffer is allocated on (and, when it grows, released
# to torch's caching allocator from) the stream that uses it.
_WS = {}


def _workspace(device, nbytes):
    torch = _torch()
    stream = torch.cuda.current_stream(device)
    key = (device.type, device.index, stream.cuda_stream)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        _WS.pop(key, None)
        buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _WS[key] = buf
    return buf


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def ns_workspace_bytes(n, rows, cols, cfg):
    out = ctypes.c_size_t(0)
    _lib.check(lib().muon_ns_workspace_bytes(int(n), int(rows), int(cols), ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def normuon_workspace_bytes(n, rows, cols):
    out = ctypes.c_size_t(0)
    _lib.check(lib().normuon_workspace_bytes(int(n), int(rows), int(cols), ctypes.byref(out)))
    return out.value


def per_head_view(p, heads):
    """[heads * hb, F] -> the [heads, hb, F] view (no copy)."""
    out, f = p.shape
    if out % heads:
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, f"rows {out} not divisible by heads {heads}")
    return p.view(heads, out // heads, f)


def _as3(t):
    if t.dim() == 2:
        return t.unsqueeze(0)
    if t.dim() == 3:
        return t
    raise MuonError(_lib.MUON_ERR_INVALID_ARG, "expected a [rows, cols] or [n, rows, cols] tensor")


def ns_batched(x, out=None, *, steps=5, coeffs=QUINTIC, eps=1e-7, compute_dtype="bf16", max_batch=0,
               cfg=None, workspace=None):
    """NS5 of each matrix of ``x`` ([rows, cols] or [n, rows, cols], unit column stride)."""
    torch = _torch()
    cfg = cfg if cfg is not None else ns_config(steps, coeffs, eps, compute_dtype, max_batch)
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    x3, y3 = _as3(x), _as3(out)
    if x3.shape != y3.shape:
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, f"out shape {tuple(out.shape)} != x shape {tuple(x.shape)}")
    if x3.numel() and (x3.stride(2) != 1 or y3.stride(2) != 1):
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, "x and out need unit column stride")
    n, rows, cols = x3.shape
    need = ns_workspace_bytes(n, rows, cols, cfg)
    ws = workspace if workspace is not None else _workspace(x.device, need)
    _lib.check(lib().muon_ns_batched(
        _ptr(x3), _dt(x3), x3.stride(0), x3.stride(1),
        _ptr(y3), _dt(y3), y3.stride(0), y3.stride(1),
        n, rows, cols, ctypes.byref(cfg), _ptr(ws), ws.numel(), _stream(x)))
    return out


def ns_batched_noalloc(x, out=None, *, steps=5, coeffs=QUINTIC, eps=1e-7, compute_dtype="bf16", max_batch=0,
                       cfg=None):
    """ns_batched through muon_ns_batched_noalloc: no workspace argument; the
    library works in its fixed per-GPU scratch array (at most
    NOALLOC_WORKSPACE_BYTES of workspace).  Calls that can overlap on one GPU
    race; calls on one stream are ordered."""
    torch = _torch()
    cfg = cfg if cfg is not None else ns_config(steps, coeffs, eps, compute_dtype, max_batch)
    if out is None:
        out = torch.empty_like(x, memory_format=torch.contiguous_format)
    x3, y3 = _as3(x), _as3(out)
    if x3.shape != y3.shape:
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, f"out shape {tuple(out.shape)} != x shape {tuple(x.shape)}")
    if x3.numel() and (x3.stride(2) != 1 or y3.stride(2) != 1):
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, "x and out need unit column stride")
    n, rows, cols = x3.shape
    _lib.check(lib().muon_ns_batched_noalloc(
        _ptr(x3), _dt(x3), x3.stride(0), x3.stride(1),
        _ptr(y3), _dt(y3), y3.stride(0), y3.stride(1),
        n, rows, cols, ctypes.byref(cfg), _stream(x)))
    return out


NOALLOC_WORKSPACE_BYTES = 256 << 20


def _ns_problems(xs, outs):
    if len(xs) != len(outs):
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, f"{len(xs)} inputs but {len(outs)} outputs")
    probs = (NSProblem * max(len(xs), 1))()
    for i, (x, y) in enumerate(zip(xs, outs)):
        x3, y3 = _as3(x), _as3(y)
        if x3.shape != y3.shape:
            raise MuonError(_lib.MUON_ERR_INVALID_ARG, f"problem {i}: out shape {tuple(y.shape)} != x shape {tuple(x.shape)}")
        if x3.numel() and (x3.stride(2) != 1 or y3.stride(2) != 1):
            raise MuonError(_lib.MUON_ERR_INVALID_ARG, f"problem {i}: x and out need unit column stride")
        n, rows, cols = x3.shape
        probs[i] = NSProblem(_ptr(x3), _dt(x3), x3.stride(0), x3.stride(1),
                             _ptr(y3), _dt(y3), y3.stride(0), y3.stride(1), n, rows, cols)
    return probs


def ns_groups_workspace_bytes(shapes, cfg):
    """Workspace of ns_groups for problems of these (n, rows, cols) shapes."""
    probs = (NSProblem * max(len(shapes), 1))()
    for i, (n, rows, cols) in enumerate(shapes):
        probs[i] = NSProblem(None, MUON_BF16, 0, cols, None, MUON_BF16, 0, cols, n, rows, cols)
    out = ctypes.c_size_t(0)
    _lib.check(lib().muon_ns_groups_workspace_bytes(probs, len(shapes), ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def ns_groups(xs, outs=None, *, steps=5, coeffs=QUINTIC, eps=1e-7, compute_dtype="bf16", max_batch=0,
              cfg=None, workspace=None):
    """ns_batched on each tensor of ``xs`` (each [rows, cols] or [n, rows, cols], unit
    column stride), one call and one set of Newton-Schulz launches for all of them."""
    torch = _torch()
    cfg = cfg if cfg is not None else ns_config(steps, coeffs, eps, compute_dtype, max_batch)
    xs = list(xs)
    if outs is None:
        outs = [torch.empty_like(x, memory_format=torch.contiguous_format) for x in xs]
    outs = list(outs)
    if not xs:
        return outs
    probs = _ns_problems(xs, outs)
    need = ns_groups_workspace_bytes([tuple(_as3(x).shape) for x in xs], cfg)
    ws = workspace if workspace is not None else _workspace(xs[0].device, need)
    _lib.check(lib().muon_ns_groups(probs, len(xs), ctypes.byref(cfg), _ptr(ws), ws.numel(), _stream(xs[0])))
    return outs


def normuon_normalize(o, v, beta2=0.95, eps=1e-8, workspace=None):
    """In place on o ([rows, cols] or [n, rows, cols]) and v ([rows] or [n, rows], fp32)."""
    o3 = _as3(o)
    v2 = v.unsqueeze(0) if v.dim() == 1 else v
    n, rows, cols = o3.shape
    if tuple(v2.shape) != (n, rows) or (v2.numel() and v2.stride(1) != 1):
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, "v must be [n, rows] with unit stride")
    if o3.numel() and o3.stride(2) != 1:
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, "o needs unit column stride")
    need = normuon_workspace_bytes(n, rows, cols)
    ws = workspace if workspace is not None else _workspace(o.device, need)
    _lib.check(lib().normuon_normalize(
        _ptr(o3), _dt(o3), o3.stride(0), o3.stride(1), n, rows, cols,
        _ptr(v2), v2.stride(0), float(beta2), float(eps), _ptr(ws), ws.numel(), _stream(o)))
    return o


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
    return arr


def _make_group(w_master, grads, moms, variances=None, w_model=None, heads=1, split_rows=None):
    n = len(w_master)
    if not (len(grads) == len(moms) == n):
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, "w_master, grads and moms must have the same length")
    shape = tuple(w_master[0].shape)
    rows = shape[0]
    cols = int(math.prod(shape[1:])) if len(shape) > 1 else 1
    for lst in (w_master, grads, moms) + ((w_model,) if w_model else ()):
        for t in lst:
            if tuple(t.shape) != shape or not t.is_contiguous():
                raise MuonError(_lib.MUON_ERR_INVALID_ARG, "group tensors must be contiguous and of one shape")
    g = Group()
    g.n, g.rows, g.cols, g.heads = n, rows, cols, int(heads)
    g.grad_dtype = _dt(grads[0])
    g.mom_dtype = _dt(moms[0])
    g.model_dtype = MUON_BF16 if w_model else -1
    # `keep` holds the pointer tables and the tensors themselves: a Group is
    # only valid while its tensors' memory is, so whoever holds the Group past
    # this call holds `keep` with it.
    keep = [_ptr_array(w_master), _ptr_array(grads), _ptr_array(moms),
            (list(w_master), list(grads), list(moms), list(variances or []), list(w_model or []))]
    g.w_master = ctypes.cast(keep[0], ctypes.POINTER(ctypes.c_void_p))
    g.grad = ctypes.cast(keep[1], ctypes.POINTER(ctypes.c_void_p))
    g.mom = ctypes.cast(keep[2], ctypes.POINTER(ctypes.c_void_p))
    if variances is not None:
        keep.append(_ptr_array(variances))
        g.var = ctypes.cast(keep[-1], ctypes.POINTER(ctypes.c_void_p))
    if w_model:
        keep.append(_ptr_array(w_model))
        g.w_model = ctypes.cast(keep[-1], ctypes.POINTER(ctypes.c_void_p))
    if split_rows:
        if len(shape) != 2:
            # Row blocks are cut on dim -2, which is the row axis of 2-D weights only.
            raise MuonError(_lib.MUON_ERR_INVALID_ARG, "split_rows needs 2-D parameters")
        keep.append((ctypes.c_int64 * len(split_rows))(*[int(h) for h in split_rows]))
        g.nsplit = len(split_rows)
        g.split_rows = ctypes.cast(keep[-1], ctypes.POINTER(ctypes.c_int64))
    return g, keep


def step_workspace_bytes(group, hp):
    out = ctypes.c_size_t(0)
    _lib.check(lib().muon_step_workspace_bytes(ctypes.byref(group), ctypes.byref(hp), ctypes.byref(out)))
    return out.value


def step_group(w_master, grads, moms, variances=None, w_model=None, *, heads=1, split_rows=None, hp=None,
               workspace=None, **kw):
    """One Muon / NorMuon step for a list of same-shape parameters (see muon_step_group).

    ``split_rows`` (a list of block heights summing to the row count) runs
    Newton-Schulz on each row block of every parameter on its own, e.g. the q,
    k and v blocks of a fused projection weight.
    """
    hp = hp if hp is not None else hparams(**kw)
    g, keep = _make_group(w_master, grads, moms, variances, w_model, heads, split_rows)
    need = step_workspace_bytes(g, hp)
    ws = workspace if workspace is not None else _workspace(w_master[0].device, need)
    _lib.check(lib().muon_step_group(ctypes.byref(g), ctypes.byref(hp), _ptr(ws), ws.numel(),
                                     _stream(w_master[0])))
    del keep
    return None


def step_groups_workspace_bytes(groups, hp):
    arr = (Group * max(1, len(groups)))(*groups)
    out = ctypes.c_size_t(0)
    _lib.check(lib().muon_step_groups_workspace_bytes(arr, len(groups), ctypes.byref(hp), ctypes.byref(out)))
    return out.value


def step_groups(groups, *, hp=None, workspace=None, **kw):
    """One Muon / NorMuon step over several shape groups in one call (see muon_step_groups).

    ``groups`` is a list of dicts with the arguments of :func:`step_group`:
    ``w_master``, ``grads``, ``moms`` and optionally ``variances``, ``w_model``,
    ``heads``, ``split_rows``.  Every parameter comes out bitwise as it would from its own
    ``step_group`` call.
    """
    hp = hp if hp is not None else hparams(**kw)
    made = [_make_group(d["w_master"], d["grads"], d["moms"], d.get("variances"), d.get("w_model"),
                        d.get("heads", 1), d.get("split_rows")) for d in groups]
    if not made:
        return None
    arr = (Group * len(made))(*[g for g, _ in made])
    need = ctypes.c_size_t(0)
    _lib.check(lib().muon_step_groups_workspace_bytes(arr, len(made), ctypes.byref(hp), ctypes.byref(need)))
    first = groups[0]["w_master"][0]
    ws = workspace if workspace is not None else _workspace(first.device, need.value)
    _lib.check(lib().muon_step_groups(arr, len(made), ctypes.byref(hp), _ptr(ws), ws.numel(), _stream(first)))
    del made
    return None


def _check_scalars(hp):
    """The scalar hyperparameter checks of muon_step_groups, run early."""
    vals = (hp.lr, hp.momentum, hp.weight_decay, hp.extra_scale)
    if not all(math.isfinite(v) for v in vals):
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, "lr, momentum, weight_decay and extra_scale must be finite")
    if hp.normuon and not (0.0 <= hp.beta2 <= 1.0 and 0.0 <= hp.norm_eps < math.inf):
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, "beta2 must be in [0,1] and norm_eps >= 0")
    if hp.fan_out < 0 or hp.fan_in < 0:
        raise MuonError(_lib.MUON_ERR_INVALID_ARG, "fan_out/fan_in must be >= 0")


class MuonNS5:
    """Muon / NorMuon over a list of matrix-shaped parameters.

    ``heads`` and ``split_rows`` map ``id(param)`` to a head count or to a list
    of row-block heights (a fused q/k/v weight); parameters are grouped by
    (flattened shape, dtype, heads, split); each group's fp32
    master weights, momentum and NorMuon variance are held here, and one
    ``step_groups`` call runs the step of every group on the current stream.
    After the step the bf16 model parameters hold RNE(master).
    """

    def __init__(self, params, lr=0.05, momentum=0.95, nesterov=True, weight_decay=0.0, extra_scale=1.0,
                 normuon=False, beta2=0.95, norm_eps=1e-8, ns_steps=5, coeffs=QUINTIC, ns_eps=1e-7,
                 compute_dtype="bf16", mom_dtype=None, max_batch=0, heads=None, split_rows=None):
        torch = _torch()
        self.params = [p for p in params]
        heads = heads or {}
        split_rows = split_rows or {}
        self.hp = hparams(lr, momentum, nesterov, weight_decay, extra_scale, normuon, beta2, norm_eps,
                          ns=ns_config(ns_steps, coeffs, ns_eps, compute_dtype, max_batch))
        self.groups = OrderedDict()
        for p in self.params:
            if p.dim() < 2:
                raise MuonError(_lib.MUON_ERR_INVALID_ARG, "MuonNS5 takes matrix-shaped (2-D+) parameters")
            sp = split_rows.get(id(p))
            key = (tuple(p.shape), p.dtype, int(heads.get(id(p), 1)), tuple(int(h) for h in sp) if sp else None)
            self.groups.setdefault(key, []).append(p)
        self.state = {}
        # The library takes contiguous row-major tensors.  A contiguous fp32
        # parameter is its own master weight; any other parameter gets a
        # contiguous fp32 master.  A bf16 parameter receives RNE(master) from
        # the update kernel: in place when contiguous, else into a contiguous
        # bf16 buffer that step() copies into the parameter (a channels_last
        # conv weight, say).  A non-contiguous fp32 parameter gets its
        # master copied back the same way.
        self._copy_back = []
        for key, ps in self.groups.items():
            for p in ps:
                md = mom_dtype or p.dtype
                own = p.dtype == torch.float32 and p.is_contiguous()
                master = p.data if own else p.detach().to(torch.float32).contiguous().clone()
                model = None
                if p.dtype == torch.bfloat16:
                    model = p.data if p.is_contiguous() else torch.empty(p.shape, dtype=torch.bfloat16,
                                                                          device=p.device)
                self.state[id(p)] = {
                    "master": master,
                    "mom": torch.zeros(p.shape, dtype=md, device=p.device),
                    "var": torch.zeros(p.shape[0], dtype=torch.float32, device=p.device) if normuon else None,
                    "model": model,
                }
                if not own and not (model is not None and model.data_ptr() == p.data_ptr()):
                    self._copy_back.append(p)
        # Reject bad geometry (heads, row splits) and hyperparameters here, not
        # at the first step: the workspace query checks every group's shape
        # and the Newton-Schulz configuration without touching device memory.
        _check_scalars(self.hp)
        made = []
        for (shape, dt, h, sp), ps in self.groups.items():
            masters = [self.state[id(p)]["master"] for p in ps]
            made.append(_make_group(masters, masters, [self.state[id(p)]["mom"] for p in ps], None, None, h,
                                    list(sp) if sp else None))
        self.workspace_bytes = step_groups_workspace_bytes([g for g, _ in made], self.hp) if made else 0

    def state_dict(self):
        """The optimizer state, per parameter in the order given: fp32 master weight,
        momentum and NorMuon variance (the tensors themselves), tagged with the
        library's state layout version (one fp32 variance per output channel)."""
        return {"state_layout_version": state_layout_version(),
                "state": [{k: self.state[id(p)][k] for k in ("master", "mom", "var")} for p in self.params]}

    def load_state_dict(self, sd):
        """Copy a state_dict() into this optimizer's state (same parameters, same
        shapes and dtypes).  Refuses another state layout version, checked before
        anything is copied."""
        torch = _torch()
        if sd.get("state_layout_version") != state_layout_version():
            raise MuonError(_lib.MUON_ERR_INVALID_ARG,
                            f"state layout version {sd.get('state_layout_version')} != {state_layout_version()}")
        entries = sd.get("state", [])
        if len(entries) != len(self.params):
            raise MuonError(_lib.MUON_ERR_INVALID_ARG, f"{len(entries)} parameter states for {len(self.params)} parameters")
        for p, e in zip(self.params, entries):
            st = self.state[id(p)]
            for k in ("master", "mom", "var"):
                a, b = st[k], e.get(k)
                if (a is None) != (b is None) or (a is not None and (a.shape != b.shape or a.dtype != b.dtype)):
                    raise MuonError(_lib.MUON_ERR_INVALID_ARG, f"state '{k}' does not match the parameter's")
        with torch.no_grad():
            for p, e in zip(self.params, entries):
                st = self.state[id(p)]
                for k in ("master", "mom", "var"):
                    if st[k] is not None:
                        st[k].copy_(e[k])

    def step(self):
        torch = _torch()
        todo = []
        for (shape, dt, h, sp), ps in self.groups.items():
            live = [p for p in ps if p.grad is not None]
            if not live:
                continue
            st = [self.state[id(p)] for p in live]
            todo.append({
                "w_master": [s["master"] for s in st],
                "grads": [p.grad.contiguous() for p in live],
                "moms": [s["mom"] for s in st],
                "variances": [s["var"] for s in st] if self.hp.normuon else None,
                "w_model": [s["model"] for s in st] if dt == torch.bfloat16 else None,
                "heads": h,
                "split_rows": list(sp) if sp else None,
            })
        step_groups(todo, hp=self.hp)
        # Parameters whose storage the library does not write: copy the new
        # values in (a layout change only, on the same stream).
        with torch.no_grad():
            for p in self._copy_back:
                if p.grad is None:
                    continue
                st = self.state[id(p)]
                p.data.copy_(st["model"] if p.dtype == torch.bfloat16 else st["master"])


# ---- launch timing ---------------------------------------------------------------
def profile_enable(on=True):
    _lib.check(lib().muon_profile_enable(int(bool(on))))


def profile_classes(names=None):
    """Time only these kernel classes (names from KERNEL_CLASSES; None: all)."""
    names = KERNEL_CLASSES if names is None else names
    mask = 0
    for n in names:
        mask |= 1 << KERNEL_CLASSES.index(n)
    return _lib.check(lib().muon_profile_classes(mask))


def profile_reset():
    _lib.check(lib().muon_profile_reset())


def profile_query(kernel_class):
    if isinstance(kernel_class, str):
        kernel_class = KERNEL_CLASSES.index(kernel_class)
    n, ms, fl, by = ctypes.c_int64(0), ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
    _lib.check(lib().muon_profile_query(int(kernel_class), ctypes.byref(n), ctypes.byref(ms), ctypes.byref(fl),
                                        ctypes.byref(by)))
    return {"launches": n.value, "ms": ms.value, "flop": fl.value, "bytes": by.value}
