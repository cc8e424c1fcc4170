"""ctypes view of libmuon_mi355x.so (the C ABI declared in include/muon_mi355x.h).

Argument marshalling only: every step of the optimizer runs in the library's
HIP kernels.  Loading fails loudly when the library has not been built; there
is no fallback of any kind.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmuon_mi355x.so")

MUON_OK = 0
MUON_ERR_INVALID_ARG = -1
MUON_ERR_UNSUPPORTED = -2
MUON_ERR_WORKSPACE = -3
MUON_ERR_HIP = -4

MUON_F32 = 0
MUON_BF16 = 1

KERNEL_CLASSES = ("prep", "norm", "gram", "poly", "update", "rowstat", "rho", "apply")
MUON_K_UPDATE = 4

# Every function the header declares, with its ctypes signature.
c_i32, c_i64, c_f32, c_f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
c_vp, c_sz = ctypes.c_void_p, ctypes.c_size_t


NS_MAX_STEPS = 64


class NSConfig(ctypes.Structure):
    _fields_ = [("steps", c_i32), ("a", c_f32), ("b", c_f32), ("c", c_f32), ("eps", c_f32),
                ("compute_dtype", c_i32), ("schedule", c_i32), ("max_batch", c_i64),
                ("coeffs", (c_f32 * 3) * NS_MAX_STEPS)]


class NSProblem(ctypes.Structure):
    _fields_ = [("x", c_vp), ("x_dtype", c_i32), ("x_batch_stride", c_i64), ("x_row_stride", c_i64),
                ("y", c_vp), ("y_dtype", c_i32), ("y_batch_stride", c_i64), ("y_row_stride", c_i64),
                ("n", c_i64), ("rows", c_i64), ("cols", c_i64)]


class Group(ctypes.Structure):
    _fields_ = [("n", c_i64), ("rows", c_i64), ("cols", c_i64), ("heads", c_i64),
                ("grad_dtype", c_i32), ("mom_dtype", c_i32), ("model_dtype", c_i32), ("reserved", c_i32),
                ("w_master", ctypes.POINTER(c_vp)), ("w_model", ctypes.POINTER(c_vp)),
                ("grad", ctypes.POINTER(c_vp)), ("mom", ctypes.POINTER(c_vp)), ("var", ctypes.POINTER(c_vp)),
                ("nsplit", c_i64), ("split_rows", ctypes.POINTER(c_i64))]


class HParams(ctypes.Structure):
    _fields_ = [("lr", c_f32), ("momentum", c_f32), ("nesterov", c_i32), ("weight_decay", c_f32),
                ("extra_scale", c_f32), ("normuon", c_i32), ("beta2", c_f32), ("norm_eps", c_f32),
                ("fan_out", c_i64), ("fan_in", c_i64), ("ns", NSConfig)]


SIGNATURES = {
    "muon_ns_default_config": (None, [ctypes.POINTER(NSConfig)]),
    "muon_default_hparams": (None, [ctypes.POINTER(HParams)]),
    "muon_abi_version": (c_i32, []),
    "muon_state_layout_version": (c_i32, []),
    "muon_status_string": (ctypes.c_char_p, [c_i32]),
    "muon_last_error": (ctypes.c_char_p, []),
    "muon_ns_workspace_bytes": (c_i32, [c_i64, c_i64, c_i64, ctypes.POINTER(NSConfig), ctypes.POINTER(c_sz)]),
    "muon_ns_batched": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_vp, c_i32, c_i64, c_i64, c_i64, c_i64, c_i64,
                                ctypes.POINTER(NSConfig), c_vp, c_sz, c_vp]),
    "muon_ns_batched_noalloc": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_vp, c_i32, c_i64, c_i64, c_i64, c_i64, c_i64,
                                        ctypes.POINTER(NSConfig), c_vp]),
    "muon_ns_groups_workspace_bytes": (c_i32, [ctypes.POINTER(NSProblem), c_i64, ctypes.POINTER(NSConfig),
                                               ctypes.POINTER(c_sz)]),
    "muon_ns_groups": (c_i32, [ctypes.POINTER(NSProblem), c_i64, ctypes.POINTER(NSConfig), c_vp, c_sz, c_vp]),
    "normuon_workspace_bytes": (c_i32, [c_i64, c_i64, c_i64, ctypes.POINTER(c_sz)]),
    "normuon_normalize": (c_i32, [c_vp, c_i32, c_i64, c_i64, c_i64, c_i64, c_i64, c_vp, c_i64, c_f32, c_f32,
                                  c_vp, c_sz, c_vp]),
    "muon_step_workspace_bytes": (c_i32, [ctypes.POINTER(Group), ctypes.POINTER(HParams), ctypes.POINTER(c_sz)]),
    "muon_step_group": (c_i32, [ctypes.POINTER(Group), ctypes.POINTER(HParams), c_vp, c_sz, c_vp]),
    "muon_step_groups_workspace_bytes": (c_i32, [ctypes.POINTER(Group), c_i64, ctypes.POINTER(HParams),
                                                 ctypes.POINTER(c_sz)]),
    "muon_step_groups": (c_i32, [ctypes.POINTER(Group), c_i64, ctypes.POINTER(HParams), c_vp, c_sz, c_vp]),
    "muon_profile_enable": (c_i32, [c_i32]),
    "muon_profile_classes": (c_i32, [ctypes.c_uint32]),
    "muon_profile_reset": (c_i32, []),
    "muon_profile_query": (c_i32, [c_i32, ctypes.POINTER(c_i64), ctypes.POINTER(c_f64), ctypes.POINTER(c_f64),
                                   ctypes.POINTER(c_f64)]),
    "muon_kernel_class_name": (ctypes.c_char_p, [c_i32]),
}

_LIB = None


class MuonError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{status_name(status)} ({status}): {detail}")


def status_name(status):
    return {0: "MUON_OK", -1: "MUON_ERR_INVALID_ARG", -2: "MUON_ERR_UNSUPPORTED",
            -3: "MUON_ERR_WORKSPACE", -4: "MUON_ERR_HIP"}.get(status, "MUON_ERR_?")


def _hip_runtimes_mapped():
    try:
        maps = open("/proc/self/maps").read()
    except OSError:
        return []
    return sorted({line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line})


def lib():
    """The loaded library.  Raises if it has not been built.

    PyTorch ships its own HIP runtime.  The library is loaded after torch so
    that its libamdhip64.so.7 dependency resolves (by soname) to the runtime
    torch already holds: one process, one HIP runtime, so device pointers and
    streams from torch are valid in the library.  Two runtimes in one process
    are refused.
    """
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m newton_schulz_ns5_amd.build` "
                "(there is no fallback implementation)")
        try:
            import torch  # noqa: F401  (binds the HIP runtime first)
        except ImportError:
            pass
        h = ctypes.CDLL(LIB_PATH)
        runtimes = _hip_runtimes_mapped()
        if len(runtimes) > 1:
            raise RuntimeError(f"two HIP runtimes are loaded in this process: {runtimes}")
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _LIB = h
    return _LIB


def check(status):
    if status != MUON_OK:
        detail = lib().muon_last_error()
        raise MuonError(status, detail.decode() if detail else "")
    return status
