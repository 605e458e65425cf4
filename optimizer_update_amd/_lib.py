"""ctypes binding of liboptimizer_update.so (argument marshalling only).

Every function here has the name of the C entry point it calls and does
nothing but check and convert arguments: all arithmetic runs in the HIP
kernels.  If the library has not been built, loading it raises; there is no
fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "liboptimizer_update.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "optimizer_update.h")

OU_F32, OU_F16, OU_BF16 = 0, 1, 2
OU_ADAM, OU_ADEMAMIX, OU_MOMENTUM, OU_RMSPROP, OU_ADAGRAD, OU_LION = 0, 1, 2, 3, 4, 5
OU_DECAY_AFTER = 0x100
STATUS = {0: "OU_OK", -1: "OU_EINVAL", -2: "OU_EUNSUPPORTED", -3: "OU_EALIGN",
          -4: "OU_EOVERLAP", -5: "OU_ENOMEM", -6: "OU_EHIP", -7: "OU_ECAPTURE"}


class OptimizerUpdateError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class ou_hparams(ctypes.Structure):
    _fields_ = [("beta1", ctypes.c_float), ("beta2", ctypes.c_float), ("beta3", ctypes.c_float),
                ("alpha", ctypes.c_float), ("eps", ctypes.c_float),
                ("weight_decay", ctypes.c_float), ("lr", ctypes.c_float),
                ("skip_zeros", ctypes.c_int32), ("step", ctypes.c_int64)]


class ou_segment(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("state1", ctypes.c_void_p), ("state2", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ou_segment8(ctypes.Structure):
    _fields_ = [("param", ctypes.c_void_p), ("grad", ctypes.c_void_p),
                ("state1", ctypes.c_void_p), ("state2", ctypes.c_void_p),
                ("absmax1", ctypes.c_void_p), ("absmax2", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


OU_8BIT_BLOCK = 256


def header_functions(path: str = HEADER) -> list[str]:
    """Names of the functions the public header declares."""
    with open(path) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)


_lib = None


def load(path: str = LIBRARY) -> ctypes.CDLL:
    """Load the HIP library (raises if it is missing: no fallback exists)."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() "
                          "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    i32, i64, f32, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    lib.optimizer_update_32bit.argtypes = [i32, i32, vp, vp, vp, vp, i64, f32, f32, f32, f32,
                                           f32, f32, i64, f32, i32, vp]
    lib.optimizer_update_32bit.restype = i32
    lib.ou_clip_workspace_bytes.argtypes = [i64]
    lib.ou_clip_workspace_bytes.restype = i64
    lib.optimizer_update_32bit_clip.argtypes = [i32, i32, vp, vp, vp, vp, i64, f32, f32, f32, f32,
                                                f32, f32, i64, f32, i32, f32, vp, i64, vp]
    lib.optimizer_update_32bit_clip.restype = i32
    lib.optimizer_update_32bit_clip_noalloc.argtypes = [i32, i32, vp, vp, vp, vp, i64, f32, f32, f32,
                                                        f32, f32, f32, i64, f32, i32, f32, vp]
    lib.optimizer_update_32bit_clip_noalloc.restype = i32
    lib.ou_clip_noalloc_max_elements.argtypes = []
    lib.ou_clip_noalloc_max_elements.restype = i64
    lib.optimizer_update_32bit_multi.argtypes = [i32, ctypes.POINTER(ou_segment), ctypes.c_int32,
                                                 ctypes.POINTER(ou_hparams), vp]
    lib.optimizer_update_32bit_multi.restype = i32
    lib.ou_plan_create.argtypes = [i32, ctypes.POINTER(ou_segment), ctypes.c_int32,
                                   ctypes.POINTER(vp)]
    lib.ou_plan_create.restype = i32
    lib.ou_plan_step.argtypes = [vp, ctypes.POINTER(ou_hparams), vp]
    lib.ou_plan_step.restype = i32
    lib.ou_plan_step_clip.argtypes = [vp, ctypes.POINTER(ou_hparams), f32, vp]
    lib.ou_plan_step_clip.restype = i32
    lib.ou_plan_clip_factors.argtypes = [vp, ctypes.POINTER(f32), ctypes.c_int32]
    lib.ou_plan_clip_factors.restype = i32
    lib.ou_plan_graph_step.argtypes = [vp, ctypes.POINTER(ou_hparams), vp]
    lib.ou_plan_graph_step.restype = i32
    lib.ou_plan_graph_step_clip.argtypes = [vp, ctypes.POINTER(ou_hparams), f32, vp]
    lib.ou_plan_graph_step_clip.restype = i32
    lib.ou_plan_describe.argtypes = [vp, ctypes.POINTER(ctypes.c_int32),
                                     ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.ou_plan_describe.restype = i32
    lib.ou_plan_destroy.argtypes = [vp]
    lib.ou_plan_destroy.restype = None
    lib.ou_8bit_qmap.argtypes = [i32, ctypes.POINTER(f32), ctypes.c_int32]
    lib.ou_8bit_qmap.restype = i32
    lib.optimizer_update_8bit_blockwise.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, i64, f32, f32,
                                                    f32, f32, f32, f32, i64, f32, i32, vp]
    lib.optimizer_update_8bit_blockwise.restype = i32
    lib.ou_plan8_create.argtypes = [i32, ctypes.POINTER(ou_segment8), ctypes.c_int32,
                                    ctypes.POINTER(vp)]
    lib.ou_plan8_create.restype = i32
    lib.ou_plan8_step.argtypes = [vp, ctypes.POINTER(ou_hparams), vp]
    lib.ou_plan8_step.restype = i32
    lib.ou_plan8_graph_step.argtypes = [vp, ctypes.POINTER(ou_hparams), vp]
    lib.ou_plan8_graph_step.restype = i32
    lib.ou_plan8_destroy.argtypes = [vp]
    lib.ou_plan8_destroy.restype = None
    lib.ou_graph_create.argtypes = [ctypes.POINTER(vp), ctypes.c_int32, ctypes.POINTER(vp), ctypes.c_int32,
                                    ctypes.POINTER(vp)]
    lib.ou_graph_create.restype = i32
    lib.ou_graph_step.argtypes = [vp, ctypes.POINTER(ou_hparams), vp]
    lib.ou_graph_step.restype = i32
    lib.ou_graph_destroy.argtypes = [vp]
    lib.ou_graph_destroy.restype = None
    lib.ou_status_string.argtypes = [i32]
    lib.ou_status_string.restype = ctypes.c_char_p
    lib.ou_last_error.argtypes = []
    lib.ou_last_error.restype = ctypes.c_char_p
    # test hooks (not in the public header)
    lib.ou__select_single.argtypes = [i32, i32, i32, i32, i32, i64, i32, ctypes.POINTER(i64)]
    lib.ou__select_single.restype = i32
    lib.ou__select_multi.argtypes = [i32, i32, i32, i32, i32, i64, ctypes.POINTER(i64)]
    lib.ou__select_multi.restype = i32
    lib.ou__force_single.argtypes = [i32, i32, i32, i64, i32, i32]
    lib.ou__force_single.restype = None
    lib.ou__force_multi.argtypes = [i32, i32, i32, i32, i32]
    lib.ou__force_multi.restype = None
    lib.ou__step_scalars.argtypes = [ctypes.POINTER(ou_hparams), ctypes.POINTER(f32)]
    lib.ou__step_scalars.restype = i32
    lib.ou__force_8bit.argtypes = [i32, i32, i32, i32]
    lib.ou__force_8bit.restype = None
    lib.ou__narrow.argtypes = [i32, vp, vp, i64, vp]
    lib.ou__narrow.restype = i32
    lib.ou__sqrt.argtypes = [vp, vp, i64, vp]
    lib.ou__sqrt.restype = i32
    lib.ou__recip8.argtypes = [vp, vp, i64, vp]
    lib.ou__recip8.restype = i32
    lib.ou__quant8.argtypes = [vp, vp, vp, vp, i64, vp]
    lib.ou__quant8.restype = i32
    lib.ou__stream_probe.argtypes = [i32, vp, vp, vp, vp, i64, vp]
    lib.ou__stream_probe.restype = i32
    lib.ou__valu_probe.argtypes = [i32, i64, ctypes.c_int32, vp, vp]
    lib.ou__valu_probe.restype = i32
    lib.ou__force_xcd.argtypes = [i32]
    lib.ou__force_xcd.restype = None
    lib.ou__validate_only.argtypes = [i32]
    lib.ou__validate_only.restype = None
    if path == LIBRARY:
        _install_fast(lib)
        _lib = lib
    return lib


# Per-step entry points that the CPython module _fast also exposes.
FAST_ENTRY_POINTS = ("optimizer_update_32bit", "optimizer_update_8bit_blockwise", "ou_plan_step",
                     "ou_plan8_step")


def _install_fast(lib: ctypes.CDLL) -> None:
    """Route the per-step entry points of the in-tree library through _fast
    when it is built: the same C functions of the same loaded library, the
    same positional arguments, converted in C instead of by ctypes.  A
    struct argument is the ou_hparams instance or its int address (not
    byref(), pointer() or c_void_p: those raise TypeError).  Like ctypes,
    the calls release the GIL while the library runs."""
    try:
        from . import _fast
    except ImportError:
        return
    for name in FAST_ENTRY_POINTS:
        setattr(lib, name, getattr(_fast, name))


def check(status: int, lib: ctypes.CDLL | None = None) -> None:
    if status != 0:
        lib = lib or load()
        raise OptimizerUpdateError(status, lib.ou_last_error().decode(errors="replace"))
