"""CPU oracle for the 32-bit two-state optimizer update.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``optimizer_update_amd``) never imports it, and the two share no code.

This module is a ctypes wrapper around ``oracle.c`` (a plain per-element C
loop; see that file for the formulas and the passages they follow).  Arrays
are numpy: fp32 storage as ``float32``; fp16 and bf16 storage as ``uint16``
bit patterns; states as ``float32``.  Every call updates its arguments in
place, exactly like the product entry points.

``oracle_update_f32`` is the parity oracle.  ``oracle_update_f64`` exists to
check the formulas against closed forms.  Every exported function is pinned
to something other than itself by the pins in ``tests/oracle_pins.py``, run
by ``tests/test_oracle.py``.  Where the page is silent, the reading taken is
stated in ``oracle.c`` at the function it governs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

ADAM, ADEMAMIX = 0, 1
MOMENTUM, RMSPROP, ADAGRAD, LION = 2, 3, 4, 5
F32, F16, BF16 = 0, 1, 2
KINDS = {"adam": ADAM, "ademamix": ADEMAMIX, "momentum": MOMENTUM, "rmsprop": RMSPROP,
         "adagrad": ADAGRAD, "lion": LION}
ONE_STATE = (MOMENTUM, RMSPROP, ADAGRAD, LION)
# OR'ed into a kind: decoupled decay applied to the updated parameter,
# (p - lr*u)*d, instead of the default p*d - lr*u (ADAM, ADEMAMIX, LION).
DECAY_AFTER = 0x100
# elements per block of the 8-bit block-wise states
QBLOCK = 256
DTYPES = {"fp32": F32, "fp16": F16, "bf16": BF16}

# -O2 without contraction or fast-math: each C operation is one correctly
# rounded IEEE operation, and denormals are kept (no crtfastmath, no FTZ/DAZ).
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fno-unsafe-math-optimizations", "-fopenmp", "-fPIC", "-shared"]


def build(out_path: str = LIBRARY, plant: int = 0) -> str:
    """Compile ``oracle.c`` with gcc into ``out_path`` (atomically).

    ``plant`` != 0 builds a copy with one planted mistake; the test suite uses
    it to show that the pins catch such mistakes."""
    cmd = ["gcc", *CFLAGS]
    if plant:
        cmd.append(f"-DORACLE_PLANT={int(plant)}")
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=os.path.dirname(out_path) or ".")
    os.close(fd)
    try:
        subprocess.run(cmd + ["-o", tmp, SOURCE, "-lm"], check=True)
        os.replace(tmp, out_path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return out_path


class _Scalars32(ctypes.Structure):
    _fields_ = [(n, ctypes.c_float) for n in ("bc1", "bc2", "decay", "omb1", "omb2", "omb3")]


@dataclass(frozen=True)
class HParams:
    """Hyperparameters of one step.  beta3 and alpha are used by AdEMAMix only."""
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    beta3: float = 0.9999
    alpha: float = 5.0
    eps: float = 1e-8
    weight_decay: float = 0.0
    skip_zeros: bool = False


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags.c_contiguous
    return ctypes.c_void_p(a.ctypes.data)


class Oracle:
    """A loaded oracle library (the normal one, or a planted-mistake copy)."""

    def __init__(self, path: str):
        self.path = path
        lib = ctypes.CDLL(path)
        self._lib = lib
        i64, f32, f64, vp, ci = (ctypes.c_int64, ctypes.c_float, ctypes.c_double,
                                 ctypes.c_void_p, ctypes.c_int)
        lib.oracle_update_f32.argtypes = [ci, ci, vp, vp, vp, vp, i64,
                                          f32, f32, f32, f32, f32, f32, i64, f32, ci, ci]
        lib.oracle_update_f32.restype = ci
        lib.oracle_update_f64.argtypes = [ci, vp, vp, vp, vp, i64,
                                          f64, f64, f64, f64, f64, f64, i64, f64, ci]
        lib.oracle_update_f64.restype = ci
        lib.oracle_update_f32_clip.argtypes = [ci, ci, vp, vp, vp, vp, i64, f32, f32, f32, f32,
                                               f32, f32, i64, f32, ci, f32,
                                               ctypes.POINTER(ctypes.c_float)]
        lib.oracle_update_f32_clip.restype = ci
        lib.oracle_update_f64_clip.argtypes = [ci, vp, vp, vp, vp, i64, f64, f64, f64, f64, f64,
                                               f64, i64, f64, ci, f64,
                                               ctypes.POINTER(ctypes.c_double)]
        lib.oracle_update_f64_clip.restype = ci
        lib.oracle_update1_f32.argtypes = [ci, ci, vp, vp, vp, i64, f32, f32, f32, f32, i64, f32,
                                           ci, ci]
        lib.oracle_update1_f32.restype = ci
        lib.oracle_update1_f64.argtypes = [ci, vp, vp, vp, i64, f64, f64, f64, f64, i64, f64, ci]
        lib.oracle_update1_f64.restype = ci
        lib.oracle_qmap.argtypes = [ci, vp]
        lib.oracle_qmap.restype = ci
        lib.oracle_qcode.argtypes = [ci, f32, f32]
        lib.oracle_qcode.restype = ci
        lib.oracle_qvalue.argtypes = [ci, ci]
        lib.oracle_qvalue.restype = f32
        lib.oracle_update_8bit_f32.argtypes = [ci, ci, vp, vp, vp, vp, vp, vp, i64, f32, f32, f32,
                                               f32, f32, f32, i64, f32, ci, ci]
        lib.oracle_update_8bit_f32.restype = ci
        lib.oracle_step_scalars.argtypes = [f32, f32, f32, f32, f32, i64,
                                            ctypes.POINTER(_Scalars32)]
        lib.oracle_step_scalars.restype = None
        for name in ("oracle_f32_to_bf16_array", "oracle_f32_to_f16_array",
                     "oracle_f16_to_f32_array", "oracle_bf16_to_f32_array"):
            getattr(lib, name).argtypes = [vp, vp, i64]
            getattr(lib, name).restype = None
        lib.oracle_max_threads.restype = ci
        lib.oracle_planted.restype = ci
        self.planted = lib.oracle_planted()

    # ------------------------------------------------------------ storage
    def f32_to_storage(self, x: np.ndarray, dtype: int) -> np.ndarray:
        """fp32 -> storage dtype, round to nearest even (fp32 is a copy)."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        if dtype == F32:
            return x.copy()
        y = np.empty(x.shape, np.uint16)
        fn = self._lib.oracle_f32_to_f16_array if dtype == F16 else self._lib.oracle_f32_to_bf16_array
        fn(_ptr(x), _ptr(y), x.size)
        return y

    def storage_to_f32(self, x: np.ndarray, dtype: int) -> np.ndarray:
        """storage dtype -> fp32 (exact)."""
        if dtype == F32:
            return np.ascontiguousarray(x, dtype=np.float32).copy()
        x = np.ascontiguousarray(x, dtype=np.uint16)
        y = np.empty(x.shape, np.float32)
        fn = self._lib.oracle_f16_to_f32_array if dtype == F16 else self._lib.oracle_bf16_to_f32_array
        fn(_ptr(x), _ptr(y), x.size)
        return y

    # ------------------------------------------------------------ update
    def step_scalars(self, hp: HParams, step: int) -> dict:
        out = _Scalars32()
        self._lib.oracle_step_scalars(hp.beta1, hp.beta2, hp.beta3, hp.lr,
                                      hp.weight_decay, step, ctypes.byref(out))
        return {n: getattr(out, n) for n, _ in _Scalars32._fields_}

    def update_f32(self, kind: int, dtype: int, param: np.ndarray, grad: np.ndarray,
                   state1: np.ndarray, state2: np.ndarray, hp: HParams, step: int,
                   nthreads: int = 1) -> None:
        """One step of the fp32 update, in place (see ``oracle_update_f32``)."""
        n = param.size
        sdt = np.float32 if dtype == F32 else np.uint16
        assert param.dtype == sdt and grad.dtype == sdt and grad.size == n
        assert state1.dtype == np.float32 and state2.dtype == np.float32
        assert state1.size == (2 * n if kind & 0xff == ADEMAMIX else n) and state2.size == n
        rc = self._lib.oracle_update_f32(
            kind, dtype, _ptr(param), _ptr(grad), _ptr(state1), _ptr(state2), n,
            hp.beta1, hp.beta2, hp.beta3, hp.alpha, hp.eps, hp.weight_decay, step,
            hp.lr, int(bool(hp.skip_zeros)), nthreads)
        if rc != 0:
            raise ValueError(f"oracle_update_f32 rejected kind={kind} dtype={dtype}")

    def update_f64(self, kind: int, param: np.ndarray, grad: np.ndarray, state1: np.ndarray,
                   state2: np.ndarray, hp: HParams, step: int) -> None:
        """One step of the binary64 update, in place (see ``oracle_update_f64``)."""
        n = param.size
        for a in (param, grad, state1, state2):
            assert a.dtype == np.float64 and a.flags.c_contiguous
        assert state1.size == (2 * n if kind & 0xff == ADEMAMIX else n) and state2.size == n
        rc = self._lib.oracle_update_f64(
            kind, _ptr(param), _ptr(grad), _ptr(state1), _ptr(state2), n,
            hp.beta1, hp.beta2, hp.beta3, hp.alpha, hp.eps, hp.weight_decay, step,
            hp.lr, int(bool(hp.skip_zeros)))
        if rc != 0:
            raise ValueError(f"oracle_update_f64 rejected kind={kind}")

    def update1_f32(self, kind: int, dtype: int, param: np.ndarray, grad: np.ndarray,
                    state1: np.ndarray, hp: HParams, step: int, nthreads: int = 1) -> None:
        """One step of a one-state kind, in place (see ``oracle_update1_f32``)."""
        n = param.size
        sdt = np.float32 if dtype == F32 else np.uint16
        assert param.dtype == sdt and grad.dtype == sdt and grad.size == n
        assert state1.dtype == np.float32 and state1.size == n
        rc = self._lib.oracle_update1_f32(kind, dtype, _ptr(param), _ptr(grad), _ptr(state1), n,
                                          hp.beta1, hp.beta2, hp.eps, hp.weight_decay, step, hp.lr,
                                          int(bool(hp.skip_zeros)), nthreads)
        if rc != 0:
            raise ValueError(f"oracle_update1_f32 rejected kind={kind} dtype={dtype}")

    def update1_f64(self, kind: int, param: np.ndarray, grad: np.ndarray, state1: np.ndarray,
                    hp: HParams, step: int) -> None:
        """One binary64 step of a one-state kind, in place."""
        for a in (param, grad, state1):
            assert a.dtype == np.float64 and a.flags.c_contiguous and a.size == param.size
        rc = self._lib.oracle_update1_f64(kind, _ptr(param), _ptr(grad), _ptr(state1), param.size,
                                          hp.beta1, hp.beta2, hp.eps, hp.weight_decay, step, hp.lr,
                                          int(bool(hp.skip_zeros)))
        if rc != 0:
            raise ValueError(f"oracle_update1_f64 rejected kind={kind}")

    def qmap(self, signed: bool) -> np.ndarray:
        """Magnitudes of the 8-bit dynamic type: 128 (signed) or 256 (unsigned)."""
        out = np.zeros(256, np.float32)
        count = self._lib.oracle_qmap(int(bool(signed)), _ptr(out))
        return out[:count].copy()

    def qcode(self, signed: bool, value: float, absmax: float = 1.0) -> int:
        """Code of a state value in a block with the given absmax
        (``oracle_qcode``): the magnitude nearest to |value| / absmax."""
        return int(self._lib.oracle_qcode(int(bool(signed)), float(value), float(absmax)))

    def qvalue(self, signed: bool, code: int) -> float:
        """Normalised value of a code (``oracle_qvalue``)."""
        return float(self._lib.oracle_qvalue(int(bool(signed)), int(code)))

    def update_8bit_f32(self, kind: int, dtype: int, param: np.ndarray, grad: np.ndarray,
                        state1: np.ndarray, state2: np.ndarray, absmax1: np.ndarray,
                        absmax2: np.ndarray, hp: HParams, step: int, nthreads: int = 1) -> None:
        """One step with 8-bit block-wise states, in place (``oracle_update_8bit_f32``)."""
        n = param.size
        k = 2 if kind & 0xff == ADEMAMIX else 1
        nb = -(-n // QBLOCK)
        sdt = np.float32 if dtype == F32 else np.uint16
        assert param.dtype == sdt and grad.dtype == sdt and grad.size == n
        assert state1.dtype == np.uint8 and state1.size == k * n
        assert state2.dtype == np.uint8 and state2.size == n
        assert absmax1.dtype == np.float32 and absmax1.size == k * nb
        assert absmax2.dtype == np.float32 and absmax2.size == nb
        rc = self._lib.oracle_update_8bit_f32(
            kind, dtype, _ptr(param), _ptr(grad), _ptr(state1), _ptr(state2), _ptr(absmax1),
            _ptr(absmax2), n, hp.beta1, hp.beta2, hp.beta3, hp.alpha, hp.eps, hp.weight_decay,
            step, hp.lr, int(bool(hp.skip_zeros)), nthreads)
        if rc != 0:
            raise ValueError(f"oracle_update_8bit_f32 rejected kind={kind} dtype={dtype}")

    def update_f32_clip(self, kind: int, dtype: int, param: np.ndarray, grad: np.ndarray,
                        state1: np.ndarray, state2: np.ndarray, hp: HParams, step: int,
                        max_unorm: float) -> float:
        """One clipped step, in place (see ``oracle_update_f32_clip``);
        returns the clip factor s."""
        n = param.size
        sdt = np.float32 if dtype == F32 else np.uint16
        assert param.dtype == sdt and grad.dtype == sdt and grad.size == n
        assert state1.size == (2 * n if kind & 0xff == ADEMAMIX else n) and state2.size == n
        out = ctypes.c_float()
        rc = self._lib.oracle_update_f32_clip(
            kind, dtype, _ptr(param), _ptr(grad), _ptr(state1), _ptr(state2), n,
            hp.beta1, hp.beta2, hp.beta3, hp.alpha, hp.eps, hp.weight_decay, step, hp.lr,
            int(bool(hp.skip_zeros)), max_unorm, ctypes.byref(out))
        if rc != 0:
            raise ValueError(f"oracle_update_f32_clip failed ({rc})")
        return out.value

    def update_f64_clip(self, kind: int, param: np.ndarray, grad: np.ndarray, state1: np.ndarray,
                        state2: np.ndarray, hp: HParams, step: int, max_unorm: float) -> float:
        """One clipped binary64 step, in place; returns the clip factor s."""
        n = param.size
        for a in (param, grad, state1, state2):
            assert a.dtype == np.float64 and a.flags.c_contiguous
        out = ctypes.c_double()
        rc = self._lib.oracle_update_f64_clip(
            kind, _ptr(param), _ptr(grad), _ptr(state1), _ptr(state2), n,
            hp.beta1, hp.beta2, hp.beta3, hp.alpha, hp.eps, hp.weight_decay, step, hp.lr,
            int(bool(hp.skip_zeros)), max_unorm, ctypes.byref(out))
        if rc != 0:
            raise ValueError(f"oracle_update_f64_clip failed ({rc})")
        return out.value

    def max_threads(self) -> int:
        return self._lib.oracle_max_threads()


_default: Oracle | None = None


def load() -> Oracle:
    """The oracle library next to this file; compiled first only if absent."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build(LIBRARY)
        _default = Oracle(LIBRARY)
    return _default
