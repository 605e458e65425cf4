"""MI355X (gfx950) 32-bit optimizer update: Adam/AdamW and AdEMAMix (two
fp32 states), and momentum SGD, RMSprop, Adagrad and Lion (one fp32 state).

Thin torch-facing binding of ``liboptimizer_update.so`` (``include/optimizer_update.h``).
Functions carry the names of the C entry points and only marshal arguments
(device pointers, dtype codes, the current stream); every step of the update
runs in the HIP kernels.  There is no CPU fallback: without the built
library, or without a GPU, calls raise.

    optimizer_update_32bit(kind, param, grad, state1, state2, step=..., lr=..., ...)
    optimizer_update_32bit_clip(..., max_unorm=..., workspace=...)   update-norm clipping
    optimizer_update_32bit_clip_noalloc(..., max_unorm=...)   the same, allocating nothing
    optimizer_update_32bit_multi(kind, segments, hp, step)
    Plan(kind, segments)  -> .step(hp, step) / .graph_step(hp, step) / .close()
                             .step_clip / .graph_step_clip(hp, step, max_unorm)
    AdamW32, AdEMAMix32, Momentum32, RMSprop32, Adagrad32, Lion32
                           collection optimizers over a fixed parameter list

Layout: param and grad are contiguous tensors of one storage dtype
(float32, float16 or bfloat16); state1 holds n floats (Adam) or 2n floats
(AdEMAMix: fast EMA, then slow EMA); state2 holds n floats for the
two-state kinds and is None for the one-state kinds.
"""
from __future__ import annotations

import ctypes
import functools
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import OptimizerUpdateError, check, load

__all__ = ["HParams", "optimizer_update_32bit", "optimizer_update_32bit_clip",
           "clip_workspace_bytes", "clip_workspace", "clip_scale",
           "optimizer_update_32bit_clip_noalloc", "clip_noalloc_max_elements",
           "optimizer_update_32bit_multi", "Plan",
           "OptimizerUpdateError", "KINDS", "DTYPES", "load", "state_sizes"]

KINDS = {"adam": _lib.OU_ADAM, "ademamix": _lib.OU_ADEMAMIX, "momentum": _lib.OU_MOMENTUM,
         "rmsprop": _lib.OU_RMSPROP, "adagrad": _lib.OU_ADAGRAD, "lion": _lib.OU_LION}
TWO_STATE = (_lib.OU_ADAM, _lib.OU_ADEMAMIX)
DTYPES = {torch.float32: _lib.OU_F32, torch.float16: _lib.OU_F16, torch.bfloat16: _lib.OU_BF16}


@dataclass(frozen=True)
class HParams:
    """Step hyperparameters; beta3 and alpha are used by AdEMAMix only.
    For the one-state kinds beta1 is the momentum (momentum SGD), the
    smoothing constant (RMSprop) or Lion's interpolation beta, beta2 Lion's
    moment beta; Adagrad uses neither."""
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.999
    beta3: float = 0.9999
    alpha: float = 5.0
    eps: float = 1e-8
    weight_decay: float = 0.0
    skip_zeros: bool = False

    @functools.cached_property
    def _struct(self) -> _lib.ou_hparams:
        return _lib.ou_hparams(self.beta1, self.beta2, self.beta3, self.alpha, self.eps,
                               self.weight_decay, self.lr, int(bool(self.skip_zeros)), 1)

    def c(self, step: int) -> _lib.ou_hparams:
        """The C struct for `step`.  The instance is frozen, so the struct is
        built once and only its step is set; it is passed on at once (the
        library copies what it needs), never kept."""
        s = self._struct
        s.step = int(step)
        return s


def _kind(kind, decay_after: bool = False) -> int:
    """The C kind argument: an ou_kind, OR'ed with OU_DECAY_AFTER when the
    decoupled decay is to apply to the updated parameter, (p - lr*u)*d."""
    k = KINDS[kind] if isinstance(kind, str) else int(kind)
    return k | (_lib.OU_DECAY_AFTER if decay_after else 0)


def state_sizes(kind, n: int) -> tuple[int, int]:
    """Elements of state1 and state2 for a tensor of n elements (state2 is 0
    for the one-state kinds)."""
    k = _kind(kind) & ~_lib.OU_DECAY_AFTER
    return (2 * n if k == _lib.OU_ADEMAMIX else n), (n if k in TWO_STATE else 0)


_GET_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _raw_stream(index: int) -> int:
    """Handle of the current stream of device `index` (torch's own accessor,
    falling back to the public one)."""
    if _GET_RAW_STREAM is not None:
        return _GET_RAW_STREAM(index)
    return torch.cuda.current_stream(index).cuda_stream


_GET_DEVICE = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device


def _stream_arg(stream) -> int:
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _on(index: int, fn, *args):
    """fn(*args) with device `index` current, switching only when it is not."""
    prev = _GET_DEVICE()
    if prev == index:
        return fn(*args)
    torch.cuda.set_device(index)
    try:
        return fn(*args)
    finally:
        torch.cuda.set_device(prev)


def _stream(t: torch.Tensor, stream) -> int:
    if stream is None:
        return _raw_stream(t.get_device())
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class _on_device:
    """Make `device` current for a call, only if it is not already."""

    __slots__ = ("index", "prev")

    def __init__(self, device: torch.device):
        self.index = device.index

    def __enter__(self):
        self.prev = torch.cuda.current_device()
        if self.prev != self.index:
            torch.cuda.set_device(self.index)

    def __exit__(self, *exc):
        if self.prev != self.index:
            torch.cuda.set_device(self.prev)
        return False


def _tensor_args(kind: int, param, grad, state1, state2) -> tuple[int, int, int]:
    """Check one tensor's four operands; returns (n, dtype code, device index).
    The common case costs one attribute read per property and tensor; the
    specific error is worked out only when a check fails."""
    kind &= ~_lib.OU_DECAY_AFTER
    two = kind in TWO_STATE
    if not two and state2 is not None:
        raise ValueError("the one-state kinds take state2=None")
    try:
        dev = param.get_device()
        ok = (dev >= 0 and grad.get_device() == dev and state1.get_device() == dev
              and param.is_contiguous() and grad.is_contiguous() and state1.is_contiguous()
              and (not two or (state2.get_device() == dev and state2.is_contiguous())))
    except AttributeError:
        ok = False
    if not ok:
        _tensor_error(param, grad, state1, state2, two)
    pdt = param.dtype
    dt = DTYPES.get(pdt)
    if dt is None or grad.dtype != pdt:
        raise ValueError("param and grad must share one of float32/float16/bfloat16")
    if state1.dtype != torch.float32 or (two and state2.dtype != torch.float32):
        raise ValueError("states must be float32")
    n = param.numel()
    s1 = state1.numel()
    s2 = state2.numel() if two else 0
    if grad.numel() != n or s1 != (2 * n if kind == _lib.OU_ADEMAMIX else n) or (two and s2 != n):
        raise ValueError(f"sizes: param {n}, grad {grad.numel()}, state1 {s1} "
                         f"(want {2 * n if kind == _lib.OU_ADEMAMIX else n}), state2 {s2} "
                         f"(want {n if two else 0})")
    return n, dt, dev


def _tensor_error(param, grad, state1, state2, two: bool):
    """Raise the ValueError that names the first operand failing a check."""
    named = [("param", param), ("grad", grad), ("state1", state1)]
    if two:
        named.append(("state2", state2))
    for name, t in named:
        if not isinstance(t, torch.Tensor) or t.get_device() < 0:
            raise ValueError(f"{name} must be a tensor on a HIP device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    raise ValueError("all tensors must be on one device")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def optimizer_update_32bit(kind, param: torch.Tensor, grad: torch.Tensor, state1: torch.Tensor,
                           state2: torch.Tensor | None, *, step: int, lr: float, beta1: float = 0.9,
                           beta2: float = 0.999, beta3: float = 0.9999, alpha: float = 5.0,
                           eps: float = 1e-8, weight_decay: float = 0.0, skip_zeros: bool = False,
                           decay_after: bool = False, stream=None) -> None:
    """One update of one tensor, in place, on ``stream`` (default: current).
    decay_after: decay the updated parameter, (p - lr*u)*d (Adam, AdEMAMix,
    Lion)."""
    k = _kind(kind, decay_after)
    n, dt, dev = _tensor_args(k, param, grad, state1, state2)
    lib = load()
    args = (k, dt, param.data_ptr(), grad.data_ptr(), state1.data_ptr(),
            None if state2 is None else state2.data_ptr(), n, beta1, beta2, beta3, alpha, eps,
            weight_decay, int(step), lr, int(bool(skip_zeros)),
            _raw_stream(dev) if stream is None else _stream_arg(stream))
    fn = lib.optimizer_update_32bit
    st = fn(*args) if _GET_DEVICE() == dev else _on(dev, fn, *args)
    if st:
        check(st, lib)


def clip_workspace_bytes(n: int) -> int:
    """Bytes of device workspace ``optimizer_update_32bit_clip`` needs for n elements."""
    return int(load().ou_clip_workspace_bytes(int(n)))


def clip_workspace(n: int, device) -> torch.Tensor:
    """A workspace tensor (uint8) for ``optimizer_update_32bit_clip``."""
    return torch.empty(clip_workspace_bytes(n), dtype=torch.uint8, device=device)


def clip_scale(workspace: torch.Tensor) -> float:
    """The clip factor s of the last clipped step that used ``workspace``
    (synchronises with the device)."""
    return float(workspace[4:8].view(torch.float32).item())


def optimizer_update_32bit_clip(kind, param: torch.Tensor, grad: torch.Tensor,
                                state1: torch.Tensor, state2: torch.Tensor | None, *, step: int,
                                lr: float, max_unorm: float, workspace: torch.Tensor | None = None,
                                beta1: float = 0.9, beta2: float = 0.999, beta3: float = 0.9999,
                                alpha: float = 5.0, eps: float = 1e-8, weight_decay: float = 0.0,
                                skip_zeros: bool = False, decay_after: bool = False,
                                stream=None) -> torch.Tensor | None:
    """One update of one tensor with update-norm clipping (max_unorm > 0),
    in place.  ``workspace``: a uint8 device tensor of
    ``clip_workspace_bytes(n)`` bytes (allocated here if None); returned so
    that ``clip_scale`` can read the clip factor."""
    k = _kind(kind, decay_after)
    n, dt, _ = _tensor_args(k, param, grad, state1, state2)
    if workspace is None and max_unorm > 0 and n > 0:
        workspace = clip_workspace(n, param.device)
    if workspace is not None and (not workspace.is_cuda or workspace.dtype != torch.uint8
                                  or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 tensor on the device")
    lib = load()
    wp = workspace.data_ptr() if workspace is not None else None
    wb = workspace.numel() if workspace is not None else 0
    with _on_device(param.device):
        st = lib.optimizer_update_32bit_clip(k, dt, param.data_ptr(), grad.data_ptr(),
                                             state1.data_ptr(), _ptr(state2), n, beta1, beta2,
                                             beta3, alpha, eps, weight_decay, int(step), lr,
                                             int(bool(skip_zeros)), max_unorm, wp, wb,
                                             _stream(param, stream))
    check(st, lib)
    return workspace


def optimizer_update_32bit_clip_noalloc(kind, param: torch.Tensor, grad: torch.Tensor,
                                        state1: torch.Tensor, state2: torch.Tensor | None, *,
                                        step: int, lr: float, max_unorm: float, beta1: float = 0.9,
                                        beta2: float = 0.999, beta3: float = 0.9999,
                                        alpha: float = 5.0, eps: float = 1e-8,
                                        weight_decay: float = 0.0, skip_zeros: bool = False,
                                        decay_after: bool = False, stream=None) -> None:
    """``optimizer_update_32bit_clip`` without a workspace: the library's
    static device scratch holds the partial norms, so nothing is allocated
    (n up to ``clip_noalloc_max_elements()``).  Calls that overlap in time
    on one GPU share that scratch and race."""
    k = _kind(kind, decay_after)
    n, dt, _ = _tensor_args(k, param, grad, state1, state2)
    lib = load()
    with _on_device(param.device):
        st = lib.optimizer_update_32bit_clip_noalloc(k, dt, param.data_ptr(), grad.data_ptr(),
                                                     state1.data_ptr(), _ptr(state2), n, beta1, beta2,
                                                     beta3, alpha, eps, weight_decay, int(step), lr,
                                                     int(bool(skip_zeros)), max_unorm,
                                                     _stream(param, stream))
    check(st, lib)


def clip_noalloc_max_elements() -> int:
    """Largest tensor ``optimizer_update_32bit_clip_noalloc`` accepts."""
    return int(load().ou_clip_noalloc_max_elements())


def _segments(kind: int, segments) -> ctypes.Array:
    arr = (_lib.ou_segment * len(segments))()
    for i, (p, g, s1, s2) in enumerate(segments):
        n, dt, _ = _tensor_args(kind, p, g, s1, s2)
        arr[i] = _lib.ou_segment(p.data_ptr(), g.data_ptr(), s1.data_ptr(), _ptr(s2), n, dt, 0)
    return arr


def optimizer_update_32bit_multi(kind, segments, hp: HParams, step: int, stream=None,
                                 decay_after: bool = False) -> None:
    """One update of a collection [(param, grad, state1, state2), ...]
    (state2 None for the one-state kinds): one
    launch per dtype group.  Builds the table on every call and waits for
    the stream; use ``Plan`` for repeated steps."""
    k = _kind(kind, decay_after)
    if not segments:
        return
    arr = _segments(k, segments)
    lib = load()
    c = hp.c(step)
    dev = segments[0][0].device
    with _on_device(dev):
        st = lib.optimizer_update_32bit_multi(k, arr, len(segments), ctypes.byref(c),
                                              _stream(segments[0][0], stream))
    check(st, lib)


class Plan:
    """Device-resident segment table of a fixed collection (``ou_plan``).

    The tensors' storage must stay allocated and in place until ``close``;
    the plan keeps references to them."""

    def __init__(self, kind, segments, decay_after: bool = False):
        self.kind = _kind(kind, decay_after)
        self._tensors = [tuple(s) for s in segments]
        self.device = (self._tensors[0][0].device if self._tensors
                       else torch.device("cuda", torch.cuda.current_device()))
        arr = _segments(self.kind, self._tensors)
        self._lib = load()
        h = ctypes.c_void_p()
        with _on_device(self.device):
            check(self._lib.ou_plan_create(self.kind, arr, len(self._tensors), ctypes.byref(h)),
                  self._lib)
        self._h = h
        self._index = self.device.index

    def step(self, hp: HParams, step: int, stream=None) -> None:
        """One step (``ou_plan_step``): the per-step path of a collection,
        kept to a few attribute lookups and one call into the library when
        the plan's device is current."""
        c = hp.c(step)
        idx = self._index
        sh = _raw_stream(idx) if stream is None else _stream_arg(stream)
        fn = self._lib.ou_plan_step
        h = self._h.value
        st = fn(h, c, sh) if _GET_DEVICE() == idx else _on(idx, fn, h, c, sh)
        if st:
            check(st, self._lib)

    def step_clip(self, hp: HParams, step: int, max_unorm: float, stream=None) -> None:
        """One step with update-norm clipping per tensor (``ou_plan_step_clip``)."""
        c = hp.c(step)
        with _on_device(self.device):
            check(self._lib.ou_plan_step_clip(self._h, ctypes.byref(c), max_unorm,
                                              self._stream(stream)), self._lib)

    def clip_factors(self) -> list[float]:
        """Clip factor of every tensor in the last clipped step (synchronous)."""
        out = (ctypes.c_float * len(self._tensors))()
        with _on_device(self.device):
            torch.cuda.synchronize(self.device)
            check(self._lib.ou_plan_clip_factors(self._h, out, len(self._tensors)), self._lib)
        return list(out)

    def graph_step(self, hp: HParams, step: int, stream=None) -> None:
        c = hp.c(step)
        with _on_device(self.device):
            check(self._lib.ou_plan_graph_step(self._h, ctypes.byref(c), self._stream(stream)),
                  self._lib)

    def graph_step_clip(self, hp: HParams, step: int, max_unorm: float, stream=None) -> None:
        """The clipped step through its HIP graph (``ou_plan_graph_step_clip``)."""
        c = hp.c(step)
        with _on_device(self.device):
            check(self._lib.ou_plan_graph_step_clip(self._h, ctypes.byref(c), max_unorm,
                                                    self._stream(stream)), self._lib)

    def describe(self) -> dict:
        g = ctypes.c_int32()
        w = ctypes.c_int64()
        e = ctypes.c_int64()
        check(self._lib.ou_plan_describe(self._h, ctypes.byref(g), ctypes.byref(w), ctypes.byref(e)),
              self._lib)
        return {"groups": g.value, "work_items": w.value, "elements": e.value}

    def _stream(self, stream) -> int:
        if stream is None:
            return _raw_stream(self.device.index)
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            torch.cuda.synchronize(self.device)
            self._lib.ou_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------- 8-bit block-wise states

QBLOCK = _lib.OU_8BIT_BLOCK


def qmap(signed: bool) -> torch.Tensor:
    """Magnitudes of the 8-bit dynamic type (128 signed, 256 unsigned), as
    the library defines them (``ou_8bit_qmap``)."""
    count = 128 if signed else 256
    out = (ctypes.c_float * count)()
    lib = load()
    check(lib.ou_8bit_qmap(int(bool(signed)), out, count), lib)
    return torch.tensor(list(out), dtype=torch.float32)


def state8_sizes(kind, n: int) -> tuple[int, int, int, int]:
    """Sizes of (state1 codes, state2 codes, absmax1, absmax2) for n elements."""
    k = 2 if (_kind(kind) & ~_lib.OU_DECAY_AFTER) == _lib.OU_ADEMAMIX else 1
    nb = -(-n // QBLOCK)
    return k * n, n, k * nb, nb


def _tensor8_args(kind: int, param, grad, state1, state2, absmax1,
                  absmax2) -> tuple[int, int, int]:
    """Check the six operands of an 8-bit update; returns (n, dtype code,
    device index)."""
    ts = (param, grad, state1, state2, absmax1, absmax2)
    try:
        dev = param.get_device()
        ok = dev >= 0 and all(t.get_device() == dev and t.is_contiguous() for t in ts)
    except AttributeError:
        ok = False
    if not ok:
        for name, t in zip(("param", "grad", "state1", "state2", "absmax1", "absmax2"), ts):
            if not isinstance(t, torch.Tensor) or t.get_device() < 0:
                raise ValueError(f"{name} must be a tensor on a HIP device")
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        raise ValueError("all tensors must be on one device")
    dt = DTYPES.get(param.dtype)
    if dt is None or grad.dtype != param.dtype:
        raise ValueError("param and grad must share one of float32/float16/bfloat16")
    if state1.dtype != torch.uint8 or state2.dtype != torch.uint8:
        raise ValueError("8-bit states must be uint8")
    if absmax1.dtype != torch.float32 or absmax2.dtype != torch.float32:
        raise ValueError("absmax buffers must be float32")
    n = param.numel()
    want = state8_sizes(kind, n)
    got = (state1.numel(), state2.numel(), absmax1.numel(), absmax2.numel())
    if grad.numel() != n or got != want:
        raise ValueError(f"sizes: n {n}, grad {grad.numel()}, states/absmax {got} (want {want})")
    return n, dt, dev


def optimizer_update_8bit_blockwise(kind, param: torch.Tensor, grad: torch.Tensor,
                                    state1: torch.Tensor, state2: torch.Tensor,
                                    absmax1: torch.Tensor, absmax2: torch.Tensor, *, step: int,
                                    lr: float, beta1: float = 0.9, beta2: float = 0.999,
                                    beta3: float = 0.9999, alpha: float = 5.0, eps: float = 1e-8,
                                    weight_decay: float = 0.0, skip_zeros: bool = False,
                                    decay_after: bool = False, stream=None) -> None:
    """One update with 8-bit block-wise states (uint8 codes, fp32 absmax per
    256 elements), in place."""
    k = _kind(kind, decay_after)
    n, dt, dev = _tensor8_args(k, param, grad, state1, state2, absmax1, absmax2)
    lib = load()
    args = (k, dt, param.data_ptr(), grad.data_ptr(), state1.data_ptr(), state2.data_ptr(),
            absmax1.data_ptr(), absmax2.data_ptr(), n, beta1, beta2, beta3, alpha, eps,
            weight_decay, int(step), lr, int(bool(skip_zeros)),
            _raw_stream(dev) if stream is None else _stream_arg(stream))
    fn = lib.optimizer_update_8bit_blockwise
    st = fn(*args) if _GET_DEVICE() == dev else _on(dev, fn, *args)
    if st:
        check(st, lib)


class Plan8:
    """Device-resident segment table of a fixed 8-bit collection
    (``ou_plan8``): [(param, grad, state1, state2, absmax1, absmax2), ...]."""

    def __init__(self, kind, segments, decay_after: bool = False):
        self.kind = _kind(kind, decay_after)
        self._tensors = [tuple(s) for s in segments]
        self.device = (self._tensors[0][0].device if self._tensors
                       else torch.device("cuda", torch.cuda.current_device()))
        arr = (_lib.ou_segment8 * len(self._tensors))()
        for i, s in enumerate(self._tensors):
            n, dt, _ = _tensor8_args(self.kind, *s)
            arr[i] = _lib.ou_segment8(*(t.data_ptr() for t in s), n, dt, 0)
        self._lib = load()
        h = ctypes.c_void_p()
        with _on_device(self.device):
            check(self._lib.ou_plan8_create(self.kind, arr, len(self._tensors), ctypes.byref(h)),
                  self._lib)
        self._h = h
        self._index = self.device.index

    def step(self, hp: HParams, step: int, stream=None) -> None:
        c = hp.c(step)
        idx = self._index
        sh = _raw_stream(idx) if stream is None else _stream_arg(stream)
        fn = self._lib.ou_plan8_step
        h = self._h.value
        st = fn(h, c, sh) if _GET_DEVICE() == idx else _on(idx, fn, h, c, sh)
        if st:
            check(st, self._lib)

    def graph_step(self, hp: HParams, step: int, stream=None) -> None:
        """The same step replayed from a HIP graph (``ou_plan8_graph_step``)."""
        c = hp.c(step)
        sh = (_raw_stream(self.device.index) if stream is None
              else (stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)))
        with _on_device(self.device):
            check(self._lib.ou_plan8_graph_step(self._h, ctypes.byref(c), sh), self._lib)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            torch.cuda.synchronize(self.device)
            self._lib.ou_plan8_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Graph:
    """One HIP graph over the plain steps of several plans (``ou_graph``):
    32-bit plans, then 8-bit plans, replayed as one chain of launches with
    each step's scalars written into its nodes.  The plans must stay open
    until this graph is closed."""

    def __init__(self, plans=(), plans8=()):
        self._plans = [p for p in plans if p is not None]
        self._plans8 = [p for p in plans8 if p is not None]
        every = self._plans + self._plans8
        self.device = every[0].device if every else torch.device("cuda", torch.cuda.current_device())
        if any(p.device != self.device for p in every):
            raise ValueError("all plans of a graph must be on one device")
        self._lib = load()
        a = (ctypes.c_void_p * max(1, len(self._plans)))(*[p._h.value for p in self._plans])
        b = (ctypes.c_void_p * max(1, len(self._plans8)))(*[p._h.value for p in self._plans8])
        h = ctypes.c_void_p()
        check(self._lib.ou_graph_create(a, len(self._plans), b, len(self._plans8), ctypes.byref(h)),
              self._lib)
        self._h = h

    def step(self, hp: HParams, step: int, stream=None) -> None:
        c = hp.c(step)
        sh = (_raw_stream(self.device.index) if stream is None
              else (stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)))
        with _on_device(self.device):
            check(self._lib.ou_graph_step(self._h, ctypes.byref(c), sh), self._lib)

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            torch.cuda.synchronize(self.device)
            self._lib.ou_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


__all__ += ["QBLOCK", "qmap", "state8_sizes", "optimizer_update_8bit_blockwise", "Plan8", "Graph"]

from .optim import AdamW32, AdEMAMix32, Adagrad32, Lion32, Momentum32, RMSprop32  # noqa: E402
from .optim import AdamW8bit, AdEMAMix8bit  # noqa: E402

__all__ += ["AdamW32", "AdEMAMix32", "Momentum32", "RMSprop32", "Adagrad32", "Lion32",
            "TWO_STATE", "AdamW8bit", "AdEMAMix8bit"]
