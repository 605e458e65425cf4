"""Collection optimizers over a fixed parameter list (argument marshalling only).

``AdamW32`` and ``AdEMAMix32`` (two fp32 states per parameter) play the part of the 32-bit collection
optimizers that the page "Investigate a 256-thread SM103 path for small
32-bit optimizer tensors" times in its eager ``optimizer.step()`` workloads
(section "B300 benchmark and acceptance"): they own the fp32 states of every
parameter and update the whole collection per step through one plan (one
launch per dtype group), its HIP-graph replay, or, for comparison, one
direct call per tensor.  ``Momentum32``, ``RMSprop32``, ``Adagrad32`` and
``Lion32`` are the one-state kinds of the same 32-bit update family, with the
same three step paths.  ``AdamW8bit`` and ``AdEMAMix8bit`` keep the
moments of tensors of at least ``min_8bit_size`` elements (4,096 by
default, the page's setting) as 8-bit block-wise states and route the
smaller ones to the 32-bit path, one plan each.

Parameters and gradients must be contiguous CUDA (HIP) tensors whose
storage stays in place for the optimizer's lifetime: the plan holds their
addresses.  When the optimizer takes its gradients from ``Parameter.grad``
(no ``grads=`` argument), every step checks that each parameter's ``.grad``
is still the tensor the plan was built on: a ``zero_grad(set_to_none=True)``
elsewhere (torch's default) makes the next backward allocate new gradient
tensors, and the plan is then rebuilt on them (a step with a parameter whose
``.grad`` is None raises).  The optimizers' own ``zero_grad()`` zeroes the
captured gradients in place, which keeps the plan.
"""
from __future__ import annotations

import torch

from . import (DTYPES, TWO_STATE, Graph, HParams, Plan, Plan8, _kind, _on_device, _ptr, _raw_stream,
               _tensor_args, check, clip_workspace, load, optimizer_update_8bit_blockwise,
               optimizer_update_32bit, optimizer_update_32bit_clip, state8_sizes, state_sizes)


class _Collection:
    kind = "adam"

    def __init__(self, params, hp: HParams, grads=None, max_unorm: float = 0.0,
                 decay_after: bool = False):
        params = list(params)
        self.params, self.grads, sources = _params_and_grads(params, grads)
        self._followed = _followed(sources)
        self.hp = hp
        self.decay_after = bool(decay_after)
        two = _kind(self.kind) in TWO_STATE
        if max_unorm and not two:
            raise ValueError("update-norm clipping is defined for Adam and AdEMAMix only")
        self.state1, self.state2 = [], []
        for p in self.params:
            n1, n2 = state_sizes(self.kind, p.numel())
            self.state1.append(torch.zeros(n1, dtype=torch.float32, device=p.device))
            self.state2.append(torch.zeros(n2, dtype=torch.float32, device=p.device)
                               if two else None)
        self.step_count = 0
        self.max_unorm = float(max_unorm)
        self._workspace = None
        self._direct = None
        self.plan = self._build_plan()

    def _build_plan(self) -> Plan:
        return Plan(self.kind, list(zip(self.params, self.grads, self.state1, self.state2)),
                    decay_after=self.decay_after)

    def _sync_grads(self) -> None:
        """Rebuild the plan if a parameter's .grad is no longer the captured tensor."""
        if self._followed and _grads_moved(self._followed, self.grads):
            self.plan.close()
            self.plan = self._build_plan()
            self._direct = None

    def zero_grad(self, set_to_none: bool = False) -> None:
        """Zero the captured gradients in place (the plan keeps its
        addresses; set_to_none is accepted for torch's signature and ignored)."""
        del set_to_none
        _zero_in_place(self._followed, self.grads)

    def segments(self):
        return list(zip(self.params, self.grads, self.state1, self.state2))

    def step(self, graph: bool = False, stream=None) -> None:
        """One step of the whole collection: plan launch, or graph replay.
        With max_unorm > 0 every tensor's update is clipped by its own norms."""
        self._sync_grads()
        self.step_count += 1
        if self.max_unorm > 0:
            (self.plan.graph_step_clip if graph else self.plan.step_clip)(
                self.hp, self.step_count, self.max_unorm, stream)
        elif graph:
            self.plan.graph_step(self.hp, self.step_count, stream)
        else:
            self.plan.step(self.hp, self.step_count, stream)

    @torch.no_grad()
    def step_per_tensor(self, stream=None) -> None:
        """The same step as one direct call per tensor (the tensors were
        checked when the optimizer was built; only the step changes)."""
        self._sync_grads()
        self.step_count += 1
        h = self.hp
        if self.max_unorm > 0:
            if self._workspace is None:
                self._workspace = clip_workspace(max(p.numel() for p in self.params),
                                                 self.params[0].device)
            for p, g, s1, s2 in self.segments():   # one workspace, reused in stream order
                optimizer_update_32bit_clip(self.kind, p, g, s1, s2, step=self.step_count,
                                            lr=h.lr, max_unorm=self.max_unorm,
                                            workspace=self._workspace, beta1=h.beta1,
                                            beta2=h.beta2, beta3=h.beta3, alpha=h.alpha,
                                            eps=h.eps, weight_decay=h.weight_decay,
                                            skip_zeros=h.skip_zeros,
                                            decay_after=self.decay_after, stream=stream)
            return
        if self._direct is None:
            for p, g, s1, s2 in self.segments():   # full checks once
                _tensor_args(_kind(self.kind), p, g, s1, s2)
            self._direct = [(_kind(self.kind, self.decay_after), DTYPES[p.dtype], p.data_ptr(), g.data_ptr(),
                             s1.data_ptr(), _ptr(s2), p.numel())
                            for p, g, s1, s2 in self.segments()]
        lib = load()
        sh = (_raw_stream(self.params[0].device.index) if stream is None
              else (stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)))
        tail = (h.beta1, h.beta2, h.beta3, h.alpha, h.eps, h.weight_decay, self.step_count, h.lr,
                int(bool(h.skip_zeros)), sh)
        fn = lib.optimizer_update_32bit
        with _on_device(self.params[0].device):
            for args in self._direct:
                st = fn(*args, *tail)
                if st:
                    check(st, lib)

    def state_dict(self) -> dict:
        return {"step": self.step_count,
                "state1": [s.clone() for s in self.state1],
                "state2": [None if s is None else s.clone() for s in self.state2]}

    def load_state_dict(self, sd: dict) -> None:
        self.step_count = int(sd["step"])
        for dst, src in zip(self.state1, sd["state1"]):
            dst.copy_(src)
        for dst, src in zip(self.state2, sd["state2"]):
            if dst is not None:
                dst.copy_(src)

    def close(self) -> None:
        self.plan.close()


class AdamW32(_Collection):
    """Adam with decoupled weight decay (weight_decay = 0 gives Adam)."""
    kind = "adam"

    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01,
                 skip_zeros=False, grads=None, max_unorm=0.0, decay_after=False):
        super().__init__(params, HParams(lr=lr, beta1=betas[0], beta2=betas[1], eps=eps,
                                         weight_decay=weight_decay, skip_zeros=skip_zeros), grads,
                         max_unorm, decay_after)


class AdEMAMix32(_Collection):
    """AdEMAMix: Adam plus a slow EMA (beta3) mixed in with weight alpha."""
    kind = "ademamix"

    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999, 0.9999), alpha=5.0, eps=1e-8,
                 weight_decay=0.01, skip_zeros=False, grads=None, max_unorm=0.0,
                 decay_after=False):
        super().__init__(params, HParams(lr=lr, beta1=betas[0], beta2=betas[1], beta3=betas[2],
                                         alpha=alpha, eps=eps, weight_decay=weight_decay,
                                         skip_zeros=skip_zeros), grads, max_unorm, decay_after)


class Momentum32(_Collection):
    """SGD with heavy-ball momentum (no dampening, no Nesterov) and L2
    weight decay added to the gradient."""
    kind = "momentum"

    def __init__(self, params, lr=1e-2, momentum=0.9, weight_decay=0.0, skip_zeros=False,
                 grads=None):
        super().__init__(params, HParams(lr=lr, beta1=momentum, beta2=0.0, eps=0.0,
                                         weight_decay=weight_decay, skip_zeros=skip_zeros), grads)


class RMSprop32(_Collection):
    """RMSprop (smoothing constant alpha, eps outside the root, L2 weight
    decay added to the gradient)."""
    kind = "rmsprop"

    def __init__(self, params, lr=1e-2, alpha=0.99, eps=1e-8, weight_decay=0.0,
                 skip_zeros=False, grads=None):
        super().__init__(params, HParams(lr=lr, beta1=alpha, beta2=0.0, eps=eps,
                                         weight_decay=weight_decay, skip_zeros=skip_zeros), grads)


class Adagrad32(_Collection):
    """Adagrad (accumulator starts at zero, no learning-rate decay, L2
    weight decay added to the gradient)."""
    kind = "adagrad"

    def __init__(self, params, lr=1e-2, eps=1e-10, weight_decay=0.0, skip_zeros=False,
                 grads=None):
        super().__init__(params, HParams(lr=lr, beta1=0.0, beta2=0.0, eps=eps,
                                         weight_decay=weight_decay, skip_zeros=skip_zeros), grads)


class Lion32(_Collection):
    """Lion: sign of the beta1 interpolation, moment tracked with beta2,
    decoupled weight decay."""
    kind = "lion"

    def __init__(self, params, lr=1e-4, betas=(0.9, 0.99), weight_decay=0.0, skip_zeros=False,
                 grads=None, decay_after=False):
        super().__init__(params, HParams(lr=lr, beta1=betas[0], beta2=betas[1], eps=0.0,
                                         weight_decay=weight_decay, skip_zeros=skip_zeros), grads,
                         0.0, decay_after)


def _params_and_grads(params, grads):
    """(parameter data, gradients, sources): sources[i] is the Parameter
    whose .grad the optimizer follows, or None when the gradients were given
    explicitly (or the parameter is a plain tensor)."""
    params = list(params)
    ps = [p.data if isinstance(p, torch.nn.Parameter) else p for p in params]
    if grads is not None:
        return ps, list(grads), [None] * len(ps)
    gs, sources = [], []
    for p, src in zip(ps, params):
        g = getattr(src, "grad", None)
        if g is None:
            g = torch.zeros_like(p)
            if isinstance(src, torch.nn.Parameter):
                src.grad = g
        gs.append(g)
        sources.append(src if isinstance(src, torch.nn.Parameter) else None)
    return ps, gs, sources


def _followed(sources) -> list:
    """(index, Parameter) of the parameters whose .grad the optimizer follows."""
    return [(i, src) for i, src in enumerate(sources) if src is not None]


def _grads_moved(followed, grads) -> bool:
    """True (and grads updated) if a followed Parameter's .grad is a tensor
    at another address than the captured one; raises if it is None.  The
    same address (the allocator handed the memory back) needs no rebuild.
    Gradients given explicitly are not followed and cost nothing here."""
    moved = False
    for i, src in followed:
        g = src.grad
        if g is grads[i]:
            continue
        if g is None:
            raise RuntimeError(f"parameter {i} has no .grad: run backward before step(), and use the "
                               "optimizer's zero_grad() (in place) rather than set_to_none=True")
        if g.shape != grads[i].shape or g.dtype != grads[i].dtype or g.device != grads[i].device:
            raise RuntimeError(f"parameter {i}: .grad changed shape, dtype or device")
        if not g.is_contiguous():
            raise RuntimeError(f"parameter {i}: .grad is not contiguous")
        moved |= g.data_ptr() != grads[i].data_ptr()
        grads[i] = g
    return moved


def _zero_in_place(followed, grads) -> None:
    for i, src in followed:
        if src.grad is not None and src.grad is not grads[i]:
            src.grad.zero_()
    torch._foreach_zero_(list(grads))


class _Collection8:
    """Tensors of at least ``min_8bit_size`` elements keep 8-bit block-wise
    states (uint8 codes, fp32 absmax per 256 elements) and step through one
    8-bit plan; smaller tensors keep fp32 states and step through one 32-bit
    plan."""
    kind = "adam"

    def __init__(self, params, hp: HParams, grads=None, min_8bit_size: int = 4096,
                 decay_after: bool = False):
        self.params, self.grads, sources = _params_and_grads(params, grads)
        self._followed = _followed(sources)
        self.hp = hp
        self.min_8bit_size = int(min_8bit_size)
        self.decay_after = bool(decay_after)
        self.step_count = 0
        self.state = []            # per parameter: ("8bit", s1, s2, a1, a2) or ("32bit", s1, s2)
        for p in self.params:
            if p.numel() >= self.min_8bit_size:
                n1, n2, na1, na2 = state8_sizes(self.kind, p.numel())
                st = ("8bit", torch.zeros(n1, dtype=torch.uint8, device=p.device),
                      torch.zeros(n2, dtype=torch.uint8, device=p.device),
                      torch.zeros(na1, dtype=torch.float32, device=p.device),
                      torch.zeros(na2, dtype=torch.float32, device=p.device))
            else:
                n1, n2 = state_sizes(self.kind, p.numel())
                st = ("32bit", torch.zeros(n1, dtype=torch.float32, device=p.device),
                      torch.zeros(n2, dtype=torch.float32, device=p.device))
            self.state.append(st)
        self.plan8 = self.plan32 = None
        self._graph = None
        self._build_plans()

    def _build_plans(self) -> None:
        seg8, seg32 = [], []
        for p, g, st in zip(self.params, self.grads, self.state):
            (seg8 if st[0] == "8bit" else seg32).append((p, g, *st[1:]))
        self.plan8 = Plan8(self.kind, seg8, decay_after=self.decay_after) if seg8 else None
        self.plan32 = Plan(self.kind, seg32, decay_after=self.decay_after) if seg32 else None

    def _sync_grads(self) -> None:
        """Rebuild the plans if a parameter's .grad is no longer the captured tensor."""
        if self._followed and _grads_moved(self._followed, self.grads):
            self.close()
            self._build_plans()

    def zero_grad(self, set_to_none: bool = False) -> None:
        """Zero the captured gradients in place (the plans keep their
        addresses; set_to_none is accepted for torch's signature and ignored)."""
        del set_to_none
        _zero_in_place(self._followed, self.grads)

    def step(self, graph: bool = False, stream=None) -> None:
        """One step: the 8-bit plan, then the 32-bit plan (one launch per
        dtype group each), or one HIP graph over both (built on the first
        graph step)."""
        self._sync_grads()
        self.step_count += 1
        if graph:
            if self._graph is None:
                self._graph = Graph([self.plan32], [self.plan8])
            self._graph.step(self.hp, self.step_count, stream)
            return
        if self.plan8 is not None:
            self.plan8.step(self.hp, self.step_count, stream)
        if self.plan32 is not None:
            self.plan32.step(self.hp, self.step_count, stream)

    @torch.no_grad()
    def step_per_tensor(self, stream=None) -> None:
        """The same step as one direct call per tensor (the eager loop)."""
        self._sync_grads()
        self.step_count += 1
        h = self.hp
        kw = dict(step=self.step_count, lr=h.lr, beta1=h.beta1, beta2=h.beta2, beta3=h.beta3,
                  alpha=h.alpha, eps=h.eps, weight_decay=h.weight_decay,
                  skip_zeros=h.skip_zeros, decay_after=self.decay_after, stream=stream)
        for p, g, st in zip(self.params, self.grads, self.state):
            if st[0] == "8bit":
                optimizer_update_8bit_blockwise(self.kind, p, g, *st[1:], **kw)
            else:
                optimizer_update_32bit(self.kind, p, g, *st[1:], **kw)

    def state_dict(self) -> dict:
        return {"step": self.step_count,
                "state": [(st[0], *[x.clone() for x in st[1:]]) for st in self.state]}

    def load_state_dict(self, sd: dict) -> None:
        self.step_count = int(sd["step"])
        for dst, src in zip(self.state, sd["state"]):
            if dst[0] != src[0]:
                raise ValueError("state layout differs (min_8bit_size or shapes changed)")
            for a, b in zip(dst[1:], src[1:]):
                a.copy_(b)

    def close(self) -> None:
        if self._graph is not None:       # the graph goes before its plans
            self._graph.close()
            self._graph = None
        for plan in (self.plan8, self.plan32):
            if plan is not None:
                plan.close()


class AdamW8bit(_Collection8):
    """AdamW with 8-bit block-wise moments for tensors of at least
    min_8bit_size elements (32-bit states below)."""
    kind = "adam"

    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01,
                 skip_zeros=False, grads=None, min_8bit_size=4096, decay_after=False):
        super().__init__(params, HParams(lr=lr, beta1=betas[0], beta2=betas[1], eps=eps,
                                         weight_decay=weight_decay, skip_zeros=skip_zeros), grads,
                         min_8bit_size, decay_after)


class AdEMAMix8bit(_Collection8):
    """AdEMAMix with 8-bit block-wise moments for tensors of at least
    min_8bit_size elements (32-bit states below)."""
    kind = "ademamix"

    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999, 0.9999), alpha=5.0, eps=1e-8,
                 weight_decay=0.01, skip_zeros=False, grads=None, min_8bit_size=4096,
                 decay_after=False):
        super().__init__(params, HParams(lr=lr, beta1=betas[0], beta2=betas[1], beta3=betas[2],
                                         alpha=alpha, eps=eps, weight_decay=weight_decay,
                                         skip_zeros=skip_zeros), grads, min_8bit_size, decay_after)
