"""GPU tests of the collection entry points and stream/graph plumbing.

A plan over a mixed-dtype collection (one launch per dtype group), the eager
multi-tensor entry, work on a non-default stream, and a plan step (plain or
clipped) captured into the caller's own HIP graph: each must give, bitwise,
what one direct call per tensor gives, and match the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

MIXED = [("fp32", 1000), ("bf16", 4096), ("fp16", 77), ("fp32", 1 << 16), ("bf16", 3),
         ("fp16", 20000), ("fp32", 1), ("bf16", 70001)]


def _collection(kind, seed):
    gen = W.rng(0, 11, seed)
    host = []
    for storage, n in MIXED:
        host.append((storage, W.params(n, storage, gen), W.grads(n, "normal", storage, gen)))
    return host


def _device(kind, host):
    k = 2 if kind == "ademamix" else 1
    return [(H.to_dev(p, s), H.to_dev(g, s), torch.zeros(k * p.size, device="cuda"),
             torch.zeros(p.size, device="cuda")) for s, p, g in host]


def _bits(t):
    return W.from_torch(t).tobytes()


def _direct_reference(L, kind, host, hp, steps):
    segs = _device(kind, host)
    for t in range(1, steps + 1):
        for (s, _, _), (p, g, s1, s2) in zip(host, segs):
            assert H.raw_update(L, kind, s, p, g, s1, s2, p.numel(), hp, t, H.stream_handle()) == 0
    torch.cuda.synchronize()
    return segs


@pytest.mark.parametrize("kind", ["adam", "ademamix"])
def test_mixed_dtype_plan_graph_and_multi(kind):
    """A collection mixing fp32, fp16 and bf16: the plan has three dtype
    groups (three launches, three graph nodes).  Plan steps, graph replays
    and the eager multi entry equal per-tensor direct calls bitwise, and the
    oracle."""
    import optimizer_update_amd as ou
    L = H.lib()
    orc = O.load()
    hp = O.HParams(lr=1e-3, weight_decay=0.01, skip_zeros=True)
    php = H.pkg_hp(hp)
    host = _collection(kind, 1)
    steps = 5
    ref = _direct_reference(L, kind, host, hp, steps)
    a = _device(kind, host)
    plan = ou.Plan(kind, a)
    assert plan.describe()["groups"] == 3
    b = _device(kind, host)
    c = _device(kind, host)
    for t in range(1, steps + 1):
        plan.step(php, t)
        ou.optimizer_update_32bit_multi(kind, c, php, t)
    torch.cuda.synchronize()
    plan.close()
    gplan = ou.Plan(kind, b)
    for t in range(1, steps + 1):
        gplan.graph_step(php, t)
    torch.cuda.synchronize()
    gplan.close()
    for name, got in (("plan", a), ("graph", b), ("multi", c)):
        for i, (r, x) in enumerate(zip(ref, got)):
            for j in (0, 2, 3):
                assert _bits(r[j]) == _bits(x[j]), (name, i, j)
    for (s, p0, g0), (p, _, s1, s2) in zip(host, ref):
        pr, (s1r, s2r) = p0.copy(), W.zero_states(p0.size, kind)
        for t in range(1, steps + 1):
            orc.update_f32(H.KIND[kind], H.DT[s], pr, g0, s1r, s2r, hp, t)
        H.assert_parity(W.from_torch(p), pr, s, f"p {s} {p0.size}")
        H.assert_parity(W.from_torch(s1), s1r, "fp32", f"s1 {s} {p0.size}")
        H.assert_parity(W.from_torch(s2), s2r, "fp32", f"s2 {s} {p0.size}")


def test_non_default_stream_orders_with_torch_work():
    """Updates enqueued on a side stream run after torch work queued before
    them on that stream and before work queued after them."""
    import optimizer_update_amd as ou
    n = 1 << 20
    side = torch.cuda.Stream()
    p = torch.zeros(n, device="cuda")
    g = torch.empty(n, device="cuda")
    s1 = torch.zeros(n, device="cuda")
    s2 = torch.zeros(n, device="cuda")
    ref = [torch.zeros(n, device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        g.fill_(0.5)          # must land before the update reads g
        p.fill_(1.0)
        ou.optimizer_update_32bit("adam", p, g, s1, s2, step=1, lr=1e-3, stream=side)
        out = p * 2.0         # must see the updated p
    side.synchronize()
    with torch.cuda.stream(side):
        ref[1].fill_(0.5)
        ref[0].fill_(1.0)
    side.synchronize()
    ou.optimizer_update_32bit("adam", ref[0], ref[1], ref[2], ref[3], step=1, lr=1e-3)
    torch.cuda.synchronize()
    assert torch.equal(p, ref[0]) and torch.equal(out, ref[0] * 2.0)
    assert torch.equal(s1, ref[2]) and torch.equal(s2, ref[3])


def test_plan_step_captured_in_caller_graph():
    """ou_plan_step is capture-safe: captured into a torch CUDA graph it
    replays the captured step (fixed scalars).  Each of several replays, with
    eager work and synchronisations between them, equals the same step run
    eagerly on a copy."""
    import optimizer_update_amd as ou
    kind = "adam"
    host = _collection(kind, 2)
    hp = ou.HParams(lr=1e-3, weight_decay=0.01)
    segs = _device(kind, host)
    eager = _device(kind, host)
    plan = ou.Plan(kind, segs)
    eplan = ou.Plan(kind, eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    # capture: the state buffers are restored to zero before replays below
    with torch.cuda.graph(graph, stream=s):
        plan.step(hp, 1, stream=s)
    torch.cuda.synchronize()
    p0 = [x[0].clone() for x in segs]
    for rep in range(4):
        for (p, _, s1, s2), pp in zip(segs, p0):
            p.copy_(pp)
            s1.zero_()
            s2.zero_()
        for (p, _, s1, s2), (sh, pinit, _) in zip(eager, host):
            p.copy_(W.to_torch(pinit, sh, "cuda"))
            s1.zero_()
            s2.zero_()
        torch.cuda.synchronize()
        graph.replay()
        eplan.step(hp, 1)
        torch.zeros(1 << 16, device="cuda").add_(1.0)   # unrelated eager work
        torch.cuda.synchronize()
        for x, y in zip(segs, eager):
            for j in (0, 2, 3):
                assert _bits(x[j]) == _bits(y[j]), (rep, j)
    plan.close()
    eplan.close()


def test_plan_step_clip_captured_in_caller_graph():
    """ou_plan_step_clip (three launches per dtype group, partial norms in the
    plan) is capture-safe too: each replay of the captured clipped step, with
    eager work between replays, equals the same step run eagerly, clip
    factors included."""
    import optimizer_update_amd as ou
    kind = "adam"
    host = _collection(kind, 4)
    hp = ou.HParams(lr=1e-2, weight_decay=0.01)
    segs = _device(kind, host)
    eager = _device(kind, host)
    plan = ou.Plan(kind, segs)
    eplan = ou.Plan(kind, eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        plan.step_clip(hp, 1, 0.05, stream=s)
    torch.cuda.synchronize()
    p0 = [x[0].clone() for x in segs]
    for rep in range(3):
        for (p, _, s1, s2), pp in zip(segs, p0):
            p.copy_(pp)
            s1.zero_()
            s2.zero_()
        for (p, _, s1, s2), (sh, pinit, _) in zip(eager, host):
            p.copy_(W.to_torch(pinit, sh, "cuda"))
            s1.zero_()
            s2.zero_()
        torch.cuda.synchronize()
        graph.replay()
        eplan.step_clip(hp, 1, 0.05)
        torch.zeros(1 << 16, device="cuda").add_(1.0)   # unrelated eager work
        torch.cuda.synchronize()
        for x, y in zip(segs, eager):
            for j in (0, 2, 3):
                assert _bits(x[j]) == _bits(y[j]), (rep, j)
        fa, fb = plan.clip_factors(), eplan.clip_factors()
        assert fa == fb and min(fa) < 1.0, (fa, fb)
    plan.close()
    eplan.close()


def test_graph_step_rejected_under_capture_and_multi_too():
    """Entry points that build or launch their own graph, or allocate, refuse
    to run inside a caller's capture instead of corrupting it."""
    import optimizer_update_amd as ou
    host = _collection("adam", 3)
    segs = _device("adam", host)
    plan = ou.Plan("adam", segs)
    hp = ou.HParams()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    errors = []
    x = torch.zeros(1, device="cuda")
    try:
        with torch.cuda.graph(graph, stream=s):
            x.add_(1.0)      # keep the captured graph non-empty
            for fn in (lambda: plan.graph_step(hp, 1, stream=s),
                       lambda: plan.graph_step_clip(hp, 1, 0.5, stream=s),
                       lambda: ou.optimizer_update_32bit_multi("adam", segs, hp, 1, stream=s)):
                try:
                    fn()
                except ou.OptimizerUpdateError as e:
                    errors.append(e.status)
    finally:
        torch.cuda.synchronize()
    assert errors == [-7, -7, -7]
    plan.close()


@pytest.mark.parametrize("kind", ["adam", "ademamix"])
def test_one_graph_over_several_plans(kind):
    """ou_graph: one HIP graph over a mixed-dtype 32-bit plan (three dtype
    groups), a second 32-bit plan with the other decay order and a
    mixed-dtype 8-bit plan (six chained launches).  Every replay equals the
    plans' own steps bitwise, with eager torch work and synchronisations
    between replays."""
    import optimizer_update_amd as ou
    hp = ou.HParams(lr=1e-3, weight_decay=0.01)
    host = _collection(kind, 3)
    host_b = _collection(kind, 4)
    gen8 = W.rng(0, 12, 0)
    host8 = [(s, W.params(n, s, gen8), W.grads(n, "normal", s, gen8))
             for s, n in (("bf16", 5000), ("fp32", 4096 + 37), ("fp16", 70000))]

    def state8(s, p, g):
        sizes = ou.state8_sizes(kind, p.size)
        return (H.to_dev(p, s), H.to_dev(g, s), torch.zeros(sizes[0], dtype=torch.uint8, device="cuda"),
                torch.zeros(sizes[1], dtype=torch.uint8, device="cuda"), torch.zeros(sizes[2], device="cuda"),
                torch.zeros(sizes[3], device="cuda"))

    def build():
        a = _device(kind, host)
        b = _device(kind, host_b)
        c = [state8(*x) for x in host8]
        return a, b, c, ou.Plan(kind, a), ou.Plan(kind, b, decay_after=True), ou.Plan8(kind, c)

    ref = build()
    got = build()
    graph = ou.Graph([got[3], got[4]], [got[5]])
    steps = 4
    for t in range(1, steps + 1):
        ref[3].step(hp, t)
        ref[4].step(hp, t)
        ref[5].step(hp, t)
        graph.step(hp, t)
        if t == 2:              # eager work and a synchronisation between replays
            torch.cuda.synchronize()
            _ = (got[0][0][0].float() * 3).sum().item()
    torch.cuda.synchronize()
    graph.close()
    for r, x in zip(ref[:3], got[:3]):
        for tr, tx in zip(r, x):
            for u, v in zip(tr, tx):
                assert u.dtype == v.dtype
                assert u.cpu().view(torch.uint8).numpy().tobytes() == v.cpu().view(torch.uint8).numpy().tobytes()
    for p in ref[3:] + got[3:]:
        p.close()


def test_direct_ops_name_the_bad_operand():
    """The binding's checks of the direct ops: each kind of bad operand is
    refused with a ValueError naming it, before anything is launched, and a
    good call afterwards still updates."""
    import optimizer_update_amd as ou
    n = 1000
    p, g, m, v = (torch.zeros(n, device="cuda") for _ in range(4))
    g.fill_(1e-3)

    def call(*ts, kind="adam"):
        ou.optimizer_update_32bit(kind, *ts, step=1, lr=1e-3)

    strided = torch.zeros(2 * n, device="cuda")[::2]
    cases = [((p, g, m.cpu(), v), "adam", "state1 must be a tensor on a HIP device"),
             ((p, g, 1.0, v), "adam", "state1 must be a tensor on a HIP device"),
             ((p, strided, m, v), "adam", "grad must be contiguous"),
             ((p, g, m, strided), "adam", "state2 must be contiguous"),
             ((p, g, m, v), "lion", "one-state kinds take state2=None"),
             ((p, g.bfloat16(), m, v), "adam", "param and grad must share"),
             ((p.double(), g.double(), m, v), "adam", "param and grad must share"),
             ((p, g, m.double(), v), "adam", "states must be float32"),
             ((p, g, m[:-1], v), "adam", "sizes"),
             ((p, g, m, v), "ademamix", "sizes"),
             ((p, g[:-1], m, v), "adam", "sizes")]
    for ts, kind, msg in cases:
        with pytest.raises(ValueError, match=msg):
            call(*ts, kind=kind)
    torch.cuda.synchronize()
    assert p.abs().sum().item() == 0            # nothing ran
    call(p, g, m, v)
    torch.cuda.synchronize()
    assert (p < 0).all().item()                 # the good call stepped against g > 0

    sizes = ou.state8_sizes("adam", n)
    c1, c2 = (torch.zeros(s, dtype=torch.uint8, device="cuda") for s in sizes[:2])
    a1, a2 = (torch.zeros(s, device="cuda") for s in sizes[2:])

    def call8(*ts):
        ou.optimizer_update_8bit_blockwise("adam", *ts, step=1, lr=1e-3)

    cases8 = [((p, g, c1, c2, a1.cpu(), a2), "absmax1 must be a tensor on a HIP device"),
              ((p, g, c1, c2, a1, None), "absmax2 must be a tensor on a HIP device"),
              ((p, g, c1, torch.zeros(2 * n, dtype=torch.uint8, device="cuda")[::2], a1, a2),
               "state2 must be contiguous"),
              ((p, g, c1.float(), c2, a1, a2), "8-bit states must be uint8"),
              ((p, g, c1, c2, a1.double(), a2), "absmax buffers must be float32"),
              ((p, g, c1[:-1], c2, a1, a2), "sizes")]
    for ts, msg in cases8:
        with pytest.raises(ValueError, match=msg):
            call8(*ts)
    before = p.clone()
    call8(p, g, c1, c2, a1, a2)
    torch.cuda.synchronize()
    assert (p < before).all().item()
