"""GPU parity of the decay-after-update order (kind | OU_DECAY_AFTER).

The page "Investigate a 256-thread SM103 path for small 32-bit optimizer
tensors" (section "Scope") says the order of the decoupled decay and the step
differs between versions of the update.  The default decays the old
parameter, p*d - lr*u; with the flag the updated parameter is decayed,
(p - lr*u)*d.  These tests run the flagged kinds (Adam, AdEMAMix, Lion) on
every storage type through the single-tensor entry, a plan and its graph
replay, forced launch variants and update-norm clipping, and compare each
with the oracle's flagged path: bitwise, except the clip factor, which may
differ by 1 ulp for the reason given in the clipping tests.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

KIND = {"adam": O.ADAM, "ademamix": O.ADEMAMIX, "lion": O.LION}
FLAG = 0x100
SIZES = (1, 33, 1023, 4097, 65539)
T = 6


@pytest.fixture(scope="module")
def orc():
    return O.load()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return H.lib()


def _hp(kind: str, wd: float, skip: bool) -> O.HParams:
    if kind == "lion":
        return O.HParams(lr=1e-3, beta1=0.9, beta2=0.99, eps=0.0, weight_decay=wd, skip_zeros=skip)
    return O.HParams(lr=1e-2, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8,
                     weight_decay=wd, skip_zeros=skip)


def _states(kind: str, n: int):
    k = 2 if kind == "ademamix" else 1
    s1 = torch.zeros(k * n, device="cuda")
    s2 = torch.zeros(n, device="cuda") if kind != "lion" else None
    return s1, s2


def _raw(L, kind, storage, P, G, S1, S2, n, hp, t, flag=FLAG):
    return L.optimizer_update_32bit(KIND[kind] | flag, H.DT[storage], P.data_ptr(), G.data_ptr(),
                                    S1.data_ptr(), None if S2 is None else S2.data_ptr(), n,
                                    hp.beta1, hp.beta2, hp.beta3, hp.alpha, hp.eps,
                                    hp.weight_decay, t, hp.lr, int(hp.skip_zeros),
                                    H.stream_handle())


def _oracle(orc, kind, storage, p0, gsteps, hp, flag=FLAG):
    n = p0.size
    p = p0.copy()
    if kind == "lion":
        s1 = np.zeros(n, np.float32)
        for t, g in enumerate(gsteps, start=1):
            orc.update1_f32(O.LION | flag, H.DT[storage], p, g.copy(), s1, hp, t)
        return p, s1, None
    s1, s2 = W.zero_states(n, kind)
    for t, g in enumerate(gsteps, start=1):
        orc.update_f32(KIND[kind] | flag, H.DT[storage], p, g.copy(), s1, s2, hp, t)
    return p, s1, s2


def _inputs(storage: str, n: int, seed: int):
    gen = W.rng(2, seed, n)
    p0 = W.params(n, storage, gen)
    gsteps = [W.cast_storage(np.where(gen.random(n) < 0.1, 0.0, gen.standard_normal(n)), storage)
              for _ in range(T)]
    return p0, gsteps


def _direct(L, kind, storage, p0, gsteps, hp, flag=FLAG, force=None):
    n = p0.size
    P, G = H.to_dev(p0, storage), torch.empty(n, dtype=W.STORAGE_TORCH[storage], device="cuda")
    S1, S2 = _states(kind, n)
    if force:
        L.ou__force_single(*force)
    try:
        for t, g in enumerate(gsteps, start=1):
            G.copy_(W.to_torch(g, storage, "cuda"))
            st = _raw(L, kind, storage, P, G, S1, S2, n, hp, t, flag)
            assert st == 0, H.last_error(L)
    finally:
        L.ou__force_single(0, 0, 0, 0, 0, 0)
    torch.cuda.synchronize()
    return W.from_torch(P), W.from_torch(S1), None if S2 is None else W.from_torch(S2)


@pytest.mark.parametrize("kind", list(KIND))
@pytest.mark.parametrize("storage", ["fp32", "fp16", "bf16"])
def test_decay_after_matches_oracle(orc, L, kind, storage):
    """Direct calls, 6 steps, wd > 0 with skip_zeros off and on: bitwise
    equal to the oracle's flagged path, and different from the default
    order (the flag reaches the kernel)."""
    wd = 0.1 if kind == "lion" else 0.05
    for skip in (False, True):
        hp = _hp(kind, wd, skip)
        for n in SIZES:
            p0, gsteps = _inputs(storage, n, 1)
            got = _direct(L, kind, storage, p0, gsteps, hp)
            ref = _oracle(orc, kind, storage, p0, gsteps, hp)
            what = f"{kind} {storage} skip={skip} n={n}"
            H.assert_parity(got[0], ref[0], storage, "p " + what)
            H.assert_parity(got[1], ref[1], "fp32", "state1 " + what)
            if ref[2] is not None:
                H.assert_parity(got[2], ref[2], "fp32", "state2 " + what)
            if n >= 1023 and storage == "fp32":
                # the orders differ by lr^2 wd |u| per step (1e-7 .. 5e-6 here):
                # visible in binary32, below the ulp of the 16-bit types
                default = _oracle(orc, kind, storage, p0, gsteps, hp, flag=0)
                assert default[0].tobytes() != got[0].tobytes(), what


@pytest.mark.parametrize("kind", list(KIND))
def test_decay_after_with_zero_decay_is_the_default(L, kind):
    """wd = 0 makes d = 1 exactly: both orders give the same bits."""
    hp = _hp(kind, 0.0, False)
    p0, gsteps = _inputs("bf16", 4097, 2)
    a = _direct(L, kind, "bf16", p0, gsteps, hp, flag=FLAG)
    b = _direct(L, kind, "bf16", p0, gsteps, hp, flag=0)
    for x, y in zip(a, b):
        assert (x is None and y is None) or x.tobytes() == y.tobytes()


@pytest.mark.parametrize("kind", list(KIND))
def test_decay_after_launch_variants_plan_and_graph(orc, L, kind):
    """Forced single-tensor shapes, a plan of several tensors and its graph
    replay give the bits of the direct call."""
    from optimizer_update_amd import Plan
    storage = "fp32"
    hp = _hp(kind, 0.1, True)
    variants = [(64, 4, 1, 0, 0, 0), (1024, 4, 4, 0, 0, 0), (256, 4, 2, 0, 1, 0),
                (256, 4, 2, 0, 0, -1)]
    if kind != "lion":
        variants.append((256, 8, 2, 0, 0, 0))
    base = {}
    for n in SIZES:
        p0, gsteps = _inputs(storage, n, 3)
        base[n] = (p0, gsteps, _direct(L, kind, storage, p0, gsteps, hp))
        for v in variants:
            got = _direct(L, kind, storage, p0, gsteps, hp, force=v)
            for x, y in zip(got, base[n][2]):
                assert (x is None and y is None) or x.tobytes() == y.tobytes(), (v, n)
    for graph in (False, True):
        tensors = {}
        for n in SIZES:
            s1, s2 = _states(kind, n)
            tensors[n] = (H.to_dev(base[n][0], storage),
                          torch.empty(n, dtype=torch.float32, device="cuda"), s1, s2)
        plan = Plan(kind, [tensors[n] for n in SIZES], decay_after=True)
        try:
            for t in range(1, T + 1):
                for n in SIZES:
                    tensors[n][1].copy_(W.to_torch(base[n][1][t - 1], storage, "cuda"))
                (plan.graph_step if graph else plan.step)(H.pkg_hp(hp), t)
            torch.cuda.synchronize()
        finally:
            plan.close()
        for n in SIZES:
            ref = base[n][2]
            assert W.from_torch(tensors[n][0]).tobytes() == ref[0].tobytes(), (graph, n)
            assert W.from_torch(tensors[n][2]).tobytes() == ref[1].tobytes(), (graph, n)


@pytest.mark.parametrize("kind", ["adam", "ademamix"])
@pytest.mark.parametrize("storage", ["fp32", "bf16"])
def test_decay_after_with_clipping(orc, kind, storage):
    """Update-norm clipping with the flag: moments bitwise, clip factor
    within 1 ulp, parameters within the parity tolerance of the oracle's
    flagged clipped step; the plan's per-tensor clip gives the single
    entry's bits."""
    import optimizer_update_amd as ou
    hp = _hp(kind, 0.5, True)
    for n in (33, 4097, 65539):
        p0, gsteps = _inputs(storage, n, 4)
        for bound in (0.05, 1e6):
            P = H.to_dev(p0, storage)
            G = torch.empty(n, dtype=W.STORAGE_TORCH[storage], device="cuda")
            S1, S2 = _states(kind, n)
            ws = ou.clip_workspace(n, "cuda")
            pr = p0.copy()
            s1r, s2r = W.zero_states(n, kind)
            for t, g in enumerate(gsteps, start=1):
                G.copy_(W.to_torch(g, storage, "cuda"))
                ou.optimizer_update_32bit_clip(kind, P, G, S1, S2, step=t, lr=hp.lr, beta1=hp.beta1,
                                               beta2=hp.beta2, beta3=hp.beta3, alpha=hp.alpha,
                                               eps=hp.eps, weight_decay=hp.weight_decay,
                                               skip_zeros=hp.skip_zeros, max_unorm=bound,
                                               workspace=ws, decay_after=True)
                s_gpu = ou.clip_scale(ws)
                s_ref = orc.update_f32_clip(KIND[kind] | FLAG, H.DT[storage], pr, g.copy(), s1r,
                                            s2r, hp, t, bound)
                ia = int(np.float32(s_gpu).view(np.int32))
                ib = int(np.float32(s_ref).view(np.int32))
                assert abs(ia - ib) <= 1, (kind, storage, n, bound, t, s_gpu, s_ref)
            torch.cuda.synchronize()
            what = f"{kind} {storage} n={n} bound={bound}"
            H.assert_parity(W.from_torch(P), pr, storage, "p " + what, bitwise=False)
            H.assert_parity(W.from_torch(S1), s1r, "fp32", "state1 " + what)
            H.assert_parity(W.from_torch(S2), s2r, "fp32", "state2 " + what)


@pytest.mark.parametrize("cls,kw", [("AdamW32", dict(lr=1e-2, weight_decay=0.1)),
                                    ("AdEMAMix32", dict(lr=1e-2, weight_decay=0.1)),
                                    ("Lion32", dict(lr=1e-3, weight_decay=0.5))])
def test_decay_after_collections(orc, cls, kw):
    """Collection classes with decay_after=True: plan, graph and per-tensor
    steps agree bitwise and match the oracle."""
    import optimizer_update_amd as ou
    shapes = [(1024,), (33,), (16, 1024), (4097,)]
    rows = [(W.params(W.numel(s), "bf16", W.rng(2, 7, i)),
             W.grads(W.numel(s), "normal", "bf16", W.rng(2, 8, i))) for i, s in enumerate(shapes)]
    runs = {}
    for mode in ("plan", "graph", "per_tensor"):
        ps = [H.to_dev(p0, "bf16") for p0, _ in rows]
        gs = [H.to_dev(g, "bf16") for _, g in rows]
        opt = getattr(ou, cls)(ps, grads=gs, decay_after=True, **kw)
        for _ in range(3):
            if mode == "per_tensor":
                opt.step_per_tensor()
            else:
                opt.step(graph=(mode == "graph"))
        torch.cuda.synchronize()
        runs[mode] = [W.from_torch(p) for p in ps] + [W.from_torch(s) for s in opt.state1]
        hp = O.HParams(**{k: getattr(opt.hp, k) for k in ("lr", "beta1", "beta2", "beta3", "alpha",
                                                          "eps", "weight_decay", "skip_zeros")})
        kind = ou.optim.__dict__[cls].kind
        opt.close()
    for mode in ("graph", "per_tensor"):
        for a, b in zip(runs["plan"], runs[mode]):
            assert a.tobytes() == b.tobytes(), (cls, mode)
    for i, (p0, g) in enumerate(rows):
        ref = _oracle(orc, kind, "bf16", p0, [g] * 3, hp)
        H.assert_parity(runs["plan"][i], ref[0], "bf16", f"{cls} p {i}")
        H.assert_parity(runs["plan"][len(rows) + i][:ref[1].size], ref[1], "fp32", f"{cls} m {i}")
