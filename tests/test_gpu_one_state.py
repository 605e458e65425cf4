"""GPU parity of the one-state kinds (momentum SGD, RMSprop, Adagrad, Lion)
against the CPU oracle, through the C ABI.

These are the other members of the 32-bit update family that the page
"Investigate a 256-thread SM103 path for small 32-bit optimizer tensors"
keeps apart from its two-state kinds.  The coverage mirrors the two-state
tests: every storage type, zero and nonzero weight decay, skip_zeros off and
on, zero/normal/mixed-magnitude gradients, the tensor sizes of the coverage
matrix, launch variants and graph replay, a large tensor checked on sampled
elements.  The kernels perform the oracle's operation sequence, so results
must be bit-identical; the tolerance of the comparison rule is checked too.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

KINDS = {"momentum": O.MOMENTUM, "rmsprop": O.RMSPROP, "adagrad": O.ADAGRAD, "lion": O.LION}
STORAGES = ("fp32", "fp16", "bf16")
SNAP = (1, 2, 10)


@pytest.fixture(scope="module")
def orc():
    return O.load()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return H.lib()


def _hp(kind: str, wd: bool, skip: bool) -> O.HParams:
    """Usual settings of each kind; the L2 coefficient of momentum/RMSprop/
    Adagrad and Lion's decoupled coefficient when wd is on."""
    if kind == "lion":
        return O.HParams(lr=1e-4, beta1=0.9, beta2=0.99, eps=0.0,
                         weight_decay=0.1 if wd else 0.0, skip_zeros=skip)
    if kind == "momentum":
        return O.HParams(lr=1e-2, beta1=0.9, beta2=0.0, eps=0.0,
                         weight_decay=0.01 if wd else 0.0, skip_zeros=skip)
    if kind == "rmsprop":
        return O.HParams(lr=1e-2, beta1=0.99, beta2=0.0, eps=1e-8,
                         weight_decay=0.01 if wd else 0.0, skip_zeros=skip)
    return O.HParams(lr=1e-2, beta1=0.0, beta2=0.0, eps=1e-10,
                     weight_decay=0.01 if wd else 0.0, skip_zeros=skip)


def _raw1(L, kind: str, storage: str, p: torch.Tensor, g: torch.Tensor, s1: torch.Tensor, n: int,
          hp: O.HParams, step: int, state2=None) -> int:
    """optimizer_update_32bit for a one-state kind (state2 NULL unless given)."""
    return L.optimizer_update_32bit(KINDS[kind], H.DT[storage], p.data_ptr(), g.data_ptr(),
                                    s1.data_ptr(), state2, n, hp.beta1, hp.beta2, hp.beta3,
                                    hp.alpha, hp.eps, hp.weight_decay, step, hp.lr,
                                    int(hp.skip_zeros), H.stream_handle())


SWEEP = [(n, pat) for n in W.SWEEP_N for pat in W.GRAD_PATTERNS]


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("storage", STORAGES)
def test_sweep_direct_and_plan(orc, L, kind, storage):
    """Every (size, gradient pattern) of the coverage matrix as one
    collection, 10 steps, direct per-tensor calls and one plan, both against
    the oracle at steps 1, 2 and 10, for wd off/on and skip_zeros off/on."""
    from optimizer_update_amd import Plan
    sizes = [n for n, _ in SWEEP]
    offs, total = H.padded_offsets(sizes)
    T = max(SNAP)
    for wd in (False, True):
        for skip in (False, True):
            hp = _hp(kind, wd, skip)
            key = (list(KINDS).index(kind), STORAGES.index(storage), int(wd), int(skip))
            P0 = np.zeros(total, W.STORAGE_NP[storage])
            G = np.zeros((T, total), W.STORAGE_NP[storage])
            for i, ((n, pat), o) in enumerate(zip(SWEEP, offs)):
                P0[o:o + n] = W.params(n, storage, W.rng(1, 1, *key, i))
                for t in range(T):
                    G[t, o:o + n] = W.grads(n, pat, storage, W.rng(1, 2, *key, i, t))
            refs = [(P0[o:o + n].copy(), np.zeros(n, np.float32)) for (n, _), o in zip(SWEEP, offs)]
            bufs = {}
            for path in ("direct", "plan"):
                bufs[path] = (H.to_dev(P0, storage), torch.zeros(total, device="cuda"))
            g_dev = H.to_dev(G[0], storage)
            segs = [(bufs["plan"][0][o:o + n], g_dev[o:o + n], bufs["plan"][1][o:o + n], None)
                    for (n, _), o in zip(SWEEP, offs)]
            plan = Plan(kind, segs)
            try:
                for t in range(1, T + 1):
                    g_dev.copy_(W.to_torch(G[t - 1], storage, device="cuda"))
                    pd, sd = bufs["direct"]
                    for (n, _), o in zip(SWEEP, offs):
                        st = _raw1(L, kind, storage, pd[o:o + n], g_dev[o:o + n], sd[o:o + n], n,
                                   hp, t)
                        assert st == 0, H.last_error(L)
                    plan.step(H.pkg_hp(hp), t)
                    for (n, _), o, r in zip(SWEEP, offs, refs):
                        orc.update1_f32(KINDS[kind], H.DT[storage], r[0], G[t - 1, o:o + n].copy(),
                                        r[1], hp, t)
                    if t in SNAP:
                        torch.cuda.synchronize()
                        got = {k: tuple(W.from_torch(b) for b in v) for k, v in bufs.items()}
                        for (n, pat), o, r in zip(SWEEP, offs, refs):
                            what = f"{kind} {storage} wd={wd} skip={skip} n={n} {pat} step {t}"
                            H.assert_parity(got["plan"][0][o:o + n], r[0], storage, "p " + what)
                            H.assert_parity(got["plan"][1][o:o + n], r[1], "fp32", "m " + what)
                        for a, b in zip(got["plan"], got["direct"]):
                            assert a.tobytes() == b.tobytes(), f"direct != plan at step {t}"
                assert W.from_torch(g_dev).tobytes() == G[T - 1].tobytes(), "grad changed"
            finally:
                plan.close()


VARIANT_N = (1, 33, 1023, 4097, 65539, (1 << 20) + 5)
# (block, elements per lane, unroll, grid, per-lane path, LDS cap); the
# one-state kinds are built with 4 elements per lane only.
SINGLE_VARIANTS = [(64, 4, 1, 0, 0, 0), (1024, 4, 4, 0, 0, 0), (512, 4, 2, 1, 0, 0),
                   (128, 4, 4, 3, 0, 0), (256, 4, 2, 0, 1, 0), (256, 4, 2, 0, 0, -1),
                   (256, 4, 2, 0, 0, 65536)]
MULTI_SHAPES = [(0, 0, 0, 0, 0), (1, 4, 1, 256 * 4 * 2, 0), (2, 4, 2, 4096, 65536),
                (4, 4, 2, 1024, -1), (8, 4, 4, 512 * 4, 0)]


def _inputs(n: int, storage: str):
    gen = W.rng(1, 6, n)
    p0 = W.params(n, storage, gen)
    g = W.cast_storage(np.where(gen.random(n) < 0.1, 0.0, gen.standard_normal(n)), storage)
    return p0, g


def _run(L, kind, storage, p0, g_host, T, hp, force=None, offset=0):
    n = p0.size
    P = H.to_dev(np.concatenate([np.zeros(offset, p0.dtype), p0]), storage)[offset:]
    G = H.to_dev(np.concatenate([np.zeros(offset, g_host.dtype), g_host]), storage)[offset:]
    S1 = torch.zeros(n + offset, device="cuda")[offset:]
    if force:
        L.ou__force_single(*force)
    try:
        for t in range(1, T + 1):
            st = _raw1(L, kind, storage, P, G, S1, n, hp, t)
            assert st == 0, H.last_error(L)
    finally:
        L.ou__force_single(0, 0, 0, 0, 0, 0)
    torch.cuda.synchronize()
    return W.from_torch(P), W.from_torch(S1), W.from_torch(G)


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("storage", ("fp32", "bf16"))
def test_launch_variants_bitwise(orc, L, kind, storage):
    """Block widths, unrolls, grids, the per-lane path, the LDS cap,
    misaligned starts, the multi-tensor walk in several shapes and orders,
    and graph replay all give the oracle's bits."""
    from optimizer_update_amd import Plan
    T = 3
    hp = _hp(kind, True, True)
    base = {}
    for n in VARIANT_N:
        p0, g_host = _inputs(n, storage)
        out = _run(L, kind, storage, p0, g_host, T, hp)
        base[n] = (p0, g_host, out)
        assert out[2].tobytes() == g_host.tobytes(), "grad changed"
        idx = np.arange(n) if n < 70000 else np.unique(np.r_[0:4096, n - 4096:n, 0:n:4099])
        p_ref, m_ref = p0[idx].copy(), np.zeros(idx.size, np.float32)
        for t in range(1, T + 1):
            orc.update1_f32(KINDS[kind], H.DT[storage], p_ref, g_host[idx].copy(), m_ref, hp, t)
        H.assert_parity(out[0][idx], p_ref, storage, f"p n={n}")
        H.assert_parity(out[1][idx], m_ref, "fp32", f"m n={n}")
        for v in SINGLE_VARIANTS:
            o = _run(L, kind, storage, p0, g_host, T, hp, force=v)
            assert o[0].tobytes() == out[0].tobytes() and o[1].tobytes() == out[1].tobytes(), \
                f"variant {v} differs at n={n}"
        for off in (1, 3):
            o = _run(L, kind, storage, p0, g_host, T, hp, offset=off)
            assert o[0].tobytes() == out[0].tobytes() and o[1].tobytes() == out[1].tobytes(), \
                f"offset {off} differs at n={n}"
    sizes = list(VARIANT_N)
    for shape in MULTI_SHAPES:
        for order in (sizes, sizes[::-1]):
            for graph in (False, True):
                L.ou__force_multi(*shape)
                try:
                    tensors = {n: (H.to_dev(base[n][0], storage), H.to_dev(base[n][1], storage),
                                   torch.zeros(n, device="cuda")) for n in order}
                    plan = Plan(kind, [(*tensors[n], None) for n in order])
                finally:
                    L.ou__force_multi(0, 0, 0, 0, 0)
                try:
                    for t in range(1, T + 1):
                        (plan.graph_step if graph else plan.step)(H.pkg_hp(hp), t)
                    torch.cuda.synchronize()
                finally:
                    plan.close()
                for n in order:
                    ref = base[n][2]
                    assert W.from_torch(tensors[n][0]).tobytes() == ref[0].tobytes(), \
                        f"multi {shape} graph={graph} p differs at n={n}"
                    assert W.from_torch(tensors[n][2]).tobytes() == ref[1].tobytes(), \
                        f"multi {shape} graph={graph} m differs at n={n}"


@pytest.mark.parametrize("kind", list(KINDS))
def test_eight_per_lane_is_rejected(L, kind):
    """The one-state kernels exist with 4 elements per lane only: forcing 8
    is refused before any launch."""
    n = 4096
    p = torch.zeros(n, device="cuda")
    g = torch.zeros(n, device="cuda")
    m = torch.zeros(n, device="cuda")
    L.ou__force_single(256, 8, 2, 0, 0, 0)
    try:
        st = _raw1(L, kind, "fp32", p, g, m, n, _hp(kind, False, False), 1)
    finally:
        L.ou__force_single(0, 0, 0, 0, 0, 0)
    assert st == -1
    torch.cuda.synchronize()
    assert not p.any() and not m.any()


@pytest.mark.parametrize("kind", list(KINDS))
def test_state2_is_never_touched(orc, L, kind):
    """A state2 pointer given to a one-state kind is ignored: a sentinel
    buffer passed there, even one overlapping nothing else, is left as is,
    and the result equals the NULL-state2 call."""
    n = 10007
    p0, g_host = _inputs(n, "fp32")
    hp = _hp(kind, True, False)
    ref = _run(L, kind, "fp32", p0, g_host, 2, hp)
    P, G = H.to_dev(p0, "fp32"), H.to_dev(g_host, "fp32")
    M = torch.zeros(n, device="cuda")
    sentinel = torch.full((n,), 12345.0, device="cuda")
    for t in (1, 2):
        st = _raw1(L, kind, "fp32", P, G, M, n, hp, t, state2=sentinel.data_ptr())
        assert st == 0, H.last_error(L)
    torch.cuda.synchronize()
    assert bool((sentinel == 12345.0).all())
    assert W.from_torch(P).tobytes() == ref[0].tobytes()
    assert W.from_torch(M).tobytes() == ref[1].tobytes()


@pytest.mark.parametrize("kind,storage", [("lion", "fp32"), ("momentum", "bf16"),
                                          ("rmsprop", "fp16"), ("adagrad", "fp32")])
def test_large_tensor_sampled(orc, L, kind, storage):
    """2^26 + 3 elements in the bench's launch configuration, 3 steps,
    checked on sampled elements (head, tail, a stride) against the oracle."""
    n = (1 << 26) + 3
    gen = W.rng(1, 9, n)
    p0 = W.params(n, storage, gen)
    g_host = W.grads(n, "normal", storage, W.rng(1, 10, n))
    hp = _hp(kind, True, False)
    P, G = H.to_dev(p0, storage), H.to_dev(g_host, storage)
    M = torch.zeros(n, device="cuda")
    for t in (1, 2, 3):
        st = _raw1(L, kind, storage, P, G, M, n, hp, t)
        assert st == 0, H.last_error(L)
    torch.cuda.synchronize()
    idx = np.unique(np.r_[0:8192, n - 8192:n, 0:n:65537])
    p_ref, m_ref = p0[idx].copy(), np.zeros(idx.size, np.float32)
    for t in (1, 2, 3):
        orc.update1_f32(KINDS[kind], H.DT[storage], p_ref, g_host[idx].copy(), m_ref, hp, t)
    it = torch.from_numpy(idx).cuda()
    H.assert_parity(W.from_torch(P[it]), p_ref, storage, f"p {kind} {storage}")
    H.assert_parity(W.from_torch(M[it]), m_ref, "fp32", f"m {kind} {storage}")
    del P, G, M
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cls,kw", [("Momentum32", dict(lr=1e-2, momentum=0.9, weight_decay=1e-2)),
                                    ("RMSprop32", dict(lr=1e-3, alpha=0.99, eps=1e-8)),
                                    ("Adagrad32", dict(lr=1e-2, eps=1e-10, weight_decay=1e-3)),
                                    ("Lion32", dict(lr=1e-4, betas=(0.9, 0.99), weight_decay=0.1))])
def test_collection_optimizers(orc, L, cls, kw):
    """The collection classes: plan step, graph replay and per-tensor calls
    agree bitwise, match the oracle, and round-trip through state_dict."""
    import optimizer_update_amd as ou
    shapes = [(1024,), (16, 1024), (4097,), (33,), (512, 129)]
    rows = []
    for i, s in enumerate(shapes):
        n = W.numel(s)
        p0 = W.params(n, "bf16", W.rng(1, 11, i))
        g = W.grads(n, "mixed", "bf16", W.rng(1, 12, i))
        rows.append((p0, g))
    runs = {}
    for mode in ("plan", "graph", "per_tensor"):
        ps = [H.to_dev(p0, "bf16") for p0, _ in rows]
        gs = [H.to_dev(g, "bf16") for _, g in rows]
        opt = getattr(ou, cls)(ps, grads=gs, **kw)
        assert all(s is None for s in opt.state2)
        for _ in range(4):
            if mode == "per_tensor":
                opt.step_per_tensor()
            else:
                opt.step(graph=(mode == "graph"))
        torch.cuda.synchronize()
        runs[mode] = ([W.from_torch(p) for p in ps], [W.from_torch(s) for s in opt.state1])
        if mode == "plan":
            sd = opt.state_dict()
            ps2 = [H.to_dev(W.from_torch(p), "bf16") for p in ps]
            opt2 = getattr(ou, cls)(ps2, grads=gs, **kw)
            opt2.load_state_dict(sd)
            opt.step()
            opt2.step()
            torch.cuda.synchronize()
            for a, b in zip(ps, ps2):
                assert W.from_torch(a).tobytes() == W.from_torch(b).tobytes()
            opt2.close()
        opt.close()
    for mode in ("graph", "per_tensor"):
        for a, b in zip(runs["plan"][0] + runs["plan"][1], runs[mode][0] + runs[mode][1]):
            assert a.tobytes() == b.tobytes(), f"{cls}: {mode} differs from plan"
    opt_h = getattr(ou, cls)([torch.zeros(8, device="cuda")], grads=[torch.zeros(8, device="cuda")], **kw)
    hp = O.HParams(**{k: getattr(opt_h.hp, k) for k in ("lr", "beta1", "beta2", "beta3", "alpha",
                                                         "eps", "weight_decay", "skip_zeros")})
    opt_h.close()
    kind = KINDS[ou.optim.__dict__[cls].kind]
    for (p0, g), p_got, m_got in zip(rows, runs["plan"][0], runs["plan"][1]):
        p_ref, m_ref = p0.copy(), np.zeros(p0.size, np.float32)
        for t in range(1, 5):
            orc.update1_f32(kind, O.BF16, p_ref, g.copy(), m_ref, hp, t)
        H.assert_parity(p_got, p_ref, "bf16", cls + " p")
        H.assert_parity(m_got, m_ref, "fp32", cls + " m")
    z = torch.zeros(8, device="cuda")
    with pytest.raises(ou.OptimizerUpdateError):    # clipping: two-state kinds only
        ou.optimizer_update_32bit_clip(ou.optim.__dict__[cls].kind, z, z.clone(), z.clone(), None,
                                       step=1, lr=1e-3, max_unorm=1.0)
