"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Coverage follows the page "Investigate a 256-thread SM103 path for small
32-bit optimizer tensors" (bitsandbytes fork, issue 8), section "Correctness
oracle": both kinds, fp32/fp16/bf16 storage, steps 1, 2, 10 and 1000, zero
and nonzero weight decay, skip_zeros off/on, zero, random and
mixed-magnitude gradients, n over the listed sizes and boundary controls;
the gradient must stay unchanged; launch variants must agree bitwise.

Tolerance (per element): fp32 values within 2e-6 relative, fp16/bf16
parameters within 1 ulp of the storage type.  The kernels perform the
oracle's operation sequence with correctly rounded operations, so the tests
also require bit-identical results.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

KINDS = ("adam", "ademamix")
STORAGES = ("fp32", "fp16", "bf16")


@pytest.fixture(scope="module")
def orc():
    return O.load()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return H.lib()


def _hp(kind: str, wd: float, skip: bool) -> O.HParams:
    return O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8,
                     weight_decay=wd, skip_zeros=skip)


# ------------------------------------------------------------------ config 1

def test_single_fp32_adam_n1024(orc, L):
    """fp32 Adam, n = 1024, grads N(0, 0.01^2) redrawn every step, 10 steps,
    compared after every step."""
    n, T = 1024, 10
    hp = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)
    p0 = W.params(n, "fp32", W.rng(0, 1, 0))
    p_ref, (s1_ref, s2_ref) = p0.copy(), W.zero_states(n, "adam")
    p, g = H.to_dev(p0, "fp32"), torch.empty(n, device="cuda")
    s1, s2 = torch.zeros(n, device="cuda"), torch.zeros(n, device="cuda")
    for t in range(1, T + 1):
        gt = W.grads(n, "normal", "fp32", W.rng(0, 1, t), sigma=0.01)
        g.copy_(torch.from_numpy(gt))
        st = H.raw_update(L, "adam", "fp32", p, g, s1, s2, n, hp, t, H.stream_handle())
        assert st == 0, H.last_error(L)
        orc.update_f32(O.ADAM, O.F32, p_ref, gt, s1_ref, s2_ref, hp, t)
        torch.cuda.synchronize()
        H.assert_parity(W.from_torch(p), p_ref, "fp32", f"p step {t}")
        H.assert_parity(W.from_torch(s1), s1_ref, "fp32", f"m step {t}")
        H.assert_parity(W.from_torch(s2), s2_ref, "fp32", f"v step {t}")
        assert W.from_torch(g).tobytes() == gt.tobytes(), "grad changed"


# ------------------------------------------------------------- configs 2 + 3

SWEEP = [(n, pat) for n in W.SWEEP_N for pat in W.GRAD_PATTERNS]


def _sweep_grads(storage: str, T: int, offs: list[int], total: int) -> np.ndarray:
    """[T, total] gradients, redrawn per step, each segment with its pattern."""
    out = np.zeros((T, total), W.STORAGE_NP[storage])
    for t in range(1, T + 1):
        g = W.rng(0, 2, W.STORAGE_BYTES[storage], t)
        row = np.zeros(total, np.float32)
        for (n, pat), o in zip(SWEEP, offs):
            row[o:o + n] = W.grads_f32(n, pat, g)
        out[t - 1] = W.cast_storage(row, storage)
    return out


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("storage", STORAGES)
def test_sweep_1000_steps(orc, L, kind, storage):
    """Every n of the coverage matrix x {zero, normal, mixed} gradients, as one
    collection, 1000 steps, for wd in {0, 0.01} x skip_zeros in {off, on}.
    Three paths run side by side on the same inputs: the oracle, one direct
    call per tensor, and the plan (one multi-tensor launch).  At steps 1, 2,
    10 and 1000 the plan matches the oracle and the direct calls match the
    plan bitwise."""
    T = 1000
    sizes = [n for n, _ in SWEEP]
    offs, total = H.padded_offsets(sizes)
    k = 2 if kind == "ademamix" else 1
    offs1, total1 = H.padded_offsets([k * n for n in sizes])
    G_host = _sweep_grads(storage, T, offs, total)
    G_all = H.to_dev(G_host.reshape(-1), storage).view(T, total)
    g_buf = torch.empty(total, dtype=W.STORAGE_TORCH[storage], device="cuda")
    p0_row = np.zeros(total, np.float32)
    gp = W.rng(0, 2, W.STORAGE_BYTES[storage], 0)
    for (n, _), o in zip(SWEEP, offs):
        p0_row[o:o + n] = gp.uniform(-1, 1, n)
    p0 = W.cast_storage(p0_row, storage)
    stream = H.stream_handle()
    for wd in (0.0, 0.01):
        for skip in (False, True):
            hp = _hp(kind, wd, skip)
            bufs = {}
            for path in ("plan", "direct"):
                bufs[path] = (H.to_dev(p0, storage), torch.zeros(total1, device="cuda"),
                              torch.zeros(total, device="cuda"))
            ref = [(p0[o:o + n].copy(), *W.zero_states(n, kind)) for (n, _), o in zip(SWEEP, offs)]

            def segs(path):
                P, S1, S2 = bufs[path]
                return [(P[o:o + n], g_buf[o:o + n], S1[o1:o1 + k * n], S2[o:o + n])
                        for (n, _), o, o1 in zip(SWEEP, offs, offs1)]

            from optimizer_update_amd import Plan
            plan = Plan(kind, segs("plan"))
            direct = [(p.data_ptr(), g.data_ptr(), s1.data_ptr(), s2.data_ptr(), p.numel())
                      for p, g, s1, s2 in segs("direct")]
            php = H.pkg_hp(hp)
            for t in range(1, T + 1):
                g_buf.copy_(G_all[t - 1])
                plan.step(php, t)
                for pp, gg, ss1, ss2, n in direct:
                    st = L.optimizer_update_32bit(H.KIND[kind], H.DT[storage], pp, gg, ss1, ss2, n,
                                                  hp.beta1, hp.beta2, hp.beta3, hp.alpha, hp.eps,
                                                  hp.weight_decay, t, hp.lr, int(skip), stream)
                    assert st == 0, H.last_error(L)
                for (n, _), o, r in zip(SWEEP, offs, ref):
                    orc.update_f32(H.KIND[kind], H.DT[storage], r[0], G_host[t - 1, o:o + n],
                                   r[1], r[2], hp, t, nthreads=1)
                if t in W.SNAPSHOT_STEPS:
                    torch.cuda.synchronize()
                    got = {path: tuple(W.from_torch(b) for b in bufs[path]) for path in bufs}
                    for i, ((n, pat), o, o1) in enumerate(zip(SWEEP, offs, offs1)):
                        what = f"{kind} {storage} wd={wd} skip={skip} n={n} {pat} step {t}"
                        gp_, gs1, gs2 = got["plan"]
                        H.assert_parity(gp_[o:o + n], ref[i][0], storage, "p " + what)
                        H.assert_parity(gs1[o1:o1 + k * n], ref[i][1], "fp32", "state1 " + what)
                        H.assert_parity(gs2[o:o + n], ref[i][2], "fp32", "state2 " + what)
                    for a, b in zip(got["plan"], got["direct"]):
                        assert a.tobytes() == b.tobytes(), f"direct != plan at step {t} ({kind} {storage} wd={wd} skip={skip})"
            assert W.from_torch(g_buf).tobytes() == G_host[T - 1].tobytes(), "grad changed"
            plan.close()


# ---------------------------------------------------------- launch variants

VARIANT_N = (1, 33, 1023, 4097, 65539, (1 << 20) + 5)


def _run_single(L, kind, storage, p0, g_host, T, hp, force=None, offset=0):
    """T steps of the single-tensor entry with an optional forced shape, on
    buffers placed `offset` elements past a 256-byte boundary."""
    n = p0.size
    k = 2 if kind == "ademamix" else 1
    P = H.to_dev(np.concatenate([np.zeros(offset, p0.dtype), p0]), storage)[offset:]
    G = H.to_dev(np.concatenate([np.zeros(offset, g_host.dtype), g_host]), storage)[offset:]
    S1 = torch.zeros(k * n + offset, device="cuda")[offset:]
    S2 = torch.zeros(n + offset, device="cuda")[offset:]
    if force:
        L.ou__force_single(*force)
    try:
        for t in range(1, T + 1):
            st = H.raw_update(L, kind, storage, P, G, S1, S2, n, hp, t, H.stream_handle())
            assert st == 0, H.last_error(L)
    finally:
        L.ou__force_single(0, 0, 0, 0, 0, 0)
    torch.cuda.synchronize()
    return W.from_torch(P), W.from_torch(S1), W.from_torch(S2), W.from_torch(G)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("storage", STORAGES)
def test_launch_variants_bitwise(orc, L, kind, storage):
    """Block width, elements per lane, unroll, grid size, the per-lane path,
    misaligned starts, the multi-tensor walk (waves per block, chunk size,
    position in the collection) and graph replay all give bit-identical
    parameters and states, equal to the oracle."""
    T = 3
    hp = _hp(kind, 0.01, True)
    variants = [(64, 4, 1, 0, 0, 0), (256, 8, 2, 0, 0, 0), (1024, 4, 4, 0, 0, 0),
                (128, 8, 4, 3, 0, 0), (512, 4, 2, 1, 0, 0), (64, 8, 1, 7, 0, 0),
                (256, 4, 2, 0, 1, 0), (1024, 8, 1, 2, 1, 0), (256, 4, 2, 0, 0, -1),
                (256, 4, 2, 0, 0, 65536), (512, 4, 1, 0, 0, 98304),
                (128, 4, 4, 0, 0, 0)]   # the large fp32 Adam shape
    for n in VARIANT_N:
        gen = W.rng(0, 6, n)
        p0 = W.params(n, storage, gen)
        g_host = W.cast_storage(np.where(gen.random(n) < 0.1, 0.0, gen.standard_normal(n)), storage)
        base = _run_single(L, kind, storage, p0, g_host, T, hp)
        assert base[3].tobytes() == g_host.tobytes(), "grad changed"
        # oracle (the large size is sampled: every element is independent)
        idx = np.arange(n) if n < 70000 else np.unique(np.r_[0:4096, n - 4096:n, 0:n:4099])
        p_ref = p0[idx].copy()
        s1_ref, s2_ref = W.zero_states(idx.size, kind)
        for t in range(1, T + 1):
            orc.update_f32(H.KIND[kind], H.DT[storage], p_ref, g_host[idx].copy(), s1_ref, s2_ref, hp, t)
        H.assert_parity(base[0][idx], p_ref, storage, f"p n={n}")
        H.assert_parity(base[2][idx], s2_ref, "fp32", f"v n={n}")
        H.assert_parity(base[1][:n][idx], s1_ref[:idx.size], "fp32", f"m n={n}")
        if kind == "ademamix":
            H.assert_parity(base[1][n:][idx], s1_ref[idx.size:], "fp32", f"m2 n={n}")
        for v in variants:
            out = _run_single(L, kind, storage, p0, g_host, T, hp, force=v)
            for a, b, name in zip(base[:3], out[:3], ("p", "state1", "state2")):
                assert a.tobytes() == b.tobytes(), f"variant {v} differs in {name} at n={n}"
        for off in (1, 2, 3):      # unaligned starts: per-lane path
            out = _run_single(L, kind, storage, p0, g_host, T, hp, offset=off)
            for a, b, name in zip(base[:3], out[:3], ("p", "state1", "state2")):
                assert a.tobytes() == b.tobytes(), f"offset {off} differs in {name} at n={n}"
    # multi-tensor walk: every size in one collection, several shapes, + graph
    from optimizer_update_amd import Plan
    k = 2 if kind == "ademamix" else 1
    sizes = list(VARIANT_N)
    singles = {}
    for n in sizes:
        gen = W.rng(0, 6, n)
        p0 = W.params(n, storage, gen)
        g_host = W.cast_storage(np.where(gen.random(n) < 0.1, 0.0, gen.standard_normal(n)), storage)
        singles[n] = (p0, g_host, _run_single(L, kind, storage, p0, g_host, T, hp))
    for shape in ((0, 0, 0, 0, 0), (1, 4, 1, 256 * 4 * 2, 0), (8, 8, 4, 512 * 8, 0),
                  (2, 4, 2, 4096, 65536), (4, 4, 2, 1024, -1)):
        for order in (sizes, sizes[::-1]):
            for graph in (False, True):
                L.ou__force_multi(*shape)
                try:
                    segs = []
                    for n in order:
                        p0, g_host, _ = singles[n]
                        segs.append((H.to_dev(p0, storage), H.to_dev(g_host, storage),
                                     torch.zeros(k * n, device="cuda"), torch.zeros(n, device="cuda")))
                    plan = Plan(kind, segs)
                finally:
                    L.ou__force_multi(0, 0, 0, 0, 0)
                php = H.pkg_hp(hp)
                for t in range(1, T + 1):
                    (plan.graph_step if graph else plan.step)(php, t)
                torch.cuda.synchronize()
                for n, (P, G, S1, S2) in zip(order, segs):
                    ref = singles[n][2]
                    for a, b, name in zip(ref[:3], (W.from_torch(P), W.from_torch(S1), W.from_torch(S2)),
                                          ("p", "state1", "state2")):
                        assert a.tobytes() == b.tobytes(), f"multi {shape} graph={graph} differs in {name} at n={n}"
                plan.close()


def test_forced_multi_shape_beyond_launch_bound_is_refused(L):
    """The multi-tensor kernels take at most 8 waves per block (their
    512-thread launch bound): a plan forced to 16 is refused at creation with
    OU_EINVAL, before anything is launched, and the next plan is unaffected."""
    from optimizer_update_amd import OptimizerUpdateError, Plan
    segs = [tuple(torch.zeros(1024, device="cuda") for _ in range(4))]
    L.ou__force_multi(16, 4, 1, 256, -1)
    try:
        with pytest.raises(OptimizerUpdateError, match="waves=16"):
            Plan("adam", segs)
    finally:
        L.ou__force_multi(0, 0, 0, 0, 0)
    plan = Plan("adam", segs)
    plan.close()


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("storage", ["fp32", "bf16"])
def test_xcd_tile_runs_bitwise(orc, L, kind, storage):
    """The order in which blocks take tiles (runs of tiles per XCD) only
    moves work between blocks: every run length, block order, and a
    grid-stride grid with runs give the default's bits, equal to the oracle
    on a sample; a plan's work list in each order gives the direct calls'
    bits.  n = 2^21 - 3 puts 1,024 blocks on the default shape (runs apply)
    and leaves a one-element tail."""
    T = 2
    hp = _hp(kind, 0.01, True)
    n = (1 << 21) - 3
    gen = W.rng(0, 7, n)
    p0 = W.params(n, storage, gen)
    g_host = W.cast_storage(np.where(gen.random(n) < 0.1, 0.0, gen.standard_normal(n)), storage)
    base = _run_single(L, kind, storage, p0, g_host, T, hp)
    idx = np.unique(np.r_[0:4096, n - 4096:n, 0:n:4099])
    p_ref = p0[idx].copy()
    s1_ref, s2_ref = W.zero_states(idx.size, kind)
    for t in range(1, T + 1):
        orc.update_f32(H.KIND[kind], H.DT[storage], p_ref, g_host[idx].copy(), s1_ref, s2_ref, hp, t)
    H.assert_parity(base[0][idx], p_ref, storage, "p")
    H.assert_parity(base[2][idx], s2_ref, "fp32", "v")
    for run, force in ((-1, None), (1, None), (4, None), (16, None), (128, None),
                       (8, (256, 4, 2, 512, 0, 0))):
        L.ou__force_xcd(run)
        try:
            out = _run_single(L, kind, storage, p0, g_host, T, hp, force=force)
        finally:
            L.ou__force_xcd(0)
        for a, b_, name in zip(base[:3], out[:3], ("p", "state1", "state2")):
            assert a.tobytes() == b_.tobytes(), f"run {run} force {force} differs in {name}"
    # plans order their work lists by the same runs (6,144 items of 512
    # elements: 1,536 blocks, so runs up to 16 apply)
    from optimizer_update_amd import Plan
    k = 2 if kind == "ademamix" else 1
    m = 1 << 20
    inputs = []
    for i in range(3):
        gen = W.rng(0, 8, i)
        pi = W.params(m, storage, gen)
        gi = W.cast_storage(gen.standard_normal(m), storage)
        inputs.append((pi, gi, _run_single(L, kind, storage, pi, gi, T, hp)))
    for run in (-1, 1, 16):
        L.ou__force_xcd(run)
        try:
            segs = [(H.to_dev(pi, storage), H.to_dev(gi, storage), torch.zeros(k * m, device="cuda"),
                     torch.zeros(m, device="cuda")) for pi, gi, _ in inputs]
            plan = Plan(kind, segs)
        finally:
            L.ou__force_xcd(0)
        try:
            for t in range(1, T + 1):
                plan.step(H.pkg_hp(hp), t)
            torch.cuda.synchronize()
        finally:
            plan.close()
        for (_, _, ref), (P, G, S1, S2) in zip(inputs, segs):
            for a, b_, name in zip(ref[:3], (W.from_torch(P), W.from_torch(S1), W.from_torch(S2)),
                                   ("p", "state1", "state2")):
                assert a.tobytes() == b_.tobytes(), f"plan run {run} differs in {name}"


def test_stream_probes_touch_what_they_say(L):
    """The bandwidth probes on the large-tensor shape (XCD runs and a partial
    last run): the mix reads four streams and writes three back, so every
    buffer keeps its bits; the read probe writes nothing; the write probe
    fills p, s1 and s2 with its pattern (mask 0: element i holds the bits of
    i) and leaves g alone."""
    n = (1 << 22) + 4 * 1000
    gen = W.rng(0, 9, n)
    host = [gen.standard_normal(n).astype(np.float32) for _ in range(4)]
    dev = [torch.from_numpy(h).cuda() for h in host]
    for mode in (0, 1):
        st = L.ou__stream_probe(mode, *(d.data_ptr() for d in dev), n, H.stream_handle())
        assert st == 0, H.last_error(L)
        torch.cuda.synchronize()
        for h, d in zip(host, dev):
            assert d.cpu().numpy().tobytes() == h.tobytes(), mode
    st = L.ou__stream_probe(2, *(d.data_ptr() for d in dev), n, H.stream_handle())
    assert st == 0, H.last_error(L)
    torch.cuda.synchronize()
    pattern = np.arange(n, dtype=np.uint32)
    for i, (h, d) in enumerate(zip(host, dev)):
        got = d.cpu().numpy()
        if i == 1:
            assert got.tobytes() == h.tobytes()
        else:
            assert np.array_equal(got.view(np.uint32), pattern), i


# ----------------------------------------------------------------- sentinel

def test_public_path_ademamix_fp16_n64_first_update(orc, L):
    """The cell the page reports failing through its public collection path
    (section "Correctness failure and decision"): AdEMAMix, fp16, n = 64,
    weight decay 0.01, first update, first parameter of an eager
    collection.  Here it goes through the collection optimizer (plan), the
    per-tensor direct path and graph replay, and must be bitwise equal to
    the oracle and across paths."""
    from optimizer_update_amd import AdEMAMix32
    sizes = [64, 1024, 256, 4096, 777, 64]
    gen = W.rng(0, 3, 64)
    ps = [W.params(n, "fp16", gen) for n in sizes]
    gs = [W.grads(n, "normal", "fp16", gen) for n in sizes]
    results = {}
    for mode in ("plan", "per_tensor", "graph"):
        params = [H.to_dev(p, "fp16") for p in ps]
        grads = [H.to_dev(g, "fp16") for g in gs]
        opt = AdEMAMix32(params, lr=1e-3, betas=(0.9, 0.999, 0.9999), alpha=5.0, eps=1e-8,
                         weight_decay=0.01, grads=grads)
        if mode == "per_tensor":
            opt.step_per_tensor()
        else:
            opt.step(graph=(mode == "graph"))
        torch.cuda.synchronize()
        results[mode] = [(W.from_torch(p), W.from_torch(s1), W.from_torch(s2))
                         for p, s1, s2 in zip(opt.params, opt.state1, opt.state2)]
        opt.close()
    hp = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8,
                   weight_decay=0.01)
    for i, n in enumerate(sizes):
        p_ref = ps[i].copy()
        s1_ref, s2_ref = W.zero_states(n, "ademamix")
        orc.update_f32(O.ADEMAMIX, O.F16, p_ref, gs[i], s1_ref, s2_ref, hp, 1)
        for mode, res in results.items():
            H.assert_parity(res[i][0], p_ref, "fp16", f"{mode} param {i}")
            H.assert_parity(res[i][1], s1_ref, "fp32", f"{mode} state1 {i}")
            H.assert_parity(res[i][2], s2_ref, "fp32", f"{mode} state2 {i}")


# --------------------------------------------------------- graph and resume

def test_graph_replays_match_eager_with_work_between(L):
    """Ten graph steps with eager work and synchronisations between replays
    equal ten plan steps, bitwise, after every step."""
    from optimizer_update_amd import AdamW32
    sizes = [1024, 16 * 1024, 4096, 1 << 20, 31]
    gen = W.rng(0, 8, 0)
    ps = [W.params(n, "bf16", gen) for n in sizes]
    gs = [W.grads(n, "normal", "bf16", gen, sigma=0.01) for n in sizes]
    mk = lambda: AdamW32([H.to_dev(p, "bf16") for p in ps], lr=1e-3, weight_decay=0.01,
                         grads=[H.to_dev(g, "bf16") for g in gs])
    a, b = mk(), mk()
    scratch = torch.zeros(1 << 20, device="cuda")
    for t in range(10):
        a.step()
        b.step(graph=True)
        scratch.add_(1.0)                       # unrelated eager work between replays
        torch.cuda.synchronize()
        for x, y in zip(a.params + a.state1 + a.state2, b.params + b.state1 + b.state2):
            assert W.from_torch(x).tobytes() == W.from_torch(y).tobytes(), f"graph step {t + 1}"
    a.close()
    b.close()


def test_resume_is_bitwise(L):
    """k steps, copy params and states to fresh buffers, continue from
    step k+1: identical to an uninterrupted run."""
    from optimizer_update_amd import AdEMAMix32
    sizes = [1000, 4096, 70001]
    gen = W.rng(0, 9, 0)
    ps = [W.params(n, "fp32", gen) for n in sizes]
    gsteps = [[W.grads(n, "normal", "fp32", gen) for n in sizes] for _ in range(8)]
    grads = [torch.zeros(n, device="cuda") for n in sizes]
    full = AdEMAMix32([H.to_dev(p, "fp32") for p in ps], grads=grads)
    for t in range(8):
        for g, gh in zip(grads, gsteps[t]):
            g.copy_(torch.from_numpy(gh))
        full.step()
    first = AdEMAMix32([H.to_dev(p, "fp32") for p in ps], grads=grads)
    for t in range(4):
        for g, gh in zip(grads, gsteps[t]):
            g.copy_(torch.from_numpy(gh))
        first.step()
    sd = first.state_dict()
    params2 = [p.clone() for p in first.params]
    torch.cuda.synchronize()
    first.close()
    second = AdEMAMix32(params2, grads=grads)
    second.load_state_dict(sd)
    for t in range(4, 8):
        for g, gh in zip(grads, gsteps[t]):
            g.copy_(torch.from_numpy(gh))
        second.step()
    torch.cuda.synchronize()
    for x, y in zip(full.params + full.state1 + full.state2,
                    second.params + second.state1 + second.state2):
        assert W.from_torch(x).tobytes() == W.from_torch(y).tobytes()
    full.close()
    second.close()


# ---------------------------------------------------------------- edge cases

def test_errors_write_nothing(L):
    """Invalid calls on real device buffers return an error and leave every
    buffer untouched; n = 0 is a no-op."""
    n = 1024
    p = torch.rand(n, device="cuda")
    g = torch.rand(n, device="cuda")
    s1 = torch.zeros(2 * n, device="cuda")
    s2 = torch.zeros(n, device="cuda")
    before = [W.from_torch(x) for x in (p, g, s1, s2)]
    hp = _hp("adam", 0.01, False)
    sh = H.stream_handle()
    cases = {
        "overlap p/s2": (0, 0, p.data_ptr(), g.data_ptr(), s1.data_ptr(), p.data_ptr() + 64, n),
        "grad is state": (0, 0, p.data_ptr(), s2.data_ptr(), s1.data_ptr(), s2.data_ptr(), n),
        "misaligned": (0, 0, p.data_ptr() + 2, g.data_ptr(), s1.data_ptr(), s2.data_ptr(), n),
        "bad dtype": (0, 5, p.data_ptr(), g.data_ptr(), s1.data_ptr(), s2.data_ptr(), n),
        "ademamix overlap": (1, 0, p.data_ptr(), g.data_ptr(), s1.data_ptr(), s1.data_ptr() + 4 * n + 4, n),
    }
    for name, (kind, dt, pp, gg, a, b, nn) in cases.items():
        st = L.optimizer_update_32bit(kind, dt, pp, gg, a, b, nn, hp.beta1, hp.beta2, hp.beta3,
                                      hp.alpha, hp.eps, hp.weight_decay, 1, hp.lr, 0, sh)
        assert st < 0, name
    st = L.optimizer_update_32bit(0, 0, p.data_ptr(), g.data_ptr(), s1.data_ptr(), s2.data_ptr(),
                                  n, hp.beta1, hp.beta2, hp.beta3, hp.alpha, hp.eps,
                                  hp.weight_decay, 0, hp.lr, 0, sh)
    assert st == -1     # step 0
    st = L.optimizer_update_32bit(0, 0, p.data_ptr(), g.data_ptr(), s1.data_ptr(), s2.data_ptr(),
                                  0, hp.beta1, hp.beta2, hp.beta3, hp.alpha, hp.eps,
                                  hp.weight_decay, 1, hp.lr, 0, sh)
    assert st == 0
    torch.cuda.synchronize()
    for x, b in zip((p, g, s1, s2), before):
        assert W.from_torch(x).tobytes() == b.tobytes()
