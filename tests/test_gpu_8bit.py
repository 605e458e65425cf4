"""GPU parity of the 8-bit block-wise path against the CPU oracle.

The page "Investigate a 256-thread SM103 path for small 32-bit optimizer
tensors" times AdamW8bit collections whose small tensors (below
min_8bit_size = 4,096 elements) take the 32-bit path; these tests cover the
8-bit leg and the routing.  The kernels perform the oracle's steps with the
same binary32 operations, the same exact nearest-magnitude quantizer and an
exact (order-free) block maximum, so parameters, codes and absmax must be bit-identical to the
oracle, across the kernel's launch shapes, the element-by-element path and
plans.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

KIND = {"adam": O.ADAM, "ademamix": O.ADEMAMIX}
QB = O.QBLOCK
SIZES = (1, 33, 255, 256, 257, 1023, 1024, 4095, 4096, 4097, 65539)


@pytest.fixture(scope="module")
def orc():
    return O.load()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return H.lib()


def _nb(n):
    return -(-n // QB)


def _zero_host(kind, n):
    k = 2 if kind == "ademamix" else 1
    return (np.zeros(k * n, np.uint8), np.zeros(n, np.uint8), np.zeros(k * _nb(n), np.float32),
            np.zeros(_nb(n), np.float32))


def _dev_states(kind, n, offset=0):
    """Zero states on the device, each placed `offset` bytes/elements past an
    aligned start (offset > 0 exercises the element-by-element path)."""
    k = 2 if kind == "ademamix" else 1
    c1 = torch.zeros(k * n + offset, dtype=torch.uint8, device="cuda")[offset:]
    c2 = torch.zeros(n + offset, dtype=torch.uint8, device="cuda")[offset:]
    a1 = torch.zeros(k * _nb(n), dtype=torch.float32, device="cuda")
    a2 = torch.zeros(_nb(n), dtype=torch.float32, device="cuda")
    return c1, c2, a1, a2


def _raw8(L, kind, storage, P, G, st, n, hp, t, flag=0):
    c1, c2, a1, a2 = st
    return L.optimizer_update_8bit_blockwise(KIND[kind] | flag, H.DT[storage], P.data_ptr(),
                                             G.data_ptr(), c1.data_ptr(), c2.data_ptr(),
                                             a1.data_ptr(), a2.data_ptr(), n, hp.beta1, hp.beta2,
                                             hp.beta3, hp.alpha, hp.eps, hp.weight_decay, t, hp.lr,
                                             int(hp.skip_zeros), H.stream_handle())


def _gpu_run(L, kind, storage, p0, gsteps, hp, offset=0, flag=0, force=None):
    n = p0.size
    P = H.to_dev(np.concatenate([np.zeros(offset, p0.dtype), p0]), storage)[offset:]
    G = torch.empty(n + offset, dtype=W.STORAGE_TORCH[storage], device="cuda")[offset:]
    st = _dev_states(kind, n, offset)
    if force:
        L.ou__force_8bit(*force)
    try:
        for t, g in enumerate(gsteps, start=1):
            G.copy_(W.to_torch(g, storage, "cuda"))
            rc = _raw8(L, kind, storage, P, G, st, n, hp, t, flag)
            assert rc == 0, H.last_error(L)
    finally:
        L.ou__force_8bit(0, 0, 0, 0)
    torch.cuda.synchronize()
    return (W.from_torch(P), *(x.cpu().numpy() for x in st))


def _oracle_run(orc, kind, storage, p0, gsteps, hp, flag=0):
    p = p0.copy()
    st = _zero_host(kind, p0.size)
    for t, g in enumerate(gsteps, start=1):
        orc.update_8bit_f32(KIND[kind] | flag, H.DT[storage], p, g.copy(), *st, hp, t)
    return (p, *st)


def _assert_same(got, ref, storage, what):
    H.assert_parity(got[0], ref[0], storage, "p " + what)
    names = ("state1 codes", "state2 codes", "absmax1", "absmax2")
    for a, b, name in zip(got[1:], ref[1:], names):
        assert a.tobytes() == b.tobytes(), f"{name} {what}: {np.count_nonzero(a != b)} differ"


def _grads(storage, n, T, pattern, key):
    return [W.grads(n, pattern, storage, W.rng(3, *key, t)) for t in range(T)]


@pytest.mark.parametrize("kind", list(KIND))
@pytest.mark.parametrize("storage", ["fp32", "fp16", "bf16"])
def test_8bit_matches_oracle(orc, L, kind, storage):
    """Every size of the list (partial blocks, one block, many), zero/normal/
    mixed gradients, wd 0 / 0.01, skip_zeros off/on, 10 steps: parameters,
    codes and absmax bitwise equal to the oracle's."""
    T = 10
    for pattern in W.GRAD_PATTERNS:
        for wd, skip in ((0.0, False), (0.01, True), (0.01, False)):
            hp = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8,
                           weight_decay=wd, skip_zeros=skip)
            for n in SIZES:
                key = (list(KIND).index(kind), H.DT[storage], W.GRAD_PATTERNS.index(pattern), n)
                p0 = W.params(n, storage, W.rng(3, 0, *key))
                gs = _grads(storage, n, T, pattern, key)
                got = _gpu_run(L, kind, storage, p0, gs, hp)
                ref = _oracle_run(orc, kind, storage, p0, gs, hp)
                _assert_same(got, ref, storage, f"{kind} {storage} {pattern} wd={wd} skip={skip} n={n}")


@pytest.mark.parametrize("kind", list(KIND))
@pytest.mark.parametrize("storage", ["fp32", "bf16"])
def test_8bit_launch_variants_and_paths(orc, L, kind, storage):
    """Waves per workgroup, blocks per wave, the element-by-element path and
    misaligned buffers give the same bits."""
    T = 4
    hp = O.HParams(lr=1e-2, weight_decay=0.05, skip_zeros=True)
    for n in (257, 4097, 65539, (1 << 18) + 3):
        gen = W.rng(3, 9, n)
        p0 = W.params(n, storage, gen)
        gs = [W.cast_storage(np.where(gen.random(n) < 0.1, 0.0, gen.standard_normal(n)), storage)
              for _ in range(T)]
        base = _gpu_run(L, kind, storage, p0, gs, hp)
        if n < 70000:
            _assert_same(base, _oracle_run(orc, kind, storage, p0, gs, hp), storage, f"n={n}")
        # even blocks per wave take the pipelined wide path, odd ones the
        # generic path; the last force is the element-by-element path
        for force in ((1, 1, 0, 0), (4, 1, 0, 0), (2, 8, 0, 0), (16, 2, 0, 0), (4, 3, 0, 0),
                      (8, 6, 0, 0), (4, 4, 0, 1)):
            got = _gpu_run(L, kind, storage, p0, gs, hp, force=force)
            for a, b in zip(got, base):
                assert a.tobytes() == b.tobytes(), (force, n)
        for off in (1, 3):
            got = _gpu_run(L, kind, storage, p0, gs, hp, offset=off)
            for a, b in zip(got, base):
                assert a.tobytes() == b.tobytes(), ("offset", off, n)
        for run in (4, 16):   # XCD runs of workgroups (one block each: 1,025 of them)
            L.ou__force_xcd(run)
            try:
                got = _gpu_run(L, kind, storage, p0, gs, hp, force=(1, 1, 0, 0))
            finally:
                L.ou__force_xcd(0)
            for a, b in zip(got, base):
                assert a.tobytes() == b.tobytes(), ("xcd run", run, n)


@pytest.mark.parametrize("kind", list(KIND))
def test_8bit_decay_after(orc, L, kind):
    """OU_DECAY_AFTER with 8-bit states: bitwise equal to the oracle's
    flagged path, and different from the default order in binary32."""
    T = 5
    hp = O.HParams(lr=1e-2, weight_decay=0.1)
    n = 4097
    p0 = W.params(n, "fp32", W.rng(3, 11, n))
    gs = _grads("fp32", n, T, "normal", (11, n))
    got = _gpu_run(L, kind, "fp32", p0, gs, hp, flag=O.DECAY_AFTER)
    _assert_same(got, _oracle_run(orc, kind, "fp32", p0, gs, hp, flag=O.DECAY_AFTER), "fp32", "flag")
    assert got[0].tobytes() != _oracle_run(orc, kind, "fp32", p0, gs, hp)[0].tobytes()


@pytest.mark.parametrize("kind,storage", [("adam", "fp32"), ("ademamix", "bf16")])
def test_8bit_large_tensor_sampled_blocks(orc, L, kind, storage):
    """2^26 + 3 elements, 3 steps: blocks are independent, so whole blocks
    (the first 8, the partial last one, and every 1,031st) are checked
    against the oracle run on those blocks alone."""
    n = (1 << 26) + 3
    T = 3
    hp = O.HParams(lr=1e-3, weight_decay=0.01)
    p0 = W.params(n, storage, W.rng(3, 12, n))
    gs = [W.grads(n, "normal", storage, W.rng(3, 13, t)) for t in range(T)]
    got = _gpu_run(L, kind, storage, p0, gs, hp)
    nb = _nb(n)
    blocks = np.unique(np.r_[0:8, nb - 1, 0:nb:1031])
    for b in blocks:
        lo, hi = b * QB, min(n, (b + 1) * QB)
        ref = _oracle_run(orc, kind, storage, p0[lo:hi].copy(), [g[lo:hi].copy() for g in gs], hp)
        what = f"block {b}"
        H.assert_parity(got[0][lo:hi], ref[0], storage, "p " + what)
        assert got[1][lo:hi].tobytes() == ref[1][:hi - lo].tobytes(), what
        assert got[2][lo:hi].tobytes() == ref[2].tobytes(), what
        assert got[3][b] == ref[3][0] and got[4][b] == ref[4][0], what
        if kind == "ademamix":
            assert got[1][n + lo:n + hi].tobytes() == ref[1][hi - lo:].tobytes(), what
            assert got[3][nb + b] == ref[3][1], what


@pytest.mark.parametrize("kind", list(KIND))
def test_8bit_plan_equals_direct(L, kind):
    """A plan over several tensors (all dtypes, several work-item sizes)
    gives the bits of one direct call per tensor."""
    import optimizer_update_amd as ou
    T = 3
    hp = O.HParams(lr=1e-3, weight_decay=0.01, skip_zeros=True)
    # with one-block items the bf16 group has 4,368 items (1,092 workgroups):
    # its work list takes the XCD-run order
    specs = [(4096, "bf16"), (257, "fp32"), (65539, "fp16"), (1 << 16, "bf16"), (5000, "fp32"),
             (1 << 20, "bf16")]
    inputs = []
    for i, (n, storage) in enumerate(specs):
        gen = W.rng(3, 14, i)
        p0 = W.params(n, storage, gen)
        gs = [W.cast_storage(np.where(gen.random(n) < 0.1, 0.0, gen.standard_normal(n)), storage)
              for _ in range(T)]
        inputs.append((n, storage, p0, gs, _gpu_run(L, kind, storage, p0, gs, hp)))
    for chunk in (0, 1, 2, 3, 6):
        L.ou__force_8bit(0, 0, chunk, 0)
        try:
            tensors = []
            for n, storage, p0, gs, _ in inputs:
                P = H.to_dev(p0, storage)
                G = torch.empty(n, dtype=W.STORAGE_TORCH[storage], device="cuda")
                tensors.append((P, G, *_dev_states(kind, n)))
            plan = ou.Plan8(kind, tensors)
        finally:
            L.ou__force_8bit(0, 0, 0, 0)
        try:
            for t in range(1, T + 1):
                for (n, storage, p0, gs, _), tt in zip(inputs, tensors):
                    tt[1].copy_(W.to_torch(gs[t - 1], storage, "cuda"))
                plan.step(H.pkg_hp(hp), t)
            torch.cuda.synchronize()
        finally:
            plan.close()
        for (n, storage, p0, gs, ref), tt in zip(inputs, tensors):
            got = (W.from_torch(tt[0]), *(x.cpu().numpy() for x in tt[2:]))
            for a, b in zip(got, ref):
                assert a.tobytes() == b.tobytes(), (chunk, n, storage)


@pytest.mark.parametrize("cls", ["AdamW8bit", "AdEMAMix8bit"])
def test_8bit_collection_routing(orc, cls):
    """min_8bit_size = 4,096 (the page's default): tensors below it keep fp32
    states and take the 32-bit path, the others 8-bit states.  The plan step
    equals the per-tensor loop and the graph replay bitwise (eager work
    between replays) and each tensor equals its oracle (8-bit or 32-bit)."""
    import optimizer_update_amd as ou
    shapes = [(1024,), (4096,), (16, 1024), (4095,), (64,), (1024, 16), (3000, 7)]
    rows = [(W.params(W.numel(s), "bf16", W.rng(3, 15, i)),
             W.grads(W.numel(s), "normal", "bf16", W.rng(3, 16, i))) for i, s in enumerate(shapes)]
    runs = {}
    for mode in ("plan", "per_tensor", "graph"):
        ps = [H.to_dev(p0, "bf16") for p0, _ in rows]
        gs = [H.to_dev(g, "bf16") for _, g in rows]
        opt = getattr(ou, cls)(ps, grads=gs, lr=1e-3, weight_decay=0.01)
        assert [s[0] for s in opt.state] == ["32bit" if W.numel(s) < 4096 else "8bit" for s in shapes]
        for i in range(3):
            if mode == "per_tensor":
                opt.step_per_tensor()
            else:
                opt.step(graph=(mode == "graph"))
            if i == 1:          # eager work between replays
                torch.cuda.synchronize()
                _ = (ps[0].float() * 2).sum().item()
        torch.cuda.synchronize()
        runs[mode] = [(W.from_torch(p), [x.cpu().numpy() for x in st[1:]]) for p, st in zip(ps, opt.state)]
        hp = O.HParams(**{k: getattr(opt.hp, k) for k in ("lr", "beta1", "beta2", "beta3", "alpha",
                                                          "eps", "weight_decay", "skip_zeros")})
        kind = ou.optim.__dict__[cls].kind
        opt.close()
    for mode in ("per_tensor", "graph"):
        for (pa, sa), (pb, sb) in zip(runs["plan"], runs[mode]):
            assert pa.tobytes() == pb.tobytes(), mode
            for x, y in zip(sa, sb):
                assert x.tobytes() == y.tobytes(), mode
    for (p0, g), (p, states), shape in zip(rows, runs["plan"], shapes):
        n = W.numel(shape)
        if n >= 4096:
            ref = _oracle_run(orc, kind, "bf16", p0, [g] * 3, hp)
            H.assert_parity(p, ref[0], "bf16", f"{cls} 8-bit p n={n}")
            for a, b in zip(states, ref[1:]):
                assert a.tobytes() == b.tobytes(), n
        else:
            pr = p0.copy()
            s1, s2 = W.zero_states(n, kind)
            for t in range(1, 4):
                orc.update_f32(KIND[kind], O.BF16, pr, g.copy(), s1, s2, hp, t)
            H.assert_parity(p, pr, "bf16", f"{cls} 32-bit p n={n}")
            H.assert_parity(states[0], s1, "fp32", f"{cls} 32-bit m n={n}")


@pytest.mark.parametrize("kind", list(KIND))
def test_8bit_long_run(orc, L, kind):
    """1,000 steps (the coverage matrix's horizon), bf16 storage, normal and
    mixed-magnitude gradients redrawn every step, wd 0.01: parameters, codes
    and absmax bitwise equal to the oracle at steps 1, 2, 10 and 1,000."""
    T = 1000
    hp = O.HParams(lr=1e-3, weight_decay=0.01)
    for pattern in ("normal", "mixed"):
        for n in (1, 257, 4097):
            key = (20, list(KIND).index(kind), W.GRAD_PATTERNS.index(pattern), n)
            p0 = W.params(n, "bf16", W.rng(3, *key))
            P = H.to_dev(p0, "bf16")
            G = torch.empty(n, dtype=torch.bfloat16, device="cuda")
            st = _dev_states(kind, n)
            ref = (p0.copy(), *_zero_host(kind, n))
            for t in range(1, T + 1):
                g = W.grads(n, pattern, "bf16", W.rng(3, *key, t))
                G.copy_(W.to_torch(g, "bf16", "cuda"))
                rc = _raw8(L, kind, "bf16", P, G, st, n, hp, t)
                assert rc == 0, H.last_error(L)
                orc.update_8bit_f32(KIND[kind], O.BF16, ref[0], g, *ref[1:], hp, t)
                if t in (1, 2, 10, T):
                    torch.cuda.synchronize()
                    got = (W.from_torch(P), *(x.cpu().numpy() for x in st))
                    _assert_same(got, ref, "bf16", f"{kind} {pattern} n={n} step {t}")


def test_8bit_beyond_2_31_elements(orc):
    """bf16 Adam with 8-bit states on n = 2^31 + 3 elements (element indices
    past the 32-bit range, 8,388,609 blocks), single entry and a one-segment
    plan, 2 steps: the two are bitwise equal, and sampled whole blocks (the
    first, the partial last, those around element 2^31, a stride) equal the
    oracle run on those blocks alone."""
    import optimizer_update_amd as ou
    n, T = (1 << 31) + 3, 2
    hp = O.HParams(lr=1e-3, weight_decay=0.01)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(231)
    P = torch.empty(n, device="cuda").uniform_(-1.0, 1.0, generator=gen).to(torch.bfloat16)
    G = (torch.randn(n, device="cuda", generator=gen) * 1e-3).to(torch.bfloat16)
    P2 = P.clone()
    nb = _nb(n)
    blocks = np.unique(np.r_[0:2, nb - 2:nb, (1 << 23) - 2:(1 << 23) + 2, 0:nb:500009])
    blocks = blocks[blocks < nb]          # element 2^31 lies in block 2^23, the last full one
    idx = np.concatenate([np.arange(b * QB, min(n, (b + 1) * QB)) for b in blocks])
    idx_dev = torch.from_numpy(idx).cuda()
    p0 = W.from_torch(P.index_select(0, idx_dev))
    g0 = W.from_torch(G.index_select(0, idx_dev))
    a = _dev_states("adam", n)
    b = _dev_states("adam", n)
    plan = ou.Plan8("adam", [(P2, G, *b)])
    try:
        for t in range(1, T + 1):
            ou.optimizer_update_8bit_blockwise("adam", P, G, *a, step=t, lr=hp.lr,
                                               weight_decay=hp.weight_decay)
            plan.step(H.pkg_hp(hp), t)
        torch.cuda.synchronize()
    finally:
        plan.close()
    assert torch.equal(P.view(torch.int16), P2.view(torch.int16))
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
    got_p = W.from_torch(P.index_select(0, idx_dev))
    got_c1 = a[0].index_select(0, idx_dev).cpu().numpy()
    got_c2 = a[1].index_select(0, idx_dev).cpu().numpy()
    a1 = a[2].cpu().numpy()
    a2 = a[3].cpu().numpy()
    off = 0
    for blk in blocks:
        lo, hi = blk * QB, min(n, (blk + 1) * QB)
        m = hi - lo
        ref = (p0[off:off + m].copy(), *_zero_host("adam", m))
        for t in range(1, T + 1):
            orc.update_8bit_f32(O.ADAM, O.BF16, ref[0], g0[off:off + m].copy(), *ref[1:], hp, t)
        what = f"block {blk}"
        H.assert_parity(got_p[off:off + m], ref[0], "bf16", "p " + what)
        assert got_c1[off:off + m].tobytes() == ref[1].tobytes(), what
        assert got_c2[off:off + m].tobytes() == ref[2].tobytes(), what
        assert a1[blk] == ref[3][0] and a2[blk] == ref[4][0], what
        off += m
    del P, P2, G, a, b
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kind", list(KIND))
@pytest.mark.parametrize("storage", ["fp32", "bf16"])
def test_8bit_bias_corrections_reaching_one(orc, L, kind, storage):
    """Whole-block runs leave out a bias correction once fl32(1 - beta^t)
    is exactly 1.  Steps 1-2 (neither is 1), 200-201 (m's is 1 for
    beta1 = 0.9), 10^6 and 10^6 + 1 (both are 1), and with beta1 = 0.999,
    beta2 = 0.9 step 200 (only v's is 1, which takes the general path): the
    parameters, codes and absmax equal the oracle's bitwise."""
    n = (1 << 20) + 5
    for b1, b2 in ((0.9, 0.999), (0.999, 0.9)):
        hp = O.HParams(lr=1e-3, beta1=b1, beta2=b2, weight_decay=0.01)
        key = (21, list(KIND).index(kind), H.DT[storage], int(b1 * 1000))
        p0 = W.params(n, storage, W.rng(3, *key))
        P = H.to_dev(p0, storage)
        G = torch.empty(n, dtype=W.STORAGE_TORCH[storage], device="cuda")
        st = _dev_states(kind, n)
        ref = (p0.copy(), *_zero_host(kind, n))
        for i, t in enumerate((1, 2, 200, 201, 10 ** 6, 10 ** 6 + 1)):
            g = W.grads(n, "normal", storage, W.rng(3, *key, i))
            G.copy_(W.to_torch(g, storage, "cuda"))
            rc = _raw8(L, kind, storage, P, G, st, n, hp, t)
            assert rc == 0, H.last_error(L)
            orc.update_8bit_f32(KIND[kind], H.DT[storage], ref[0], g, *ref[1:], hp, t)
            if t in (2, 201, 10 ** 6 + 1):
                torch.cuda.synchronize()
                got = (W.from_torch(P), *(x.cpu().numpy() for x in st))
                _assert_same(got, ref, storage, f"{kind} {storage} b1={b1} step {t}")


def _quantizer_cases(orc):
    """(value, absmax) pairs where a quantizer goes wrong if it is not the
    exact nearest magnitude: midpoints of both types times absmax, rounded to
    binary32, with their neighbours two ulps either way; exact ties (midpoints
    that binary32 holds, times a power-of-two absmax); values uniform and
    log-uniform below absmax, both signs; the block's own absmax; +-0 and
    NaN; absmax from subnormal to the largest binary32, 0 and +inf."""
    gen = np.random.default_rng(8080)
    f32 = np.float32
    fmax = np.finfo(np.float32).max
    mids = []
    for signed in (True, False):
        mags = orc.qmap(signed).astype(np.float64)
        mids.append((mags[:-1] + mags[1:]) / 2)
    mids = np.concatenate(mids)
    ties = np.unique(mids[mids.astype(np.float32).astype(np.float64) == mids])
    vals, amax = [], []
    for A in [f32(1.0), f32(0.7), f32(1.234567e-3), f32(2.0 ** -149), f32(3 * 2.0 ** -140),
              f32(2.0 ** -130), f32(3.4e38), fmax, f32(2.0 ** 100), f32(2.0 ** -20)]:
        near = (mids * float(A)).astype(np.float32)
        group = [near]
        for k in (1, 2):
            up, dn = near.copy(), near.copy()
            for _ in range(k):
                up = np.nextafter(up, f32(np.inf))
                dn = np.nextafter(dn, f32(0))
            group += [up, dn]
        group += [(gen.uniform(0, 1, 3000) * float(A)).astype(np.float32),
                  (10.0 ** gen.uniform(-10, 0, 3000) * float(A)).astype(np.float32),
                  np.array([A, 0.0], np.float32)]
        if float(A) in (1.0, 2.0 ** -20, 2.0 ** 100, 2.0 ** -130):   # powers of two: exact ties
            group.append((ties * float(A)).astype(np.float32))
        v = np.concatenate(group)
        v = v[np.abs(v) <= A]
        v = np.concatenate([v, -v[::3], np.array([-0.0, np.nan], np.float32)])
        vals.append(v)
        amax.append(np.full(v.size, A, np.float32))
    # absmax 0 (a block of zeros and NaNs) and +inf (finite values, and +-inf)
    vals.append(np.array([0.0, -0.0, np.nan], np.float32))
    amax.append(np.zeros(3, np.float32))
    v = np.array([0.0, 1.0, -2.0, 3e38, -1e-30, np.inf, -np.inf, np.nan], np.float32)
    vals.append(v)
    amax.append(np.full(v.size, np.inf, np.float32))
    return np.concatenate(vals), np.concatenate(amax)


def test_device_quantizer_matches_oracle(orc, L):
    """The kernels' quantizer (the ou__quant8 hook runs the update kernels'
    composition: reciprocal of absmax, offset estimate, LDS key table, one
    exact binary64 comparison) gives the oracle's code on every pair of
    _quantizer_cases: signed code of the value, unsigned code of |value|."""
    v, a = _quantizer_cases(orc)
    n = v.size
    dv = torch.from_numpy(v).cuda()
    da = torch.from_numpy(a).cuda()
    cs = torch.full((n,), 0xAA, dtype=torch.uint8, device="cuda")
    cu = torch.full((n,), 0xAA, dtype=torch.uint8, device="cuda")
    st = L.ou__quant8(dv.data_ptr(), da.data_ptr(), cs.data_ptr(), cu.data_ptr(), n, H.stream_handle())
    assert st == 0, H.last_error(L)
    got_s = cs.cpu().numpy()
    got_u = cu.cpu().numpy()
    want_s = np.array([orc.qcode(True, float(x), float(y)) for x, y in zip(v, a)], np.uint8)
    want_u = np.array([orc.qcode(False, abs(float(x)), float(y)) for x, y in zip(v, a)], np.uint8)
    bad_s = np.nonzero(got_s != want_s)[0]
    bad_u = np.nonzero(got_u != want_u)[0]
    assert bad_s.size == 0, [(float(v[i]), float(a[i]), int(got_s[i]), int(want_s[i])) for i in bad_s[:5]]
    assert bad_u.size == 0, [(float(v[i]), float(a[i]), int(got_u[i]), int(want_u[i])) for i in bad_u[:5]]
    assert n > 50000
