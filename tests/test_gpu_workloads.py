"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: the model-like collection (505 bf16 tensors, AdamW) and
flat tensors of 2^28, 2^30 and 2^31 + 3 elements.

Inputs are drawn on the device with torch's seeded generator; the values the
oracle needs are copied to the host before the first step.  Large tensors
are compared on sampled elements, which is exact because every element is
updated on its own: the sample always includes the first and last 4096
elements, the elements around 2^31 where present, and a regular stride.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    return O.load()


def _sample(n: int, stride: int = 4099) -> np.ndarray:
    parts = [np.arange(min(n, 4096)), np.arange(max(0, n - 4096), n), np.arange(0, n, stride)]
    if n > (1 << 31):
        parts.append(np.arange((1 << 31) - 2048, min(n, (1 << 31) + 2048)))
    return np.unique(np.concatenate(parts))


def _gather(t: torch.Tensor, idx_dev: torch.Tensor) -> np.ndarray:
    return W.from_torch(t.index_select(0, idx_dev))


def _flat_inputs(kind, storage, n, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    dt = W.STORAGE_TORCH[storage]
    p = torch.empty(n, device="cuda").uniform_(-1.0, 1.0, generator=gen).to(dt)
    g = (torch.randn(n, device="cuda", generator=gen) * 1e-3).to(dt)
    k = 2 if kind == "ademamix" else 1
    return p, g, torch.zeros(k * n, device="cuda"), torch.zeros(n, device="cuda")


def _check_sample(orc, kind, storage, n, p0, g0, got, idx, hp, steps):
    """Run the oracle on the sampled elements and compare."""
    m = idx.size
    p_ref = p0.copy()
    s1_ref, s2_ref = W.zero_states(m, kind)
    for t in range(1, steps + 1):
        orc.update_f32(H.KIND[kind], H.DT[storage], p_ref, g0, s1_ref, s2_ref, hp, t, nthreads=8)
    P, S1f, S1s, S2 = got
    what = f"{kind} {storage} n={n} after {steps} steps"
    H.assert_parity(P, p_ref, storage, "p " + what)
    H.assert_parity(S1f, s1_ref[:m], "fp32", "m " + what)
    H.assert_parity(S2, s2_ref, "fp32", "v " + what)
    if kind == "ademamix":
        H.assert_parity(S1s, s1_ref[m:], "fp32", "m2 " + what)


@pytest.mark.parametrize("kind,storage,log2n", [
    ("adam", "fp32", 28), ("adam", "bf16", 28), ("ademamix", "fp32", 28), ("ademamix", "bf16", 28),
    ("adam", "fp32", 30), ("adam", "bf16", 30), ("ademamix", "fp32", 30), ("ademamix", "bf16", 30)])
def test_flat_tensor_100_steps(orc, kind, storage, log2n):
    """A single flat tensor, grads N(0, 1e-3^2) fixed, 100 steps through the
    direct entry (the benchmark's launch shape), sampled against the oracle."""
    import optimizer_update_amd as ou
    n = 1 << log2n
    steps = 100
    hp = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8,
                   weight_decay=0.0 if kind == "adam" else 0.01)
    p, g, s1, s2 = _flat_inputs(kind, storage, n, seed=log2n)
    idx = _sample(n)
    idx_dev = torch.from_numpy(idx).cuda()
    p0, g0 = _gather(p, idx_dev), _gather(g, idx_dev)
    for t in range(1, steps + 1):
        ou.optimizer_update_32bit(kind, p, g, s1, s2, step=t, lr=hp.lr, beta1=hp.beta1,
                                  beta2=hp.beta2, beta3=hp.beta3, alpha=hp.alpha, eps=hp.eps,
                                  weight_decay=hp.weight_decay)
    torch.cuda.synchronize()
    got = (_gather(p, idx_dev), _gather(s1[:n], idx_dev),
           _gather(s1[n:], idx_dev) if kind == "ademamix" else None, _gather(s2, idx_dev))
    assert _gather(g, idx_dev).tobytes() == g0.tobytes(), "grad changed"
    _check_sample(orc, kind, storage, n, p0, g0, got, idx, hp, steps)


def test_beyond_2_31_elements_single_and_plan(orc):
    """fp16 Adam on n = 2^31 + 3 elements (indices past the 32-bit range),
    direct entry and a one-segment plan, 2 steps: the two paths are bitwise
    equal and the sampled elements (including those around 2^31) match the
    oracle."""
    from optimizer_update_amd import Plan
    import optimizer_update_amd as ou
    kind, storage, n, steps = "adam", "fp16", (1 << 31) + 3, 2
    hp = O.HParams(lr=1e-3, weight_decay=0.01)
    a = _flat_inputs(kind, storage, n, seed=31)
    b = (a[0].clone(), a[1], torch.zeros_like(a[2]), torch.zeros_like(a[3]))
    idx = _sample(n, stride=65537)
    idx_dev = torch.from_numpy(idx).cuda()
    p0, g0 = _gather(a[0], idx_dev), _gather(a[1], idx_dev)
    plan = Plan(kind, [b])
    php = H.pkg_hp(hp)
    for t in range(1, steps + 1):
        ou.optimizer_update_32bit(kind, *a, step=t, lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2,
                                  eps=hp.eps, weight_decay=hp.weight_decay)
        plan.step(php, t)
    torch.cuda.synchronize()
    for x, y in zip((a[0], a[2], a[3]), (b[0], b[2], b[3])):
        assert torch.equal(x.view(torch.int16) if x.dtype != torch.float32 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype != torch.float32 else y.view(torch.int32))
    got = (_gather(a[0], idx_dev), _gather(a[2], idx_dev), None, _gather(a[3], idx_dev))
    _check_sample(orc, kind, storage, n, p0, g0, got, idx, hp, steps)
    plan.close()


def test_model_collection_plan_per_tensor_graph(orc):
    """The model-like collection (24 layers of norm/bias/LoRA/weight tensors
    plus a 32000x1024 embedding; bf16 params and grads, fp32 states; AdamW
    lr 1e-3, wd 0.01; grads N(0, 0.01^2) fixed), 10 steps three ways: one
    plan launch per step, one direct call per tensor, graph replay.  The
    three are bitwise equal; every tensor of <= 16384 elements is compared
    whole with the oracle, larger ones on sampled elements."""
    from optimizer_update_amd import AdamW32
    shapes = W.model_collection()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    ps, gs = [], []
    for _, shp in shapes:
        m = W.numel(shp)
        ps.append(torch.empty(m, device="cuda").uniform_(-1, 1, generator=gen).to(torch.bfloat16))
        gs.append((torch.randn(m, device="cuda", generator=gen) * 0.01).to(torch.bfloat16))
    samples = []
    for p, g in zip(ps, gs):
        m = p.numel()
        idx = np.arange(m) if m <= 16384 else _sample(m)
        idx_dev = torch.from_numpy(idx).cuda()
        samples.append((idx, idx_dev, _gather(p, idx_dev), _gather(g, idx_dev)))
    opts = {mode: AdamW32([p.clone() for p in ps], lr=1e-3, weight_decay=0.01, grads=gs)
            for mode in ("plan", "per_tensor", "graph")}
    for _ in range(10):
        opts["plan"].step()
        opts["per_tensor"].step_per_tensor()
        opts["graph"].step(graph=True)
    torch.cuda.synchronize()
    ref = opts["plan"]
    for mode in ("per_tensor", "graph"):
        o = opts[mode]
        for a, b in zip(ref.params + ref.state1 + ref.state2, o.params + o.state1 + o.state2):
            va = a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32)
            vb = b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)
            assert torch.equal(va, vb), mode
    hp = O.HParams(lr=1e-3, weight_decay=0.01)
    for (name, shp), (idx, idx_dev, p0, g0), p, s1, s2 in zip(shapes, samples, ref.params,
                                                               ref.state1, ref.state2):
        got = (_gather(p, idx_dev), _gather(s1, idx_dev), None, _gather(s2, idx_dev))
        _check_sample(orc, "adam", "bf16", W.numel(shp), p0, g0, got, idx, hp, 10)
    for o in opts.values():
        o.close()
