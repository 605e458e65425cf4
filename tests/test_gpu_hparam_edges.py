"""GPU parity at the edges of the hyperparameter domain, two-state kinds.

The entry points accept beta in [0, 1), eps >= 0, any finite lr and weight
decay, and any step >= 1. At the ends of that domain:
- beta = 0: the moments are the current gradient and the bias corrections are 1.
- beta = 1 - 2^-24: the largest binary32 below 1, so the first step's bias
  correction is 2^-24, the smallest the host can form.
- eps = 0: an element with v = 0 divides 0 by 0.
- lr = 0 with decay: d = 1 and lr·u = 0, so every parameter keeps its bits.
- lr·wd = 2: the decay factor d = 1 - lr·wd is -1, flipping the parameter's sign each step.
- a jump to step 10^6: both bias corrections round to 1.
- AdEMAMix with alpha = 0, beta3 = 0 or a negative alpha.
The 32-bit path and the 8-bit path each run these cases against the oracle
for several steps, on a tensor of several tiles with a ragged tail, with
mixed gradients (zeros included) and skip_zeros off and on.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import gpu_helpers as H
from tests.test_gpu_8bit import _assert_same, _gpu_run, _oracle_run

pytestmark = pytest.mark.gpu

N = 4099
STEPS = (1, 2, 3, 1_000_000)

EDGES = {
    "beta 0": dict(beta1=0.0, beta2=0.0, beta3=0.0),
    "largest betas": dict(beta1=1.0 - 2.0 ** -24, beta2=1.0 - 2.0 ** -24, beta3=1.0 - 2.0 ** -24),
    "eps 0": dict(eps=0.0),
    "lr 0 with decay": dict(lr=0.0, weight_decay=0.5),
    "decay factor -1": dict(lr=0.5, weight_decay=4.0),
    "alpha 0, beta3 0": dict(alpha=0.0, beta3=0.0),
    "negative alpha": dict(alpha=-2.0),
}


def _hp(edge, skip):
    base = dict(lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8, weight_decay=0.01,
                skip_zeros=skip)
    base.update(EDGES[edge])
    return O.HParams(**base)


@pytest.fixture(scope="module")
def orc():
    return O.load()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return H.lib()


def _inputs(kind, storage, edge):
    """Parameters U(-1,1); mixed gradients with +0 at every 7th element and
    -0 at every 11th from the 3rd (so eps = 0 meets 0/0 and skip_zeros has
    work)."""
    key = (list(H.KIND).index(kind), H.DT[storage], list(EDGES).index(edge))
    p0 = W.params(N, storage, W.rng(5, 0, *key))
    gs = []
    for t in range(len(STEPS)):
        g = W.grads(N, "mixed", storage, W.rng(5, 1, *key, t))
        g[::7] = 0
        g[3::11] = np.float32(-0.0) if g.dtype == np.float32 else 0x8000
        gs.append(g)
    return p0, gs


@pytest.mark.parametrize("kind", ["adam", "ademamix"])
@pytest.mark.parametrize("storage", ["fp32", "bf16"])
@pytest.mark.parametrize("edge", list(EDGES))
def test_32bit_edges(orc, L, kind, storage, edge):
    for skip in (False, True):
        hp = _hp(edge, skip)
        p0, gs = _inputs(kind, storage, edge)
        k = 2 if kind == "ademamix" else 1
        P, G = H.to_dev(p0, storage), torch.empty(N, dtype=W.STORAGE_TORCH[storage], device="cuda")
        S1, S2 = torch.zeros(k * N, device="cuda"), torch.zeros(N, device="cuda")
        p, (s1, s2) = p0.copy(), W.zero_states(N, kind)
        for t, g in zip(STEPS, gs):
            G.copy_(W.to_torch(g, storage, "cuda"))
            assert H.raw_update(L, kind, storage, P, G, S1, S2, N, hp, t, H.stream_handle()) == 0, \
                H.last_error(L)
            orc.update_f32(H.KIND[kind], H.DT[storage], p, g.copy(), s1, s2, hp, t)
        torch.cuda.synchronize()
        what = f"{kind} {storage} {edge} skip={skip}"
        H.assert_parity(W.from_torch(P), p, storage, "p " + what)
        H.assert_parity(W.from_torch(S1), s1, "fp32", "s1 " + what)
        H.assert_parity(W.from_torch(S2), s2, "fp32", "s2 " + what)


@pytest.mark.parametrize("kind", ["adam", "ademamix"])
@pytest.mark.parametrize("edge", list(EDGES))
def test_8bit_edges(orc, L, kind, edge):
    """The same edges with 8-bit block-wise states (bf16 storage): the step
    numbers are 1..4 here (the 8-bit helpers number steps consecutively)."""
    for skip in (False, True):
        hp = _hp(edge, skip)
        p0, gs = _inputs(kind, "bf16", edge)
        got = _gpu_run(L, kind, "bf16", p0, gs, hp)
        ref = _oracle_run(orc, kind, "bf16", p0, gs, hp)
        _assert_same(got, ref, "bf16", f"{kind} {edge} skip={skip}")
