"""GPU parity on IEEE special values: NaN, +-inf, +-0, subnormals, values
whose square overflows or underflows, in gradients and parameters.

The update has no special handling for them (reading R13: IEEE propagation),
the 8-bit quantizer maps NaN to code 0 and passes NaN over in the block
maximum, and update-norm clipping treats a NaN or infinite norm as the
definition says (s = 1 unless max_unorm * ||p|| / ||u|| is a number below 1).
Every path must give the oracle's results element by element (a NaN equals
a NaN; payloads are not part of the contract).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

TWO = {"adam": O.ADAM, "ademamix": O.ADEMAMIX}
ONE = {"momentum": O.MOMENTUM, "rmsprop": O.RMSPROP, "adagrad": O.ADAGRAD, "lion": O.LION}
N = 4099


@pytest.fixture(scope="module")
def orc():
    return O.load()


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return H.lib()


def _specials(storage: str, n: int, seed: int, kind_of: str) -> np.ndarray:
    """Values of the storage type: mostly normal numbers, with every class of
    special value sprinkled in (a fixed set at the start, random positions
    after)."""
    gen = W.rng(5, seed, n)
    x = gen.standard_normal(n).astype(np.float32)
    if storage == "fp32":
        special = [0.0, -0.0, np.inf, -np.inf, np.nan, 1e-40, -1e-42, 1e30, -3e25, 1e-25, 3e38,
                   np.float32(1.17549435e-38)]
    elif storage == "fp16":
        special = [0.0, -0.0, np.inf, -np.inf, np.nan, 6e-8, -3e-6, 65504.0, -1000.0, 1e-4]
    else:
        special = [0.0, -0.0, np.inf, -np.inf, np.nan, 1e-39, -9e-40, 3e38, -1e30, 1e-25]
    special = np.array(special, np.float32)
    x[:special.size] = special
    pos = gen.integers(special.size, n, 200)
    x[pos] = special[gen.integers(0, special.size, 200)]
    if kind_of == "param":      # keep most parameters ordinary, but not all
        x = np.where(np.isin(np.arange(n), pos[:50]), x, gen.uniform(-1, 1, n)).astype(np.float32)
    return W.cast_storage(x, storage)


def _assert_nan_aware(got: np.ndarray, ref: np.ndarray, what: str):
    if got.dtype == np.float32:
        same = (got.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(got) & np.isnan(ref))
    else:
        same = got.view(np.uint8) == ref.view(np.uint8)
    assert same.all(), f"{what}: {int((~same).sum())} differ, first at {int(np.argmin(same))}"


@pytest.mark.parametrize("kind", list(TWO) + list(ONE))
@pytest.mark.parametrize("storage", ["fp32", "fp16", "bf16"])
def test_special_values_32bit(orc, L, kind, storage):
    """Direct call and plan, wd > 0, skip_zeros off and on, 3 steps."""
    from optimizer_update_amd import Plan
    one = kind in ONE
    code = ONE[kind] if one else TWO[kind]
    for skip in (False, True):
        hp = O.HParams(lr=1e-2, beta1=0.9, beta2=0.99 if kind == "lion" else 0.999, beta3=0.999,
                       alpha=2.0, eps=1e-8, weight_decay=0.05, skip_zeros=skip)
        p0 = _specials(storage, N, 1, "param")
        gs = [_specials(storage, N, 2 + t, "grad") for t in range(3)]
        k = 2 if kind == "ademamix" else 1
        # oracle
        pr = p0.copy()
        s1r = np.zeros(k * N, np.float32)
        s2r = None if one else np.zeros(N, np.float32)
        for t, g in enumerate(gs, start=1):
            if one:
                orc.update1_f32(code, H.DT[storage], pr, g.copy(), s1r, hp, t)
            else:
                orc.update_f32(code, H.DT[storage], pr, g.copy(), s1r, s2r, hp, t)
        for path in ("direct", "plan"):
            P = H.to_dev(p0, storage)
            G = torch.empty(N, dtype=W.STORAGE_TORCH[storage], device="cuda")
            S1 = torch.zeros(k * N, device="cuda")
            S2 = None if one else torch.zeros(N, device="cuda")
            plan = Plan(kind, [(P, G, S1, S2)]) if path == "plan" else None
            try:
                for t, g in enumerate(gs, start=1):
                    G.copy_(W.to_torch(g, storage, "cuda"))
                    if plan is not None:
                        plan.step(H.pkg_hp(hp), t)
                    else:
                        st = L.optimizer_update_32bit(code, H.DT[storage], P.data_ptr(), G.data_ptr(),
                                                      S1.data_ptr(), None if S2 is None else S2.data_ptr(),
                                                      N, hp.beta1, hp.beta2, hp.beta3, hp.alpha, hp.eps,
                                                      hp.weight_decay, t, hp.lr, int(skip),
                                                      H.stream_handle())
                        assert st == 0, H.last_error(L)
                torch.cuda.synchronize()
            finally:
                if plan is not None:
                    plan.close()
            what = f"{kind} {storage} skip={skip} {path}"
            H.assert_parity(W.from_torch(P), pr, storage, "p " + what)
            _assert_nan_aware(W.from_torch(S1), s1r, "state1 " + what)
            if S2 is not None:
                _assert_nan_aware(W.from_torch(S2), s2r, "state2 " + what)


@pytest.mark.parametrize("kind", list(TWO))
@pytest.mark.parametrize("storage", ["fp32", "bf16"])
def test_special_values_8bit(orc, L, kind, storage):
    """8-bit states: NaN and infinite moments pass through the block maximum
    and the quantizer as the definition says; codes, absmax and parameters
    equal the oracle's."""
    import optimizer_update_amd as ou
    for skip in (False, True):
        hp = O.HParams(lr=1e-2, weight_decay=0.05, skip_zeros=skip)
        p0 = _specials(storage, N, 11, "param")
        gs = [_specials(storage, N, 12 + t, "grad") for t in range(3)]
        ref = [p0.copy(), *(np.zeros(s, np.uint8) for s in ou.state8_sizes(kind, N)[:2]),
               *(np.zeros(s, np.float32) for s in ou.state8_sizes(kind, N)[2:])]
        for t, g in enumerate(gs, start=1):
            orc.update_8bit_f32(TWO[kind], H.DT[storage], ref[0], g.copy(), *ref[1:], hp, t)
        P = H.to_dev(p0, storage)
        G = torch.empty(N, dtype=W.STORAGE_TORCH[storage], device="cuda")
        sizes = ou.state8_sizes(kind, N)
        st = [torch.zeros(sizes[0], dtype=torch.uint8, device="cuda"),
              torch.zeros(sizes[1], dtype=torch.uint8, device="cuda"),
              torch.zeros(sizes[2], device="cuda"), torch.zeros(sizes[3], device="cuda")]
        for t, g in enumerate(gs, start=1):
            G.copy_(W.to_torch(g, storage, "cuda"))
            ou.optimizer_update_8bit_blockwise(kind, P, G, *st, step=t, lr=hp.lr,
                                               weight_decay=hp.weight_decay, skip_zeros=skip)
        torch.cuda.synchronize()
        what = f"8-bit {kind} {storage} skip={skip}"
        H.assert_parity(W.from_torch(P), ref[0], storage, "p " + what)
        for got, want, name in zip(st, ref[1:], ("codes1", "codes2", "absmax1", "absmax2")):
            _assert_nan_aware(got.cpu().numpy(), want, f"{name} {what}")


@pytest.mark.parametrize("kind", list(TWO))
def test_special_values_clip(orc, kind):
    """Update-norm clipping when the norms are NaN or infinite: the clip
    factor is the oracle's (1 for NaN, 0 for an infinite update norm) and
    the moments and parameters follow."""
    import optimizer_update_amd as ou
    hp = O.HParams(lr=1e-2, weight_decay=0.01)
    for case in ("nan", "inf", "finite"):
        p0 = W.params(N, "fp32", W.rng(5, 30, N))
        g = W.grads(N, "normal", "fp32", W.rng(5, 31, N))
        if case == "nan":
            g[17] = np.nan
        elif case == "inf":
            g[17] = np.inf
        pr = p0.copy()
        s1r, s2r = W.zero_states(N, kind)
        s_ref = orc.update_f32_clip(TWO[kind], O.F32, pr, g.copy(), s1r, s2r, hp, 1, 0.01)
        P = H.to_dev(p0, "fp32")
        G = H.to_dev(g, "fp32")
        S1 = torch.zeros(s1r.size, device="cuda")
        S2 = torch.zeros(N, device="cuda")
        ws = ou.optimizer_update_32bit_clip(kind, P, G, S1, S2, step=1, lr=hp.lr,
                                            weight_decay=hp.weight_decay, max_unorm=0.01)
        s_gpu = ou.clip_scale(ws)
        torch.cuda.synchronize()
        if case != "finite":
            assert s_gpu == s_ref, (case, s_gpu, s_ref)
        H.assert_parity(W.from_torch(P), pr, "fp32", f"clip {kind} {case} p", bitwise=case != "finite")
        _assert_nan_aware(W.from_torch(S1), s1r, f"clip {kind} {case} state1")
        _assert_nan_aware(W.from_torch(S2), s2r, f"clip {kind} {case} state2")
