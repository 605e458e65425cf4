"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function takes a loaded ``oracle.Oracle`` and raises
``AssertionError`` when the oracle disagrees with what the mathematics, the
IEEE definitions or an independent library routine fix.  The regular suite
runs every pin against the oracle (all must pass); the planted-mistake suite
runs them against copies of the oracle with one known mistake compiled in
(at least one must fail for each).

``INDEPENDENT`` pins check the formulas without retyping them (closed forms,
invariants, torch's own Adam/AdamW, IEEE conversions).  The exact-emulation
pin retypes the operation sequence and pins only its rounding.

Formulas are the textbook ones (Kingma & Ba 2015 Alg. 1; Loshchilov & Hutter
2019 Alg. 2; Pagliardini, Ablin & Grangier 2024 Alg. 1); the page
"Investigate a 256-thread SM103 path for small 32-bit optimizer tensors"
names the kinds and storage types (section "Correctness oracle") and prints
no formula.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import torch

import oracle as O
from tests import exact_fp32 as X
from workloads import cast_storage, rng

HP_CFG1 = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def _run_f32(orc, kind, dtype, p, grads_per_step, hp, steps, s1=None, s2=None):
    n = p.size
    p = p.copy()
    if s1 is None:
        s1 = np.zeros((2 if kind & 0xff == O.ADEMAMIX else 1) * n, np.float32)
        s2 = np.zeros(n, np.float32)
    for t in range(1, steps + 1):
        orc.update_f32(kind, dtype, p, grads_per_step(t), s1, s2, hp, t)
    return p, s1, s2


def _run_f64(orc, kind, p0, g, hp, steps):
    n = p0.size
    p = p0.astype(np.float64).copy()
    s1 = np.zeros((2 if kind & 0xff == O.ADEMAMIX else 1) * n)
    s2 = np.zeros(n)
    gg = g.astype(np.float64)
    out = []
    for t in range(1, steps + 1):
        orc.update_f64(kind, p, gg, s1, s2, hp, t)
        out.append((p.copy(), s1.copy(), s2.copy()))
    return out


# --------------------------------------------------------------- closed form

def pin_closed_form_f64(orc):
    """Constant gradient g, zero initial states.  Exactly
    m_t = (1 - b1^t) g and v_t = (1 - b2^t) g^2, so the bias-corrected
    moments are g and g^2 and every step moves p by u = lr g / (|g| + eps)
    after the decay d = 1 - lr wd of the old p:
        p_t = d^t p0 - u (1 - d^t) / (1 - d)           (p_t = p0 - t u at wd = 0)
    AdEMAMix: the slow EMA is m2_k = (1 - b3^k) g (not bias-corrected) and
        p_t = d^t p0 - sum_k d^(t-k) lr g (1 + alpha (1 - b3^k)) / (|g| + eps)."""
    g = np.array([1.0, -0.5, 3e-3, -2.5e-6, 7.0], np.float64)
    p0 = np.array([0.5, -0.25, 0.125, 0.9, -0.75], np.float64)
    T = 1000
    for kind in (O.ADAM, O.ADEMAMIX):
        for wd in (0.0, 0.1):
            hp = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0,
                           eps=1e-8, weight_decay=wd)
            traj = _run_f64(orc, kind, p0, g, hp, T)
            d = 1.0 - hp.lr * wd
            acc = p0.copy()
            for t in range(1, T + 1):
                coef = 1.0 + (hp.alpha * (1.0 - hp.beta3 ** t) if kind == O.ADEMAMIX else 0.0)
                acc = acc * d - hp.lr * g * coef / (np.abs(g) + hp.eps)
                if t in (1, 2, 10, 100, 1000):
                    p, s1, s2 = traj[t - 1]
                    n = g.size
                    m_ref = (1.0 - hp.beta1 ** t) * g
                    v_ref = (1.0 - hp.beta2 ** t) * g * g
                    scale = np.abs(p0) + t * hp.lr * (1 + hp.alpha)
                    assert np.all(np.abs(p - acc) <= 1e-12 * scale), (kind, wd, t, p, acc)
                    assert np.allclose(s1[:n], m_ref, rtol=1e-12, atol=0), (kind, wd, t, "m")
                    assert np.allclose(s2, v_ref, rtol=1e-12, atol=0), (kind, wd, t, "v")
                    if kind == O.ADEMAMIX:
                        m2_ref = (1.0 - hp.beta3 ** t) * g
                        assert np.allclose(s1[n:], m2_ref, rtol=1e-12, atol=0), (wd, t, "m2")
            if wd == 0.0 and kind == O.ADAM:   # the plain form of the sum
                p, _, _ = traj[T - 1]
                u = hp.lr * g / (np.abs(g) + hp.eps)
                assert np.all(np.abs(p - (p0 - T * u)) <= 1e-12 * (np.abs(p0) + T * hp.lr))


def pin_f32_tracks_f64(orc):
    """The binary32 instantiation follows the same formulas as the binary64
    one: over 10 steps of random gradients its parameters stay within a
    bound set by binary32 rounding (1e-5 lr per step), far below the effect
    of any dropped or misplaced term at lr = 1e-2, wd = 0.1 (decaying after
    instead of before the update alone moves p by lr^2 wd |u| = 1e-5 per
    step)."""
    n, T = 257, 10
    g0 = rng(7, 1)
    p0 = g0.uniform(-1, 1, n).astype(np.float32)
    gs = [g0.standard_normal(n).astype(np.float32) for _ in range(T)]
    for kind in (O.ADAM, O.ADEMAMIX):
        hp = O.HParams(lr=1e-2, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0,
                       eps=1e-8, weight_decay=0.1)
        # the binary64 run gets the binary32 values of the hyperparameters
        hp64 = O.HParams(**{k: float(np.float32(v)) if isinstance(v, float) else v
                            for k, v in hp.__dict__.items()})
        p32, s1_32, s2_32 = _run_f32(orc, kind, O.F32, p0, lambda t: gs[t - 1], hp, T)
        p64 = p0.astype(np.float64)
        s1 = np.zeros((2 if kind == O.ADEMAMIX else 1) * n)
        s2 = np.zeros(n)
        for t in range(1, T + 1):
            orc.update_f64(kind, p64, gs[t - 1].astype(np.float64), s1, s2, hp64, t)
        assert np.max(np.abs(p32 - p64)) <= 1e-5 * hp.lr * T, (kind, np.max(np.abs(p32 - p64)))
        assert np.allclose(s2_32, s2, rtol=1e-6, atol=0), kind
        assert np.allclose(s1_32, s1, rtol=1e-6, atol=1e-7), kind


def pin_first_step_by_hand(orc):
    """The first step from zero states, worked by hand for one element:
    lr 1e-3, b1 0.9, b2 0.999, eps 1e-8, wd 0.01, p0 = 0.5, g = 0.25 gives
    m1 = 0.1 * 0.25 = 0.025, v1 = 0.001 * 0.0625 = 6.25e-5, m^ = 0.25,
    v^ = 0.0625, u = 0.25 / (0.25 + 1e-8) and
    p1 = 0.5 * (1 - 1e-5) - 1e-3 * u = 0.49899500004.
    A second step with g = -0.125: m2 = 0.0225 - 0.0125 = 0.01,
    v2 = 0.999 * 6.25e-5 + 0.001 * 0.015625 = 7.80625e-5, m^ = 0.01 / 0.19,
    v^ = 7.80625e-5 / 0.001999, p2 = p1 (1 - 1e-5) - 1e-3 m^ / (sqrt(v^) + 1e-8)
    = 0.4987236...  The binary32 values must agree to binary32 precision
    (the decimal hyperparameters are not exact in binary32, which moves
    1 - b2 by 1.3e-5 relative; the bound allows for that), and bitwise to
    the exact emulation of the binary32 operation sequence, for AdamW and
    for AdEMAMix."""
    hp = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    p = np.array([0.5], np.float32)
    s1 = np.zeros(1, np.float32)
    s2 = np.zeros(1, np.float32)
    orc.update_f32(O.ADAM, O.F32, p, np.array([0.25], np.float32), s1, s2, hp, 1)
    p1 = 0.5 * (1 - 1e-5) - 1e-3 * 0.25 / (0.25 + 1e-8)
    assert abs(p[0] - p1) <= 1e-7, p[0]
    assert abs(s1[0] - 0.025) <= 1e-8, s1[0]
    assert abs(s2[0] - 6.25e-5) <= 6.25e-5 * 2e-5, s2[0]
    orc.update_f32(O.ADAM, O.F32, p, np.array([-0.125], np.float32), s1, s2, hp, 2)
    mh = 0.01 / 0.19
    vh = 7.80625e-5 / (1 - 0.999 ** 2)
    p2 = p1 * (1 - 1e-5) - 1e-3 * mh / (math.sqrt(vh) + 1e-8)
    assert abs(s1[0] - 0.01) <= 1e-8, s1[0]
    assert abs(s2[0] - 7.80625e-5) <= 7.80625e-5 * 2e-5, s2[0]
    assert abs(p[0] - p2) <= 1e-7, (p[0], p2)
    # the same two steps, and AdEMAMix's (beta3 0.9999, alpha 5), bitwise
    # against the exact-rational emulation of each rounded operation
    # (p = 0x3eff7c46 then 0x3eff58b5 for AdamW, 0x3eff7c35 then 0x3eff589a
    # for AdEMAMix)
    hp2 = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8,
                    weight_decay=0.01)
    gsteps = [np.array([0.25], np.float32), np.array([-0.125], np.float32)]
    for kind_name, kind in (("adam", O.ADAM), ("ademamix", O.ADEMAMIX)):
        _emulate_and_compare(orc, kind_name, kind, "fp32", O.F32, np.array([0.5], np.float32),
                             gsteps, hp2, 2)


# ------------------------------------------------------------- library routine

def pin_torch_adam(orc):
    """Adam (wd 0) and AdamW against torch.optim on the CPU in fp32, with
    dyadic hyperparameters so that both sides start from the same exact
    constants.  torch arranges the arithmetic differently (lerp for m,
    sqrt(v)/sqrt(bc2)), so the comparison has a tolerance: v within 8 ulp,
    m within 1e-6 of max|g| (lerp cancels differently near zero crossings).  p: within 2e-6 relative plus
    1e-6 lr absolute (near zero crossings torch's rounding of the step
    differs by a few 1e-7 of lr)."""
    n, T = 4096, 10
    for cls, wd in ((torch.optim.Adam, 0.0), (torch.optim.AdamW, 2.0 ** -7)):
        hp = O.HParams(lr=2.0 ** -10, beta1=0.875, beta2=1 - 2.0 ** -10, eps=2.0 ** -27,
                       weight_decay=wd)
        gen = rng(11, int(wd > 0))
        p0 = gen.uniform(-1, 1, n).astype(np.float32)
        gs = [gen.standard_normal(n).astype(np.float32) for _ in range(T)]
        p, s1, s2 = _run_f32(orc, O.ADAM, O.F32, p0, lambda t: gs[t - 1], hp, T)

        tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
        opt = cls([tp], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps, weight_decay=wd,
                  foreach=False)
        for t in range(T):
            tp.grad = torch.from_numpy(gs[t].copy())
            opt.step()
        st = opt.state[tp]
        tp_ = tp.detach().numpy()
        m_ = st["exp_avg"].numpy()
        v_ = st["exp_avg_sq"].numpy()

        def ulps(a, b):
            ia = a.view(np.int32).astype(np.int64)
            ib = b.view(np.int32).astype(np.int64)
            ia = np.where(ia < 0, -(ia & 0x7fffffff), ia)
            ib = np.where(ib < 0, -(ib & 0x7fffffff), ib)
            return np.abs(ia - ib)

        err = np.abs(p - tp_)
        assert np.all(err <= 2e-6 * np.abs(tp_) + 1e-6 * hp.lr), (cls.__name__, err.max())
        assert np.max(ulps(s2, v_)) <= 8, (cls.__name__, np.max(ulps(s2, v_)))
        gmax = max(float(np.max(np.abs(x))) for x in gs)
        assert np.max(np.abs(s1 - m_)) <= 1e-6 * gmax, (cls.__name__, np.max(np.abs(s1 - m_)))


# ---------------------------------------------------------------- invariants

def pin_zero_gradient(orc):
    """Zero gradient.  wd = 0: p is bitwise unchanged and the states stay +0.
    wd > 0, skip_zeros off: p follows p <- fl32(p * d) with
    d = fl32(1 - lr wd) bitwise.  skip_zeros on: p and states are bitwise
    unchanged for any wd, also for -0 gradients."""
    n, T = 64, 5
    p0 = rng(3, 0).uniform(-1, 1, n).astype(np.float32)
    for dtype in (O.F32, O.F16, O.BF16):
        ps = p0 if dtype == O.F32 else cast_storage(p0, {O.F16: "fp16", O.BF16: "bf16"}[dtype])
        zeros = np.zeros(n, np.float32) if dtype == O.F32 else np.zeros(n, np.uint16)
        negz = (np.full(n, -0.0, np.float32) if dtype == O.F32
                else np.full(n, 0x8000, np.uint16))
        for kind in (O.ADAM, O.ADEMAMIX):
            hp = O.HParams(weight_decay=0.0)
            p, s1, s2 = _run_f32(orc, kind, dtype, ps, lambda t: zeros, hp, T)
            assert np.array_equal(p.view(np.uint8), ps.view(np.uint8)), (kind, dtype)
            assert not np.any(s1.view(np.uint32)) and not np.any(s2.view(np.uint32)), (kind, dtype)
            for grad in (zeros, negz):
                hp = O.HParams(weight_decay=0.5, lr=0.01, skip_zeros=True)
                p, s1, s2 = _run_f32(orc, kind, dtype, ps, lambda t: grad, hp, T)
                assert np.array_equal(p.view(np.uint8), ps.view(np.uint8)), (kind, dtype, "skip")
                assert not np.any(s1.view(np.uint32)) and not np.any(s2.view(np.uint32))
            if dtype == O.F32:
                hp = O.HParams(weight_decay=0.5, lr=0.01)
                p, _, _ = _run_f32(orc, kind, dtype, ps, lambda t: zeros, hp, T)
                d = np.float32(1.0 - 0.01 * float(np.float32(0.5)))
                ref = p0.copy()
                lr32 = np.float32(0.01)
                for _ in range(T):    # m = v = 0: u = 0 / eps = 0, so p' = p d - lr 0
                    ref = (ref * d) - (lr32 * np.float32(0.0))
                assert np.array_equal(p.view(np.uint32), ref.view(np.uint32)), kind


def pin_ademamix_reduces_to_adam(orc):
    """AdEMAMix with alpha = 0 adds only alpha * m2 = 0 to the direction, so
    p, the fast EMA and v equal Adam's bitwise.  With beta3 = beta1 the slow
    EMA goes through the same operations as the fast one and equals it
    bitwise."""
    n, T = 300, 10
    gen = rng(5, 0)
    for dtype, name in ((O.F32, "fp32"), (O.F16, "fp16"), (O.BF16, "bf16")):
        p0 = cast_storage(gen.uniform(-1, 1, n).astype(np.float32), name)
        gs = [cast_storage(gen.standard_normal(n).astype(np.float32), name) for _ in range(T)]
        hp = O.HParams(alpha=0.0, weight_decay=0.01)
        pa, s1a, s2a = _run_f32(orc, O.ADAM, dtype, p0, lambda t: gs[t - 1], hp, T)
        pm, s1m, s2m = _run_f32(orc, O.ADEMAMIX, dtype, p0, lambda t: gs[t - 1], hp, T)
        assert np.array_equal(pa.view(np.uint8), pm.view(np.uint8)), name
        assert np.array_equal(s1a, s1m[:n]) and np.array_equal(s2a, s2m), name
        hp = O.HParams(beta3=0.9, beta1=0.9, weight_decay=0.01)
        _, s1m, _ = _run_f32(orc, O.ADEMAMIX, dtype, p0, lambda t: gs[t - 1], hp, T)
        assert np.array_equal(s1m[:n].view(np.uint32), s1m[n:].view(np.uint32)), name


def pin_element_independence(orc):
    """Each element is updated on its own: element i of an n = 4097 run
    equals a run of that element alone (n = 1), with its fast EMA at
    state1[i], its slow EMA at state1[n + i] and v at state2[i]; permuting
    the inputs permutes the outputs.  The binary32 and 8-thread runs are
    bitwise equal to the 1-thread run."""
    n, T = 4097, 3
    gen = rng(9, 0)
    for kind in (O.ADAM, O.ADEMAMIX):
        for dtype, name in ((O.F32, "fp32"), (O.BF16, "bf16")):
            p0 = cast_storage(gen.uniform(-1, 1, n).astype(np.float32), name)
            gs = [cast_storage(gen.standard_normal(n).astype(np.float32), name) for _ in range(T)]
            hp = O.HParams(weight_decay=0.01)
            p, s1, s2 = _run_f32(orc, kind, dtype, p0, lambda t: gs[t - 1], hp, T)
            for i in (0, 1, 2048, 4095, 4096):
                pi, s1i, s2i = _run_f32(orc, kind, dtype, p0[i:i + 1],
                                        lambda t: gs[t - 1][i:i + 1], hp, T)
                assert pi.view(np.uint8).tobytes() == p[i:i + 1].view(np.uint8).tobytes(), (kind, name, i)
                assert s1i[0] == s1[i] and s2i[0] == s2[i], (kind, name, i)
                if kind == O.ADEMAMIX:
                    assert s1i[1] == s1[n + i], (name, i)
            perm = gen.permutation(n)
            pp, s1p, s2p = _run_f32(orc, kind, dtype, p0[perm], lambda t: gs[t - 1][perm], hp, T)
            assert np.array_equal(pp.view(np.uint8), p[perm].view(np.uint8)), (kind, name)
            assert np.array_equal(s2p, s2[perm])
            if kind == O.ADEMAMIX:
                assert np.array_equal(s1p[n:], s1[n:][perm])
            # threads do not change the result
            p8 = p0.copy()
            s18 = np.zeros_like(s1)
            s28 = np.zeros_like(s2)
            for t in range(1, T + 1):
                orc.update_f32(kind, dtype, p8, gs[t - 1], s18, s28, hp, t, nthreads=8)
            assert np.array_equal(p8.view(np.uint8), p.view(np.uint8))
            assert np.array_equal(s18, s1) and np.array_equal(s28, s2)


def pin_grad_unchanged(orc):
    """The gradient is only read (page section "Correctness oracle")."""
    n = 1000
    gen = rng(13, 0)
    for kind in (O.ADAM, O.ADEMAMIX):
        for dtype, name in ((O.F32, "fp32"), (O.F16, "fp16"), (O.BF16, "bf16")):
            p = cast_storage(gen.uniform(-1, 1, n).astype(np.float32), name)
            g = cast_storage(gen.standard_normal(n).astype(np.float32), name)
            g0 = g.copy()
            s1 = np.zeros((2 if kind == O.ADEMAMIX else 1) * n, np.float32)
            s2 = np.zeros(n, np.float32)
            for t in (1, 2):
                orc.update_f32(kind, dtype, p, g, s1, s2, O.HParams(weight_decay=0.01), t)
            assert g.tobytes() == g0.tobytes(), (kind, name)


# --------------------------------------------------------------- conversions

def _f32_of_bits(u32: np.ndarray) -> np.ndarray:
    return u32.astype(np.uint32).view(np.float32)


def check_conversions(orc, bits: np.ndarray) -> None:
    """binary32 -> fp16 against numpy's IEEE float16 cast and binary32 ->
    bf16 against torch's bfloat16 cast (both round to nearest even), NaNs
    excluded (payloads are not part of the contract; NaN must stay NaN);
    and the exact widening back."""
    x = _f32_of_bits(bits)
    nan = np.isnan(x)
    h = orc.f32_to_storage(x, O.F16)
    h_ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(h[~nan], h_ref[~nan]), "fp16 rounding"
    assert np.all((h[nan] & 0x7c00) == 0x7c00) and np.all(h[nan] & 0x3ff), "fp16 NaN"
    b = orc.f32_to_storage(x, O.BF16)
    b_ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b[~nan], b_ref[~nan]), "bf16 rounding"
    assert np.all((b[nan] & 0x7f80) == 0x7f80) and np.all(b[nan] & 0x7f), "bf16 NaN"
    # widening is exact: fp16 via numpy, bf16 by definition (upper half)
    wh = orc.storage_to_f32(h[~nan], O.F16)
    assert np.array_equal(wh, h[~nan].view(np.float16).astype(np.float32)), "fp16 widen"
    wb = orc.storage_to_f32(b[~nan], O.BF16)
    assert np.array_equal(wb.view(np.uint32), b[~nan].astype(np.uint32) << 16), "bf16 widen"


def pin_conversions_sample(orc):
    """Storage conversions on every exponent and the rounding boundaries:
    all 2^16 bf16 patterns and all 2^16 fp16 patterns widened, plus binary32
    patterns at and around every half-way point, plus 2^20 random patterns."""
    allh = np.arange(1 << 16, dtype=np.uint32)
    b32 = allh << 16                                   # every bf16 value exactly
    mids = [b32 + 0x8000, b32 + 0x7fff, b32 + 0x8001, b32 + 1, b32 + 0xffff]
    f16v = np.arange(1 << 16, dtype=np.uint16).view(np.float16)
    f16v = f16v[np.isfinite(f16v)].astype(np.float32).view(np.uint32)
    f16mids = [f16v + 0x1000, f16v + 0xfff, f16v + 0x1001, f16v + 1, f16v - 1]
    rnd_bits = rng(17, 0).integers(0, 1 << 32, 1 << 20, dtype=np.uint64).astype(np.uint32)
    bits = np.concatenate([b32, *mids, f16v, *f16mids, rnd_bits]).astype(np.uint32)
    check_conversions(orc, bits)


# ----------------------------------------------------------- exact emulation

def pin_exact_emulation(orc):
    """Rounding: on a few elements, every kind, storage, gradient pattern,
    weight decay and skip_zeros setting, 10 steps of the oracle equal,
    bitwise, the same operation sequence with each operation rounded exactly
    once (tests/exact_fp32.py).  Patterns include gradients whose squares
    fall in the binary32 subnormal range."""
    n, T = 5, 10
    gen = rng(19, 0)
    pats = {
        "normal": lambda: gen.standard_normal(n),
        "mixed": lambda: np.where(gen.random(n) < 0.5, -1, 1) * 10.0 ** gen.uniform(-8, 3, n),
        "zero": lambda: np.array([0.0, -0.0, 0.0, 1.0, -0.0]),
        "tiny": lambda: np.where(gen.random(n) < 0.5, -1, 1) * 2.0 ** gen.uniform(-75, -60, n),
    }
    for kind_name, kind in (("adam", O.ADAM), ("ademamix", O.ADEMAMIX)):
        for sname, dtype in (("fp32", O.F32), ("fp16", O.F16), ("bf16", O.BF16)):
            for pat, draw in pats.items():
                if pat == "tiny" and sname == "fp16":
                    continue  # all round to zero in fp16: covered by "zero"
                for wd, skip in ((0.0, False), (0.01, True), (0.01, False)):
                    hp = O.HParams(weight_decay=wd, skip_zeros=skip)
                    p = cast_storage(gen.uniform(-1, 1, n).astype(np.float32), sname)
                    gsteps = [cast_storage(draw().astype(np.float32), sname) for _ in range(T)]
                    _emulate_and_compare(orc, kind_name, kind, sname, dtype, p, gsteps, hp, T)


def _storage_value(a: np.ndarray, sname: str) -> np.ndarray:
    """Storage array -> float64 values, decoded without the oracle."""
    if sname == "fp32":
        return a.astype(np.float64)
    if sname == "fp16":
        return a.view(np.float16).astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _emulate_and_compare(orc, kind_name, kind, sname, dtype, p, gsteps, hp, T, after=False):
    n = p.size
    pv = [X.F.of(float(x)) for x in _storage_value(p, sname)]
    m = [X.F.of(0.0) for _ in range(n)]
    v = [X.F.of(0.0) for _ in range(n)]
    m2 = [X.F.of(0.0) for _ in range(n)]
    b1, b2, b3 = (X.F.of(float(np.float32(b))) for b in (hp.beta1, hp.beta2, hp.beta3))
    al, ep, lr = (X.F.of(float(np.float32(x))) for x in (hp.alpha, hp.eps, hp.lr))
    f32 = lambda x: float(np.float32(x))
    po = p.copy()
    s1 = np.zeros((2 if kind == O.ADEMAMIX else 1) * n, np.float32)
    s2 = np.zeros(n, np.float32)
    karg = kind | (O.DECAY_AFTER if after else 0)
    for t in range(1, T + 1):
        sc = X.step_scalars(f32(hp.beta1), f32(hp.beta2), f32(hp.beta3), f32(hp.lr),
                            f32(hp.weight_decay), t)
        gv = _storage_value(gsteps[t - 1], sname)
        for i in range(n):
            g = X.F.of(float(gv[i]))
            pn, m[i], v[i], m2[i], wrote = X.element_step(
                kind_name, pv[i], g, m[i], v[i], m2[i], sc, b1, b2, b3, al, ep, lr,
                bool(hp.skip_zeros), after)
            if wrote:
                pv[i] = X.to_storage(pn, sname)
        orc.update_f32(karg, dtype, po, gsteps[t - 1], s1, s2, hp, t)
        got_p = _storage_value(po, sname)
        for i in range(n):
            ctx = (kind_name, sname, hp, t, i)
            assert pv[i].bits_equal(float(got_p[i])), ("p", ctx, float(pv[i]), got_p[i])
            assert m[i].bits_equal(float(s1[i])), ("m", ctx, float(m[i]), s1[i])
            assert v[i].bits_equal(float(s2[i])), ("v", ctx, float(v[i]), s2[i])
            if kind == O.ADEMAMIX:
                assert m2[i].bits_equal(float(s1[n + i])), ("m2", ctx, float(m2[i]), s1[n + i])


# ------------------------------------------------------ update-norm clipping

def pin_clip_reduces_to_plain(orc):
    """max_unorm = 0 (off) and a bound far above the update (s = 1) give the
    unclipped step bitwise, for every kind and storage, skip_zeros on."""
    n, T = 513, 4
    gen = rng(21, 0)
    for kind in (O.ADAM, O.ADEMAMIX):
        for dtype, name in ((O.F32, "fp32"), (O.F16, "fp16"), (O.BF16, "bf16")):
            p0 = cast_storage(gen.uniform(-1, 1, n).astype(np.float32), name)
            gs = [cast_storage(np.where(gen.random(n) < 0.2, 0.0, gen.standard_normal(n)).astype(np.float32), name)
                  for _ in range(T)]
            hp = O.HParams(weight_decay=0.01, skip_zeros=True)
            ref = _run_f32(orc, kind, dtype, p0, lambda t: gs[t - 1], hp, T)
            for bound in (0.0, 1e30):
                p = p0.copy()
                s1 = np.zeros_like(ref[1])
                s2 = np.zeros_like(ref[2])
                for t in range(1, T + 1):
                    sc = orc.update_f32_clip(kind, dtype, p, gs[t - 1], s1, s2, hp, t, bound)
                    assert sc == 1.0, (bound, sc)
                assert p.tobytes() == ref[0].tobytes(), (kind, name, bound)
                assert s1.tobytes() == ref[1].tobytes() and s2.tobytes() == ref[2].tobytes()


def pin_clip_closed_form_f64(orc):
    """Constant gradient g and zero initial states: every step's direction is
    u_i = g_i / (|g_i| + eps) exactly (Adam; AdEMAMix adds alpha (1 - b3^t) g_i
    over the same denominator), so the clipped trajectory is
        s_t = min(1, max_unorm ||p_(t-1)|| / ||u_t||),
        p_t = d p_(t-1) - lr s_t u_t,
    iterated here with numpy, independently of the oracle."""
    g = np.array([1.0, -0.5, 3e-3, -2.5e-6, 7.0, 0.25, -1.5, 0.0], np.float64)
    p0 = np.array([0.5, -0.25, 0.125, 0.9, -0.75, 0.3, 0.01, -0.6], np.float64)
    T = 200
    for kind in (O.ADAM, O.ADEMAMIX):
        for wd, bound in ((0.0, 2e-3), (0.1, 5e-4), (0.0, 10.0)):
            hp = O.HParams(lr=1e-2, beta1=0.9, beta2=0.999, beta3=0.99, alpha=5.0, eps=1e-8,
                           weight_decay=wd)
            p = p0.copy()
            s1 = np.zeros((2 if kind == O.ADEMAMIX else 1) * g.size)
            s2 = np.zeros(g.size)
            ref = p0.copy()
            d = 1.0 - hp.lr * wd
            for t in range(1, T + 1):
                sc = orc.update_f64_clip(kind, p, g, s1, s2, hp, t, bound)
                u = g / (np.abs(g) + hp.eps)
                if kind == O.ADEMAMIX:
                    u = u * (1.0 + hp.alpha * (1.0 - hp.beta3 ** t))
                s_ref = min(1.0, bound * np.linalg.norm(ref) / np.linalg.norm(u))
                ref = ref * d - hp.lr * s_ref * u
                assert abs(sc - s_ref) <= 1e-12 * s_ref, (kind, wd, bound, t, sc, s_ref)
                assert np.all(np.abs(p - ref) <= 1e-12 * (np.abs(p0) + t * hp.lr)), (kind, wd, bound, t)
            if bound < 1:
                assert s_ref < 1.0     # the clip was active


def pin_clip_realised_norm(orc):
    """binary32: when the clip is active the step moves p by fl32(lr s) u,
    whose norm is lr max_unorm ||p|| (here the step is ~1e5 times ulp(p), so
    the rounding of p adds ~1e-5 relative), the moments equal the unclipped
    step's bitwise, and skipped elements do not move."""
    n = 4097
    gen = rng(23, 0)
    for kind in (O.ADAM, O.ADEMAMIX):
        p0 = gen.uniform(-1, 1, n).astype(np.float32)
        g = np.where(gen.random(n) < 0.1, 0.0, gen.standard_normal(n)).astype(np.float32)
        hp = O.HParams(lr=0.1, weight_decay=0.0, skip_zeros=True)
        bound = 0.1
        p = p0.copy()
        s1, s2 = np.zeros((2 if kind == O.ADEMAMIX else 1) * n, np.float32), np.zeros(n, np.float32)
        sc = orc.update_f32_clip(kind, O.F32, p, g, s1, s2, hp, 1, bound)
        assert 0.0 < sc < 1.0
        step = (p0.astype(np.float64) - p.astype(np.float64))
        want = hp.lr * bound * np.linalg.norm(p0.astype(np.float64))
        assert abs(np.linalg.norm(step) - want) <= 1e-4 * want, (np.linalg.norm(step), want)
        assert np.all(p[g == 0] == p0[g == 0])
        pr = p0.copy()
        r1, r2 = np.zeros_like(s1), np.zeros_like(s2)
        orc.update_f32(kind, O.F32, pr, g, r1, r2, hp, 1)
        assert r1.tobytes() == s1.tobytes() and r2.tobytes() == s2.tobytes()


# ------------------------------------------------------------ one-state kinds

ONE_STATE_TORCH = {
    O.MOMENTUM: lambda prm, hp: torch.optim.SGD([prm], lr=hp.lr, momentum=hp.beta1, dampening=0.0,
                                                weight_decay=hp.weight_decay),
    O.RMSPROP: lambda prm, hp: torch.optim.RMSprop([prm], lr=hp.lr, alpha=hp.beta1, eps=hp.eps,
                                                   weight_decay=hp.weight_decay, momentum=0.0,
                                                   centered=False),
    O.ADAGRAD: lambda prm, hp: torch.optim.Adagrad([prm], lr=hp.lr, lr_decay=0.0, eps=hp.eps,
                                                   weight_decay=hp.weight_decay,
                                                   initial_accumulator_value=0.0),
}
ONE_STATE_KEY = {O.MOMENTUM: "momentum_buffer", O.RMSPROP: "square_avg", O.ADAGRAD: "sum"}


def pin_one_state_torch(orc):
    """Momentum SGD, RMSprop and Adagrad against torch.optim (CPU, fp32,
    foreach off) with dyadic hyperparameters, with and without weight
    decay, 10 steps.  torch arranges the arithmetic differently, so: p
    within 2e-6 relative plus 1e-6 lr, the state within 1e-6 relative plus
    an absolute floor of 1e-6 of its scale."""
    n, T = 2048, 10
    for kind, make in ONE_STATE_TORCH.items():
        for wd in (0.0, 2.0 ** -7):
            hp = O.HParams(lr=2.0 ** -10, beta1=0.875, eps=2.0 ** -27, weight_decay=wd)
            gen = rng(25, kind, int(wd > 0))
            p0 = gen.uniform(-1, 1, n).astype(np.float32)
            gs = [gen.standard_normal(n).astype(np.float32) for _ in range(T)]
            p = p0.copy()
            s = np.zeros(n, np.float32)
            for t in range(1, T + 1):
                orc.update1_f32(kind, O.F32, p, gs[t - 1], s, hp, t)
            prm = torch.nn.Parameter(torch.from_numpy(p0.copy()))
            opt = make(prm, hp)
            for param_group in opt.param_groups:
                param_group["foreach"] = False
            for t in range(T):
                prm.grad = torch.from_numpy(gs[t].copy())
                opt.step()
            tp = prm.detach().numpy()
            ts = opt.state[prm][ONE_STATE_KEY[kind]].numpy()
            err = np.abs(p - tp)
            assert np.all(err <= 2e-6 * np.abs(tp) + 1e-6 * hp.lr), (kind, wd, err.max())
            scale = float(np.max(np.abs(ts)))
            assert np.all(np.abs(s - ts) <= 1e-6 * np.abs(ts) + 1e-6 * scale), (kind, wd)


def pin_one_state_closed_form_f64(orc):
    """Constant gradient g, zero state, binary64:
    momentum (wd 0): m_t = g (1 - b^t)/(1 - b), p_t = p0 - lr sum_k m_k;
    RMSprop (wd 0):  v_t = (1 - b^t) g^2, p_t = p0 - lr sum_k g/(sqrt(1-b^k)|g| + eps);
    Adagrad (wd 0):  v_t = t g^2,         p_t = p0 - lr sum_k g/(sqrt(k)|g| + eps);
    Lion:            m_t = (1 - b2^t) g and c_t has the sign of g, so
                     p_t = d p_(t-1) - lr sign(g) with d = 1 - lr wd."""
    g = np.array([1.0, -0.5, 3e-3, -2.5e-6, 7.0], np.float64)
    p0 = np.array([0.5, -0.25, 0.125, 0.9, -0.75], np.float64)
    T = 300
    b, b2, eps, lr = 0.9, 0.99, 1e-8, 1e-3
    for kind in O.ONE_STATE:
        for wd in ((0.0, 0.1) if kind == O.LION else (0.0,)):
            hp = O.HParams(lr=lr, beta1=b, beta2=b2, eps=eps, weight_decay=wd)
            p = p0.copy()
            s = np.zeros_like(g)
            ref = p0.copy()
            for t in range(1, T + 1):
                orc.update1_f64(kind, p, g, s, hp, t)
                if kind == O.MOMENTUM:
                    m_ref = g * (1 - b ** t) / (1 - b)
                    ref = ref - lr * m_ref
                elif kind == O.RMSPROP:
                    m_ref = (1 - b ** t) * g * g
                    ref = ref - lr * g / (np.sqrt(1 - b ** t) * np.abs(g) + eps)
                elif kind == O.ADAGRAD:
                    m_ref = t * g * g
                    ref = ref - lr * g / (np.sqrt(t) * np.abs(g) + eps)
                else:
                    m_ref = (1 - b2 ** t) * g
                    ref = ref * (1 - lr * wd) - lr * np.sign(g)
                assert np.allclose(s, m_ref, rtol=1e-12, atol=0), (kind, wd, t)
                assert np.all(np.abs(p - ref) <= 1e-12 * (np.abs(p0) + t * lr * 10)), (kind, wd, t)


def pin_one_state_zero_gradient(orc):
    """Zero gradient, zero state: momentum, RMSprop and Adagrad leave p
    unchanged when wd = 0 (their step is 0 / (0 + eps) = 0 or lr * 0); Lion
    applies only the decay (sign(0) = 0); skip_zeros leaves everything
    untouched, also for -0 gradients and wd > 0."""
    n = 100
    p0 = rng(27, 0).uniform(-1, 1, n).astype(np.float32)
    for kind in O.ONE_STATE:
        for grad in (np.zeros(n, np.float32), np.full(n, -0.0, np.float32)):
            p = p0.copy()
            s = np.zeros(n, np.float32)
            orc.update1_f32(kind, O.F32, p, grad, s, O.HParams(weight_decay=0.0, lr=0.1), 1)
            assert p.tobytes() == p0.tobytes() and not np.any(s), kind
            p = p0.copy()
            orc.update1_f32(kind, O.F32, p, grad, s, O.HParams(weight_decay=0.5, lr=0.1,
                                                                skip_zeros=True), 3)
            assert p.tobytes() == p0.tobytes() and not np.any(s), kind
        p = p0.copy()
        s = np.zeros(n, np.float32)
        orc.update1_f32(O.LION, O.F32, p, np.zeros(n, np.float32), s,
                        O.HParams(weight_decay=0.5, lr=0.1), 1)
        d = np.float32(1.0 - 0.1 * float(np.float32(0.5)))
        assert p.tobytes() == ((p0 * d) - np.float32(0.1) * np.float32(0.0)).tobytes()


def pin_lion_by_hand(orc):
    """Lion's sign uses the interpolation c = b1 m + (1 - b1) g of the *old*
    moment; the moment is updated after (Chen et al. 2023, Algorithm 2).
    By hand, b1 0.9, b2 0.99, lr 0.1, p0 0.5: g1 = 1 gives c = 0.1 > 0,
    p1 = 0.4, m1 = 0.01; g2 = -0.085 gives c = 0.009 - 0.0085 = 0.0005 > 0,
    p2 = 0.3, m2 = 0.0099 - 0.00085 = 0.00905 (1 - b2 in binary32 is
    0.0099999905, hence the 1e-7 bound on m).  (Updating m first would give
    c = 0.00891 - 0.009265 < 0 and p2 = 0.5.)"""
    hp = O.HParams(lr=0.1, beta1=0.9, beta2=0.99, weight_decay=0.0)
    p = np.array([0.5], np.float32)
    m = np.zeros(1, np.float32)
    orc.update1_f32(O.LION, O.F32, p, np.array([1.0], np.float32), m, hp, 1)
    assert abs(p[0] - 0.4) <= 1e-7 and abs(m[0] - 0.01) <= 1e-7, (p, m)
    orc.update1_f32(O.LION, O.F32, p, np.array([-0.085], np.float32), m, hp, 2)
    assert abs(p[0] - 0.3) <= 1e-7 and abs(m[0] - 0.00905) <= 1e-7, (p, m)


def pin_exact_emulation_one_state(orc):
    """Rounding of the one-state kinds: 10 steps on a few elements, every
    storage, with and without weight decay and skip_zeros, bitwise equal to
    the same operations each rounded once (tests/exact_fp32.py)."""
    n, T = 5, 10
    gen = rng(29, 0)
    names = {O.MOMENTUM: "momentum", O.RMSPROP: "rmsprop", O.ADAGRAD: "adagrad", O.LION: "lion"}
    for kind, kname in names.items():
        for sname, dtype in (("fp32", O.F32), ("fp16", O.F16), ("bf16", O.BF16)):
            for wd, skip in ((0.0, False), (0.01, True)):
                hp = O.HParams(lr=1e-2, beta1=0.9, beta2=0.99, eps=1e-8, weight_decay=wd,
                               skip_zeros=skip)
                p = cast_storage(gen.uniform(-1, 1, n).astype(np.float32), sname)
                gsteps = [cast_storage(np.where(gen.random(n) < 0.2, 0.0, gen.standard_normal(n)).astype(np.float32), sname)
                          for _ in range(T)]
                f32 = lambda x: float(np.float32(x))
                pv = [X.F.of(float(x)) for x in _storage_value(p, sname)]
                mv = [X.F.of(0.0) for _ in range(n)]
                b1, b2, ep, w, lr = (X.F.of(f32(x)) for x in (hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.lr))
                decay = X.rnd(X.f64(1 - X.f64(Fraction(f32(hp.lr)) * Fraction(f32(hp.weight_decay)))), False)
                po = p.copy()
                so = np.zeros(n, np.float32)
                for t in range(1, T + 1):
                    gv = _storage_value(gsteps[t - 1], sname)
                    for i in range(n):
                        pn, mv[i], wrote = X.element_step1(kname, pv[i], X.F.of(float(gv[i])), mv[i],
                                                           b1, b2, ep, w, lr, decay, t == 1, skip)
                        if wrote:
                            pv[i] = X.to_storage(pn, sname)
                    orc.update1_f32(kind, dtype, po, gsteps[t - 1], so, hp, t)
                    got = _storage_value(po, sname)
                    for i in range(n):
                        ctx = (kname, sname, wd, skip, t, i)
                        assert pv[i].bits_equal(float(got[i])), ("p", ctx, float(pv[i]), got[i])
                        assert mv[i].bits_equal(float(so[i])), ("m", ctx, float(mv[i]), so[i])


# ------------------------------------------------------ weight-decay order

def pin_decay_after_by_hand(orc):
    """The two decay orders on one element where they differ grossly:
    lr 0.5, wd 1 (d = 0.5), p0 = 0.5, g = 0.25, zero states.  At step 1 the
    bias-corrected moments are g and g^2, so u = g/(|g| + eps) ~ 1 and
        old-parameter decay:    p*d - lr*u   = 0.25 - 0.5  ~ -0.25
        updated-parameter decay: (p - lr*u)*d = (0.5 - 0.5) * 0.5 ~ 0
    (both within the rounding of u, ~1e-7).  The same for Lion, whose u is
    sign(c) = 1 exactly: -0.25 and 0 exactly."""
    hp = O.HParams(lr=0.5, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=0.0, eps=1e-8,
                   weight_decay=1.0)
    for kind in (O.ADAM, O.ADEMAMIX):
        for after, want in ((False, -0.25), (True, 0.0)):
            p = np.array([0.5], np.float32)
            s1 = np.zeros(2 if kind == O.ADEMAMIX else 1, np.float32)
            s2 = np.zeros(1, np.float32)
            orc.update_f32(kind | (O.DECAY_AFTER if after else 0), O.F32, p,
                           np.array([0.25], np.float32), s1, s2, hp, 1)
            assert abs(float(p[0]) - want) <= 1e-6, (kind, after, p)
    for after, want in ((False, -0.25), (True, 0.0)):
        p = np.array([0.5], np.float32)
        m = np.zeros(1, np.float32)
        orc.update1_f32(O.LION | (O.DECAY_AFTER if after else 0), O.F32, p,
                        np.array([0.25], np.float32), m, hp, 1)
        assert float(p[0]) == want, (after, p)


def pin_decay_after_closed_form_f64(orc):
    """Constant gradient g, zero states, decay after the update: each step
    is p_t = (p_(t-1) - c_t) d with c_t = lr g (1 + alpha (1 - b3^t)) /
    (|g| + eps) (alpha = 0 for Adam), so
        p_t = d^t p0 - sum_k d^(t-k+1) c_k;
    Lion: c_t = lr sign(g).  Compared with the binary64 oracle at several
    steps (1e-12 relative)."""
    g = np.array([1.0, -0.5, 3e-3, -2.5e-6, 7.0], np.float64)
    p0 = np.array([0.5, -0.25, 0.125, 0.9, -0.75], np.float64)
    T = 300
    hp = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, beta3=0.9999, alpha=5.0, eps=1e-8,
                   weight_decay=0.1)
    d = 1.0 - hp.lr * hp.weight_decay
    for kind in (O.ADAM, O.ADEMAMIX, O.LION):
        p = p0.copy()
        n = g.size
        s1 = np.zeros((2 if kind == O.ADEMAMIX else 1) * n)
        s2 = np.zeros(n)
        for t in range(1, T + 1):
            if kind == O.LION:
                orc.update1_f64(kind | O.DECAY_AFTER, p, g, s1, hp, t)
            else:
                orc.update_f64(kind | O.DECAY_AFTER, p, g, s1, s2, hp, t)
            if t in (1, 2, 10, 300):
                ref = d ** t * p0
                for k in range(1, t + 1):
                    if kind == O.LION:
                        c = hp.lr * np.sign(g)
                    else:
                        coef = 1.0 + (hp.alpha * (1.0 - hp.beta3 ** k) if kind == O.ADEMAMIX else 0.0)
                        c = hp.lr * g * coef / (np.abs(g) + hp.eps)
                    ref = ref - d ** (t - k + 1) * c
                assert np.all(np.abs(p - ref) <= 1e-12 * (np.abs(p0) + t * hp.lr * 6)), (kind, t, p, ref)


def pin_decay_after_invariants(orc):
    """With wd = 0 (d = 1 exactly) both orders give the same bits for every
    decoupled kind; with wd > 0 they differ; the flag is refused by the L2
    kinds (their decay is part of the gradient, so it has no order)."""
    n, T = 257, 5
    gen = rng(31, 0)
    p0 = gen.uniform(-1, 1, n).astype(np.float32)
    gs = [gen.standard_normal(n).astype(np.float32) for _ in range(T)]
    for wd, same in ((0.0, True), (0.05, False)):
        hp = O.HParams(lr=0.01, weight_decay=wd)
        for kind in (O.ADAM, O.ADEMAMIX):
            a = _run_f32(orc, kind, O.F32, p0, lambda t: gs[t - 1], hp, T)
            b = _run_f32(orc, kind | O.DECAY_AFTER, O.F32, p0, lambda t: gs[t - 1], hp, T)
            assert (a[0].tobytes() == b[0].tobytes()) == same, (kind, wd)
            assert a[1].tobytes() == b[1].tobytes() and a[2].tobytes() == b[2].tobytes()
        res = []
        for karg in (O.LION, O.LION | O.DECAY_AFTER):
            p, m = p0.copy(), np.zeros(n, np.float32)
            for t in range(1, T + 1):
                orc.update1_f32(karg, O.F32, p, gs[t - 1], m, O.HParams(lr=0.01, weight_decay=wd), t)
            res.append((p, m))
        assert (res[0][0].tobytes() == res[1][0].tobytes()) == same, ("lion", wd)
        assert res[0][1].tobytes() == res[1][1].tobytes()
    for kind in (O.MOMENTUM, O.RMSPROP, O.ADAGRAD):
        try:
            orc.update1_f32(kind | O.DECAY_AFTER, O.F32, p0.copy(), gs[0], np.zeros(n, np.float32),
                            O.HParams(), 1)
        except ValueError:
            continue
        raise AssertionError(f"kind {kind} accepted the decay-order flag")


def pin_decay_after_clip(orc):
    """Clipping with the decay after the update: a bound far above the
    update (s = 1) gives the unclipped flagged step bitwise; an active
    bound moves p to (p - fl32(lr s) u) d, checked through the realised
    step norm at wd = 0.5, lr = 0.1 (d = 0.95)."""
    n, T = 513, 3
    gen = rng(33, 0)
    p0 = gen.uniform(-1, 1, n).astype(np.float32)
    gs = [np.where(gen.random(n) < 0.2, 0.0, gen.standard_normal(n)).astype(np.float32)
          for _ in range(T)]
    for kind in (O.ADAM, O.ADEMAMIX):
        karg = kind | O.DECAY_AFTER
        hp = O.HParams(weight_decay=0.01, skip_zeros=True)
        ref = _run_f32(orc, karg, O.F32, p0, lambda t: gs[t - 1], hp, T)
        p = p0.copy()
        s1, s2 = np.zeros_like(ref[1]), np.zeros_like(ref[2])
        for t in range(1, T + 1):
            assert orc.update_f32_clip(karg, O.F32, p, gs[t - 1], s1, s2, hp, t, 1e30) == 1.0
        assert p.tobytes() == ref[0].tobytes() and s1.tobytes() == ref[1].tobytes()
        hp = O.HParams(lr=0.1, weight_decay=0.5)
        bound = 0.1
        p = p0.copy()
        s1, s2 = np.zeros_like(ref[1]), np.zeros_like(ref[2])
        sc = orc.update_f32_clip(karg, O.F32, p, gs[0], s1, s2, hp, 1, bound)
        assert 0.0 < sc < 1.0
        d = float(np.float32(1.0 - 0.1 * float(np.float32(0.5))))
        step = p0.astype(np.float64) - p.astype(np.float64) / d
        want = hp.lr * bound * np.linalg.norm(p0.astype(np.float64))
        assert abs(np.linalg.norm(step) - want) <= 1e-4 * want, (np.linalg.norm(step), want)


def pin_exact_emulation_decay_after(orc):
    """Rounding of the decay-after order: a few elements, both two-state
    kinds and Lion, every storage, 6 steps, bitwise equal to the operations
    each rounded once."""
    n, T = 5, 6
    gen = rng(35, 0)
    for kind_name, kind in (("adam", O.ADAM), ("ademamix", O.ADEMAMIX)):
        for sname, dtype in (("fp32", O.F32), ("fp16", O.F16), ("bf16", O.BF16)):
            hp = O.HParams(lr=1e-2, weight_decay=0.1, skip_zeros=True)
            p = cast_storage(gen.uniform(-1, 1, n).astype(np.float32), sname)
            gsteps = [cast_storage(np.where(gen.random(n) < 0.2, 0.0, gen.standard_normal(n)).astype(np.float32), sname)
                      for _ in range(T)]
            _emulate_and_compare(orc, kind_name, kind, sname, dtype, p, gsteps, hp, T, after=True)
    f32 = lambda x: float(np.float32(x))
    for sname, dtype in (("fp32", O.F32), ("bf16", O.BF16)):
        hp = O.HParams(lr=1e-2, beta1=0.9, beta2=0.99, weight_decay=0.5)
        p = cast_storage(gen.uniform(-1, 1, n).astype(np.float32), sname)
        pv = [X.F.of(float(x)) for x in _storage_value(p, sname)]
        mv = [X.F.of(0.0) for _ in range(n)]
        b1, b2, ep, w, lr = (X.F.of(f32(x)) for x in (hp.beta1, hp.beta2, hp.eps, hp.weight_decay, hp.lr))
        decay = X.rnd(X.f64(1 - X.f64(Fraction(f32(hp.lr)) * Fraction(f32(hp.weight_decay)))), False)
        po, so = p.copy(), np.zeros(n, np.float32)
        for t in range(1, T + 1):
            gst = cast_storage(gen.standard_normal(n).astype(np.float32), sname)
            gv = _storage_value(gst, sname)
            for i in range(n):
                pn, mv[i], _ = X.element_step1("lion", pv[i], X.F.of(float(gv[i])), mv[i], b1, b2,
                                               ep, w, lr, decay, t == 1, False, after=True)
                pv[i] = X.to_storage(pn, sname)
            orc.update1_f32(O.LION | O.DECAY_AFTER, dtype, po, gst, so, hp, t)
            got = _storage_value(po, sname)
            for i in range(n):
                assert pv[i].bits_equal(float(got[i])), ("lion p", sname, t, i)
                assert mv[i].bits_equal(float(so[i])), ("lion m", sname, t, i)



# ------------------------------------------------- 8-bit block-wise states

QB = O.QBLOCK


def _blocks(n: int) -> int:
    return -(-n // QB)


def _zero_8bit(kind, n):
    k = 2 if kind == O.ADEMAMIX else 1
    return (np.zeros(k * n, np.uint8), np.zeros(n, np.uint8), np.zeros(k * _blocks(n), np.float32),
            np.zeros(_blocks(n), np.float32))


def _deq(orc, codes: np.ndarray, absmax: np.ndarray, signed: bool) -> np.ndarray:
    """Dequantized block states, decoded from the map's magnitudes and the
    code layout (sign bit, magnitude index), not with the oracle's decoder."""
    mags = orc.qmap(signed).astype(np.float32)
    c = codes.astype(np.int64)
    if signed:
        v = mags[c & 0x7f]
        v = np.where(c & 0x80, -v, v).astype(np.float32)
    else:
        v = mags[c]
    scale = np.repeat(absmax, QB)[:codes.size]
    return (v * scale).astype(np.float32)


def pin_qmap_structure(orc):
    """The 8-bit dynamic type: 128 signed / 256 unsigned magnitudes, strictly
    increasing from 0 to 1.  Decade E (values in (0.1, 1] x 10^-E) holds
    2^(P-1-E) values (P = 7 payload bits signed, 8 unsigned) that form an
    arithmetic progression with step 0.9 x 10^-E / 2^F starting half a step
    above 0.1 x 10^-E, except that the top value of decade 0 is 1."""
    for signed, P in ((True, 7), (False, 8)):
        mags = orc.qmap(signed).astype(np.float64)
        assert mags.size == 2 ** P and mags[0] == 0.0 and mags[-1] == 1.0
        assert np.all(np.diff(mags) > 0)
        for E in range(P):
            F = P - 1 - E
            lo, hi = 0.1 * 10.0 ** -E, 10.0 ** -E
            dec = mags[(mags > lo * (1 - 1e-6)) & (mags <= hi * (1 + 1e-6))]
            assert dec.size == 2 ** F, (signed, E, dec.size)
            step = 0.9 * 10.0 ** -E / 2 ** F
            want = lo + step * (np.arange(2 ** F) + 0.5)
            if E == 0:
                want[-1] = 1.0
            assert np.allclose(dec, want, rtol=1e-6, atol=0), (signed, E)


def _nearest_exact(mags: np.ndarray, value: float, absmax: float) -> int:
    """Index of the magnitude nearest to |value| / absmax in exact rational
    arithmetic, ties to the smaller magnitude: the argmin of the distances
    over the float64 estimate's neighbours (magnitudes are at least 1e-9
    apart relative, so the exact nearest is one of them)."""
    if not (absmax > 0.0) or math.isinf(absmax) or math.isnan(value):
        return 0
    rho = Fraction(abs(float(value))) / Fraction(float(absmax))
    j = int(np.searchsorted(mags, abs(value) / absmax))
    cand = [k for k in (j - 2, j - 1, j, j + 1) if 0 <= k < mags.size]
    return min(cand, key=lambda k: (abs(Fraction(float(mags[k])) - rho), k))


def pin_quantizer_nearest(orc):
    """The quantizer's code is the magnitude nearest to |value| / absmax in
    exact arithmetic, a ratio exactly halfway going to the smaller magnitude
    (brute force with rationals, not the oracle's midpoint count), for
    absmax values across the binary32 range (subnormal, near 1, near the
    largest) and values drawn uniformly, log-uniformly, on the rounded
    midpoints times absmax and their binary32 neighbours, and on exact
    ties; every magnitude times a power of two maps to itself; the code is
    monotone in the value; the sign bit is set for value < 0 only (-0 and
    NaN take code 0); an infinite absmax gives finite values code 0."""
    gen = rng(41, 0)
    f32 = np.float32
    absmaxes = [f32(1.0), f32(2.0 ** -149), f32(3 * 2.0 ** -140), f32(2.0 ** -130), f32(0.7),
                f32(3.4e38), f32(2.0 ** 100)] + list(
        (10.0 ** gen.uniform(-40, 38, 10)).astype(np.float32))
    for signed in (True, False):
        mags = orc.qmap(signed).astype(np.float64)
        mids = (mags[:-1] + mags[1:]) / 2
        for A in absmaxes:
            A = f32(A)
            vals = [gen.uniform(0, 1, 60) * A, 10.0 ** gen.uniform(-9, 0, 60) * A,
                    mids * float(A)]
            v = np.concatenate(vals).astype(np.float32)
            near = np.concatenate([np.nextafter(v[-mids.size:], f32(np.inf)),
                                   np.nextafter(v[-mids.size:], f32(0))])
            v = np.concatenate([v, near, [A, f32(0)]])
            v = v[np.abs(v) <= A]
            for x in v:
                want = _nearest_exact(mags, float(x), float(A))
                got = orc.qcode(signed, float(x), float(A))
                assert got == want, (signed, float(x), float(A), got, want)
                if signed and x > 0:
                    assert orc.qcode(True, -float(x), float(A)) == (want | 0x80), (float(x), float(A))
            prev = -1
            for x in np.sort(v[::7]):
                c = orc.qcode(signed, float(x), float(A))
                assert c >= prev, (signed, float(x), float(A))
                prev = c
        # exact ties: midpoints that binary32 holds, times powers of two
        ties = [k for k, m in enumerate(mids) if float(f32(m)) == m]
        assert ties, signed
        for k in ties:
            for e in (-100, -20, 0, 60):
                A = math.ldexp(1.0, e)
                x = float(f32(mids[k] * A))
                assert x == mids[k] * A
                assert orc.qcode(signed, x, A) == k, (signed, k, e)   # the smaller of the two
                assert orc.qcode(signed, float(np.nextafter(f32(x), f32(np.inf))), A) == k + 1
        for k, m in enumerate(mags):
            for e in (-90, -3, 0, 27):
                A = math.ldexp(1.0, e)
                assert orc.qcode(signed, float(f32(m)) * A, A) == k, (signed, k, e)
        for A in (1.0, 2.0 ** -100, float(f32(3.4e38))):
            assert orc.qcode(signed, -0.0, A) == 0 and orc.qcode(signed, float("nan"), A) == 0
        assert orc.qcode(signed, 0.0, 0.0) == 0
        assert orc.qcode(signed, -5.0, float("inf")) == (0x80 if signed else 0)
        assert orc.qcode(signed, float("inf"), float("inf")) == 0


def pin_qvalue_codes(orc):
    """The decoder, on all 256 codes of both types: a code's value is the
    magnitude its index selects in the map, negative when the signed type's
    bit 7 is set (decoded here from the map and the code layout, not with
    the oracle's decoder); values rise with the magnitude index; and the
    quantizer, whose decision-point count shares no code with the decoder,
    maps every value back to its own code (signed 0x80, minus zero, comes
    back as +0's code 0)."""
    for signed in (True, False):
        codes = np.arange(256, dtype=np.uint8)
        vals = np.array([orc.qvalue(signed, int(c)) for c in codes], np.float32)
        want = _deq(orc, codes, np.ones(1, np.float32), signed)
        assert np.array_equal(vals.view(np.uint32), want.view(np.uint32)), signed
        mags = vals[:128] if signed else vals
        assert mags[0] == 0.0 and mags[-1] == 1.0 and np.all(np.diff(mags) > 0), signed
        if signed:
            assert np.all(vals[129:] < 0) and np.array_equal(-vals[128:], vals[:128])
        for c in codes:
            back = orc.qcode(signed, float(vals[c]), 1.0)
            assert back == (0 if (signed and c == 0x80) else c), (signed, int(c), back)


def _uniform_block_grads(n, T, storage, gen):
    """Gradients whose magnitude is constant inside each 256-element block
    (drawn per block and step) with a fixed sign per element."""
    sign = np.where(gen.random(n) < 0.5, -1.0, 1.0)
    out = []
    for _ in range(T):
        mag = np.repeat(10.0 ** gen.uniform(-4, 0, _blocks(n)), QB)[:n]
        mag = cast_storage(mag.astype(np.float32), storage)
        mag = _storage_value(mag, storage)
        out.append(cast_storage((sign * mag).astype(np.float32), storage))
    return out


def pin_8bit_uniform_blocks_match_32bit(orc):
    """When every element of a block has the same gradient magnitude at each
    step (signs fixed per element), every state in the block has the same
    magnitude, normalises to +-1 and is stored exactly: the 8-bit trajectory
    then equals the 32-bit oracle's bitwise (parameters, dequantized
    moments, and absmax = |moment|), for both kinds, with weight decay, both
    decay orders."""
    n, T = 3 * QB + 77, 8
    gen = rng(43, 0)
    for kind in (O.ADAM, O.ADEMAMIX):
        for sname, dtype in (("fp32", O.F32), ("bf16", O.BF16)):
            for flag in (0, O.DECAY_AFTER):
                hp = O.HParams(lr=1e-2, weight_decay=0.05)
                p0 = cast_storage(gen.uniform(-1, 1, n).astype(np.float32), sname)
                gs = _uniform_block_grads(n, T, sname, gen)
                p8 = p0.copy()
                s1, s2, a1, a2 = _zero_8bit(kind, n)
                p32, r1, r2 = p0.copy(), *W_zero(kind, n)
                for t in range(1, T + 1):
                    orc.update_8bit_f32(kind | flag, dtype, p8, gs[t - 1], s1, s2, a1, a2, hp, t)
                    orc.update_f32(kind | flag, dtype, p32, gs[t - 1], r1, r2, hp, t)
                    ctx = (kind, sname, flag, t)
                    assert p8.tobytes() == p32.tobytes(), ctx
                    assert _deq(orc, s1[:n], a1[:_blocks(n)], True).tobytes() == r1[:n].tobytes(), ctx
                    assert _deq(orc, s2, a2, False).tobytes() == r2.tobytes(), ctx
                    if kind == O.ADEMAMIX:
                        assert _deq(orc, s1[n:], a1[_blocks(n):], True).tobytes() == r1[n:].tobytes(), ctx


def W_zero(kind, n):
    return np.zeros((2 if kind == O.ADEMAMIX else 1) * n, np.float32), np.zeros(n, np.float32)


def pin_8bit_first_step(orc):
    """From the zero state, step 1 moves the parameters exactly as the 32-bit
    step (the update uses the moments before they are quantized); the absmax
    of each block is max |fl32((1-b1) g)| and max fl32((1-b2) fl32(g g)),
    computed here with numpy; every stored state is a nearest quantization
    of its moment relative to that absmax (within half the largest gap of
    the type), and the block's largest moment is stored exactly."""
    n = 4 * QB + 5
    gen = rng(45, 0)
    for kind in (O.ADAM, O.ADEMAMIX):
        for sname, dtype in (("fp32", O.F32), ("fp16", O.F16), ("bf16", O.BF16)):
            for pat in ("normal", "mixed"):
                hp = O.HParams(lr=1e-3, weight_decay=0.01, skip_zeros=True)
                p0 = cast_storage(gen.uniform(-1, 1, n).astype(np.float32), sname)
                if pat == "normal":
                    g = np.where(gen.random(n) < 0.1, 0.0, gen.standard_normal(n))
                else:
                    g = np.where(gen.random(n) < 0.5, -1, 1) * 10.0 ** gen.uniform(-6, 2, n)
                g = cast_storage(g.astype(np.float32), sname)
                p8 = p0.copy()
                s1, s2, a1, a2 = _zero_8bit(kind, n)
                orc.update_8bit_f32(kind, dtype, p8, g, s1, s2, a1, a2, hp, 1)
                p32, r1, r2 = p0.copy(), *W_zero(kind, n)
                orc.update_f32(kind, dtype, p32, g, r1, r2, hp, 1)
                assert p8.tobytes() == p32.tobytes(), (kind, sname, pat)
                gv = _storage_value(g, sname).astype(np.float32)
                m_ref = (np.float32(1) - np.float32(hp.beta1)) * gv
                v_ref = (np.float32(1) - np.float32(hp.beta2)) * (gv * gv)
                pad = _blocks(n) * QB - n
                A1 = np.abs(np.r_[m_ref, np.zeros(pad, np.float32)]).reshape(-1, QB).max(axis=1)
                A2 = np.r_[v_ref, np.zeros(pad, np.float32)].reshape(-1, QB).max(axis=1)
                assert a1[:_blocks(n)].tobytes() == A1.astype(np.float32).tobytes(), (kind, sname, pat)
                assert a2.tobytes() == A2.astype(np.float32).tobytes()
                for signed, codes, absmax, ref in ((True, s1[:n], A1, m_ref), (False, s2, A2, v_ref)):
                    mags = orc.qmap(signed).astype(np.float64)
                    half = np.max(np.diff(mags)) / 2
                    deq = _deq(orc, codes, absmax.astype(np.float32), signed).astype(np.float64)
                    scale = np.repeat(absmax, QB)[:n].astype(np.float64)
                    assert np.all(np.abs(deq - ref) <= half * scale * (1 + 1e-6) + 1e-45), (kind, sname, pat)
                    top = np.abs(ref) == scale
                    assert np.all(deq[top] == ref[top]), "the block maximum is kept exactly"


def pin_8bit_zero_gradient(orc):
    """Zero gradients from the zero state: codes and absmax stay 0; with
    wd = 0 the parameters do not move, with wd > 0 they follow the 32-bit
    path (iterated decay) bitwise; skip_zeros leaves them untouched."""
    n = 2 * QB + 3
    p0 = rng(47, 0).uniform(-1, 1, n).astype(np.float32)
    g = np.zeros(n, np.float32)
    for kind in (O.ADAM, O.ADEMAMIX):
        for wd, skip in ((0.0, False), (0.1, False), (0.1, True)):
            hp = O.HParams(lr=0.1, weight_decay=wd, skip_zeros=skip)
            p8 = p0.copy()
            s1, s2, a1, a2 = _zero_8bit(kind, n)
            p32, r1, r2 = p0.copy(), *W_zero(kind, n)
            for t in range(1, 4):
                orc.update_8bit_f32(kind, O.F32, p8, g, s1, s2, a1, a2, hp, t)
                orc.update_f32(kind, O.F32, p32, g, r1, r2, hp, t)
            assert not s1.any() and not s2.any() and not a1.any() and not a2.any()
            assert p8.tobytes() == p32.tobytes(), (kind, wd, skip)
            if wd == 0.0 or skip:
                assert p8.tobytes() == p0.tobytes()


def pin_8bit_block_independence(orc):
    """A block's result depends on that block only: running each block as a
    tensor of its own (the partial last block too) gives the same bits, and
    permuting whole blocks permutes the results."""
    n, T = 3 * QB + 77, 4
    gen = rng(49, 0)
    for kind in (O.ADAM, O.ADEMAMIX):
        hp = O.HParams(lr=1e-2, weight_decay=0.01)
        p0 = gen.uniform(-1, 1, n).astype(np.float32)
        gs = [gen.standard_normal(n).astype(np.float32) for _ in range(T)]
        full = (p0.copy(), *_zero_8bit(kind, n))
        for t in range(1, T + 1):
            orc.update_8bit_f32(kind, O.F32, full[0], gs[t - 1], *full[1:], hp, t)
        nb = _blocks(n)
        for b in range(nb):
            lo, hi = b * QB, min(n, (b + 1) * QB)
            part = (p0[lo:hi].copy(), *_zero_8bit(kind, hi - lo))
            for t in range(1, T + 1):
                orc.update_8bit_f32(kind, O.F32, part[0], gs[t - 1][lo:hi].copy(), *part[1:], hp, t)
            assert part[0].tobytes() == full[0][lo:hi].tobytes(), (kind, b)
            assert part[1][:hi - lo].tobytes() == full[1][lo:hi].tobytes()
            assert part[2].tobytes() == full[2][lo:hi].tobytes()
            assert part[3][0] == full[3][b] and part[4][0] == full[4][b]
            if kind == O.ADEMAMIX:
                assert part[1][hi - lo:].tobytes() == full[1][n + lo:n + hi].tobytes()
                assert part[3][1] == full[3][nb + b]
        m = 3 * QB                                   # permute the three full blocks
        perm = [2, 0, 1]
        idx = np.concatenate([np.arange(b * QB, (b + 1) * QB) for b in perm])
        pp = (p0[:m][idx].copy(), *_zero_8bit(kind, m))
        for t in range(1, T + 1):
            orc.update_8bit_f32(kind, O.F32, pp[0], gs[t - 1][:m][idx].copy(), *pp[1:], hp, t)
        assert pp[0].tobytes() == full[0][:m][idx].tobytes()
        assert pp[2].tobytes() == full[2][:m][idx].tobytes()


def pin_8bit_tracks_32bit(orc):
    """Quantization error bound: the 8-bit and 32-bit moments obey the same
    recurrence m_t = b m_(t-1) + (1-b) g_t, except that the 8-bit one is
    requantized each step with an error of at most h A_t (h: half the largest
    gap of the type, A_t: the block's absmax at step t).  So
    |m8_t - m32_t| <= e_t with e_t = b e_(t-1) + h A_t, checked for every
    element over 20 steps of random gradients (1e-6 relative slack for the
    binary32 rounding of both paths)."""
    n, T = 2 * QB + 31, 20
    gen = rng(51, 0)
    hp = O.HParams(lr=1e-3, weight_decay=0.0)
    hs = np.max(np.diff(orc.qmap(True).astype(np.float64))) / 2
    hu = np.max(np.diff(orc.qmap(False).astype(np.float64))) / 2
    p0 = gen.uniform(-1, 1, n).astype(np.float32)
    p8 = p0.copy()
    s1, s2, a1, a2 = _zero_8bit(O.ADAM, n)
    p32, r1, r2 = p0.copy(), *W_zero(O.ADAM, n)
    e1 = np.zeros(n)
    e2 = np.zeros(n)
    for t in range(1, T + 1):
        g = gen.standard_normal(n).astype(np.float32)
        orc.update_8bit_f32(O.ADAM, O.F32, p8, g, s1, s2, a1, a2, hp, t)
        orc.update_f32(O.ADAM, O.F32, p32, g, r1, r2, hp, t)
        e1 = hp.beta1 * e1 + hs * np.repeat(a1, QB)[:n]
        e2 = hp.beta2 * e2 + hu * np.repeat(a2, QB)[:n]
        m8 = _deq(orc, s1, a1, True).astype(np.float64)
        v8 = _deq(orc, s2, a2, False).astype(np.float64)
        assert np.all(np.abs(m8 - r1) <= e1 * (1 + 1e-6) + 1e-6 * np.abs(r1)), t
        assert np.all(np.abs(v8 - r2) <= e2 * (1 + 1e-6) + 1e-6 * np.abs(r2)), t


INDEPENDENT = [pin_closed_form_f64, pin_f32_tracks_f64, pin_first_step_by_hand,
               pin_torch_adam, pin_zero_gradient, pin_ademamix_reduces_to_adam,
               pin_element_independence, pin_grad_unchanged, pin_conversions_sample,
               pin_clip_reduces_to_plain, pin_clip_closed_form_f64, pin_clip_realised_norm,
               pin_one_state_torch, pin_one_state_closed_form_f64, pin_one_state_zero_gradient,
               pin_lion_by_hand, pin_decay_after_by_hand, pin_decay_after_closed_form_f64,
               pin_decay_after_invariants, pin_decay_after_clip, pin_qmap_structure,
               pin_quantizer_nearest, pin_qvalue_codes, pin_8bit_uniform_blocks_match_32bit,
               pin_8bit_first_step,
               pin_8bit_zero_gradient, pin_8bit_block_independence, pin_8bit_tracks_32bit]
ALL = INDEPENDENT + [pin_exact_emulation, pin_exact_emulation_one_state,
                     pin_exact_emulation_decay_after]
