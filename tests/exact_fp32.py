"""Exact-arithmetic emulation of binary32 for pinning the oracle's rounding.

Every operation is carried out on exact rationals (``fractions.Fraction``)
and then rounded once to the nearest binary32 value, ties to even, with
gradual underflow and IEEE signed zeros.  Square root is correctly rounded
through integer square roots.  Nothing here comes from the oracle or the HIP
library; it is the IEEE 754 definition of each operation written out, so a
per-element update run through it gives *the* correctly rounded result of a
stated operation sequence.

It is slow: use it for a handful of elements and steps only.
"""
from __future__ import annotations

import math
from fractions import Fraction


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while a < Fraction(2) ** e:
        e -= 1
    while a >= Fraction(2) ** (e + 1):
        e += 1
    return e


def _round_half_even(x: Fraction) -> int:
    fl = math.floor(x)
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


class Fmt:
    """A binary floating-point format: p significand bits (with the hidden
    bit), minimum normal exponent emin, overflow threshold 2^(emax+1)."""

    def __init__(self, p: int, emin: int, emax: int):
        self.p, self.emin, self.emax = p, emin, emax

    def round(self, a: Fraction) -> Fraction:
        """Round a > 0 to this format (RNE).  Raises OverflowError on overflow."""
        e = _floor_log2(a)
        q = max(e, self.emin) - (self.p - 1)
        r = _round_half_even(a / Fraction(2) ** q) * Fraction(2) ** q
        if r >= Fraction(2) ** (self.emax + 1):
            raise OverflowError("rounds to infinity")
        return r


BINARY32 = Fmt(24, -126, 127)
BINARY16 = Fmt(11, -14, 15)
BFLOAT16 = Fmt(8, -126, 127)


class F:
    """A binary32 value: an exact rational plus the sign bit (for zeros)."""

    __slots__ = ("v", "neg")

    def __init__(self, v: Fraction, neg: bool | None = None):
        self.v = v
        self.neg = (v < 0) if v != 0 else bool(neg)

    @staticmethod
    def of(x: float, fmt: Fmt = BINARY32) -> "F":
        """An exactly representable float (checked against ``fmt``)."""
        if not math.isfinite(x):
            raise ValueError("finite values only")
        f = F(Fraction(x), math.copysign(1.0, x) < 0)
        if f.v != 0 and fmt.round(abs(f.v)) != abs(f.v):
            raise ValueError(f"{x!r} is not representable")
        return f

    def __float__(self) -> float:
        x = float(self.v)
        return -0.0 if (x == 0 and self.neg) else x

    def bits_equal(self, x: float) -> bool:
        """True iff x is the same value with the same sign (zeros included)."""
        return float(self) == x and math.copysign(1.0, float(self)) == math.copysign(1.0, x)


def rnd(exact: Fraction, neg_if_zero: bool, fmt: Fmt = BINARY32) -> F:
    if exact == 0:
        return F(Fraction(0), neg_if_zero)
    r = fmt.round(abs(exact))
    if exact < 0:
        r = -r
    if r == 0:
        return F(r, exact < 0)            # underflow keeps the sign
    return F(r)


def add(a: F, b: F) -> F:
    s = a.v + b.v
    # exact zero sum: -0 only when both addends are -0 (round to nearest)
    return rnd(s, a.neg and b.neg if s == 0 else False)


def neg(a: F) -> F:
    return F(-a.v, not a.neg)


def sub(a: F, b: F) -> F:
    return add(a, neg(b))


def mul(a: F, b: F) -> F:
    return rnd(a.v * b.v, a.neg != b.neg)


def div(a: F, b: F) -> F:
    if b.v == 0:
        raise ZeroDivisionError
    return rnd(a.v / b.v, a.neg != b.neg)


def sqrt(a: F) -> F:
    """Correctly rounded binary32 square root (a >= 0; sqrt(-0) = -0)."""
    if a.v == 0:
        return F(Fraction(0), a.neg)
    if a.v < 0:
        raise ValueError("sqrt of a negative number")
    er = _floor_log2(a.v) // 2                     # floor(log2(sqrt(a)))
    q = max(er, BINARY32.emin) - (BINARY32.p - 1)
    n4 = 4 * a.v / Fraction(4) ** q                # 4 * (sqrt(a) / 2^q)^2
    h = math.isqrt(math.floor(n4))                 # floor(2 * sqrt(a) / 2^q)
    r = h // 2
    if h % 2 == 1:                                 # fractional part >= 1/2
        if Fraction(h * h) == n4:                  # exactly 1/2: tie to even
            r += r % 2
        else:
            r += 1
    return F(Fraction(r) * Fraction(2) ** q)


def to_storage(a: F, storage: str) -> F:
    """Round a binary32 value to the storage format (RNE)."""
    fmt = {"fp32": BINARY32, "fp16": BINARY16, "bf16": BFLOAT16}[storage]
    return rnd(a.v, a.neg, fmt)


def f64(x: Fraction) -> Fraction:
    """Round to binary64 (RNE); Python floats are binary64."""
    return Fraction(float(x))


def step_scalars(beta1: float, beta2: float, beta3: float, lr: float, wd: float,
                 step: int) -> dict[str, F]:
    """The per-step scalars of the stated operation sequence: the bias
    corrections fl32(1 - fl64(beta^t)) with beta^t from the platform libm
    (math.pow), the decay fl32(1 - fl64(lr * wd)), and 1 - beta in binary32."""
    one = F(Fraction(1))
    out = {}
    for name, beta in (("bc1", beta1), ("bc2", beta2)):
        pw = Fraction(math.pow(beta, float(step)))
        out[name] = rnd(f64(1 - pw), False)
    out["decay"] = rnd(f64(1 - f64(Fraction(lr) * Fraction(wd))), False)
    out["omb1"] = sub(one, F.of(beta1))
    out["omb2"] = sub(one, F.of(beta2))
    out["omb3"] = sub(one, F.of(beta3))
    return out


def element_step(kind: str, p: F, g: F, m: F, v: F, m2: F | None, sc: dict[str, F],
                 beta1: F, beta2: F, beta3: F, alpha: F, eps: F, lr: F,
                 skip_zeros: bool, after: bool = False) -> tuple[F, F, F, F | None, bool]:
    """One element of the update, operation by operation.  Returns
    (p, m, v, m2, written) with p still in binary32 (round it to storage
    afterwards); written is False when skip_zeros leaves the element alone.
    after: the decay multiplies the updated parameter, (p - lr u) d."""
    if skip_zeros and g.v == 0:
        return p, m, v, m2, False
    m = add(mul(beta1, m), mul(sc["omb1"], g))
    v = add(mul(beta2, v), mul(sc["omb2"], mul(g, g)))
    if kind == "ademamix":
        m2 = add(mul(beta3, m2), mul(sc["omb3"], g))
    mh = div(m, sc["bc1"])
    vh = div(v, sc["bc2"])
    den = add(sqrt(vh), eps)
    num = add(mh, mul(alpha, m2)) if kind == "ademamix" else mh
    u = div(num, den)
    if after:
        p = mul(sub(p, mul(lr, u)), sc["decay"])
    else:
        p = sub(mul(p, sc["decay"]), mul(lr, u))
    return p, m, v, m2, True


def element_step1(kind: str, p: F, g: F, m: F, beta1: F, beta2: F, eps: F, wd: F, lr: F,
                  decay: F, first: bool, skip_zeros: bool,
                  after: bool = False) -> tuple[F, F, bool]:
    """One element of a one-state kind (momentum, rmsprop, adagrad, lion),
    operation by operation; returns (p, m, written) with p in binary32."""
    if skip_zeros and g.v == 0:
        return p, m, False
    one = F(Fraction(1))
    if kind == "lion":
        c = add(mul(beta1, m), mul(sub(one, beta1), g))
        u = F(Fraction((c.v > 0) - (c.v < 0)))
        pn = mul(sub(p, mul(lr, u)), decay) if after else sub(mul(p, decay), mul(lr, u))
        m = add(mul(beta2, m), mul(sub(one, beta2), g))
        return pn, m, True
    gd = add(g, mul(wd, p)) if wd.v != 0 else g
    if kind == "momentum":
        m = gd if first else add(mul(beta1, m), gd)
        return sub(p, mul(lr, m)), m, True
    if kind == "rmsprop":
        m = add(mul(beta1, m), mul(sub(one, beta1), mul(gd, gd)))
    else:
        m = add(m, mul(gd, gd))
    return sub(p, mul(lr, div(gd, add(sqrt(m), eps)))), m, True
