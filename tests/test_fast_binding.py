"""CPU tests of the CPython entry points (_fast) that stand in for ctypes on
the per-step calls: installed when built, the same status as the ctypes path
for the same arguments (validation runs in the library either way),
hyperparameters rounded to binary32 as ctypes rounds them, and argument
errors raised. The library runs in validate-only mode: no device is touched.
"""
import ctypes

import pytest

from optimizer_update_amd import _lib

OU_OK, OU_EINVAL, OU_EALIGN, OU_EOVERLAP = 0, -1, -3, -4


@pytest.fixture(scope="module")
def libs():
    fast = _lib.load()
    if not isinstance(fast.optimizer_update_32bit, type(len)):
        pytest.fail("_fast is not built: __graft_entry__.build() builds it with the library")
    plain = ctypes.CDLL(_lib.LIBRARY)      # the same loaded library, through ctypes
    i32, i64, f32, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    plain.optimizer_update_32bit.argtypes = [i32, i32, vp, vp, vp, vp, i64] + [f32] * 6 + [i64, f32, i32, vp]
    plain.optimizer_update_32bit.restype = i32
    plain.optimizer_update_8bit_blockwise.argtypes = ([i32, i32] + [vp] * 6 + [i64] + [f32] * 6 +
                                                      [i64, f32, i32, vp])
    plain.optimizer_update_8bit_blockwise.restype = i32
    for name in ("ou_plan_step", "ou_plan8_step"):
        getattr(plain, name).argtypes = [vp, ctypes.POINTER(_lib.ou_hparams), vp]
        getattr(plain, name).restype = i32
    fast.ou__validate_only(1)
    yield fast, plain
    fast.ou__validate_only(0)


def _args32(**kw):
    a = dict(kind=0, dtype=0, p=0x100000, g=0x200000, s1=0x300000, s2=0x400000, n=1024, b1=0.9,
             b2=0.999, b3=0.9999, alpha=5.0, eps=1e-8, wd=0.01, step=1, lr=1e-3, skip=0, stream=None)
    a.update(kw)
    return tuple(a.values())


CASES32 = [
    {}, dict(kind=1, s1=0x500000), dict(kind=5, s2=None), dict(kind=0x100), dict(kind=7), dict(dtype=2),
    dict(dtype=3), dict(n=0, p=0, g=0), dict(n=-1), dict(p=0x100002), dict(g=0x100000 + 64),
    dict(step=0), dict(b1=1.0), dict(b1=1.0 - 1e-9),     # rounds to 1.0f: rejected on both paths
    dict(b2=float("nan")), dict(eps=-1e-30), dict(lr=float("inf")), dict(wd=1e39),  # overflows binary32
    dict(p=(1 << 64) - 64), dict(stream=0x1234),
]


@pytest.mark.parametrize("kw", CASES32)
def test_update32_status_matches_ctypes(libs, kw):
    fast, plain = libs
    a = _args32(**kw)
    assert fast.optimizer_update_32bit(*a) == plain.optimizer_update_32bit(*a)


def test_update8_status_matches_ctypes(libs):
    fast, plain = libs
    base = [0, 2, 0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000, 4096, 0.9, 0.999,
            0.9999, 5.0, 1e-8, 0.01, 1, 1e-3, 0, None]
    cases = [dict(), {0: 1, 4: 0x700000}, {1: 3}, {6: 0x500002}, {3: 0x100000}, {8: 0}, {9: 1.0},
             {15: 0}, {0: 2}]
    for c in cases:
        a = list(base)
        for i, v in c.items():
            a[i] = v
        assert fast.optimizer_update_8bit_blockwise(*a) == plain.optimizer_update_8bit_blockwise(*a), c


def test_plan_steps_take_the_struct_or_its_address(libs):
    """A null plan is rejected on both paths, whichever form the hparams
    take; ctypes-style byref() is not a form the fast path accepts."""
    fast, plain = libs
    hp = _lib.ou_hparams(0.9, 0.999, 0.9999, 5.0, 1e-8, 0.0, 1e-3, 0, 1)
    for name in ("ou_plan_step", "ou_plan8_step"):
        f, g = getattr(fast, name), getattr(plain, name)
        assert f(None, hp, None) == g(None, hp, None) == OU_EINVAL
        assert f(None, ctypes.addressof(hp), None) == OU_EINVAL
        assert f(ctypes.c_void_p(None), hp, ctypes.c_void_p(None)) == OU_EINVAL
        with pytest.raises(TypeError):
            f(None, ctypes.byref(hp), None)


@pytest.mark.parametrize("form", ["pointer", "c_void_p", "short_bytearray", "long_bytearray", "str"])
def test_plan_steps_reject_buffers_that_are_not_the_struct(libs, form):
    """Objects whose buffer is not an ou_hparams (a ctypes pointer or
    c_void_p exports its 8-byte pointer cell, a bytearray may be short) are
    refused with TypeError: the library must never read 40 bytes from a
    smaller buffer."""
    fast, _ = libs
    hp = _lib.ou_hparams(0.9, 0.999, 0.9999, 5.0, 1e-8, 0.0, 1e-3, 0, 1)
    arg = {"pointer": lambda: ctypes.pointer(hp),
           "c_void_p": lambda: ctypes.c_void_p(ctypes.addressof(hp)),
           "short_bytearray": lambda: bytearray(4),
           "long_bytearray": lambda: bytearray(64),
           "str": lambda: "hparams"}[form]()
    for name in ("ou_plan_step", "ou_plan8_step"):
        with pytest.raises(TypeError):
            getattr(fast, name)(None, arg, None)


def test_plan_steps_accept_a_struct_sized_buffer(libs):
    fast, _ = libs
    raw = bytearray(ctypes.sizeof(_lib.ou_hparams))
    for name in ("ou_plan_step", "ou_plan8_step"):
        assert getattr(fast, name)(None, raw, None) == OU_EINVAL   # null plan, checked by the library



def test_argument_errors_raise(libs):
    fast, _ = libs
    with pytest.raises(TypeError):
        fast.optimizer_update_32bit(*_args32()[:-1])
    with pytest.raises(TypeError):
        fast.optimizer_update_32bit(*_args32(lr="0.001"))
    with pytest.raises(TypeError):
        fast.optimizer_update_32bit(*_args32(n=1.5))
    with pytest.raises(OverflowError):
        fast.optimizer_update_32bit(*_args32(p=-1))
