"""CPU tests of the C ABI: exports, layout, validation, dispatch.

The calls pass fabricated addresses.  The module runs with the library's
validate-only switch on (ou__validate_only), so every entry point returns
right after its argument checks, before it queries or touches a device: the
tests launch nothing and allocate nothing, with or without a GPU present.
"""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle as O
from optimizer_update_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "optimizer_update.h")

OU_OK, OU_EINVAL, OU_EALIGN, OU_EOVERLAP = 0, -1, -3, -4


@pytest.fixture(scope="module")
def L():
    lib = _lib.load()
    lib.ou__validate_only(1)
    yield lib
    lib.ou__validate_only(0)


def test_exports_every_header_function(L):
    names = _lib.header_functions()
    assert set(names) == {"optimizer_update_32bit", "optimizer_update_32bit_multi",
                          "ou_clip_workspace_bytes", "optimizer_update_32bit_clip",
                          "ou_plan_step_clip", "ou_plan_clip_factors",
                          "ou_plan_create", "ou_plan_step", "ou_plan_graph_step",
                          "ou_plan_graph_step_clip",
                          "ou_plan_describe", "ou_plan_destroy", "ou_status_string",
                          "ou_last_error", "ou_8bit_qmap", "optimizer_update_8bit_blockwise",
                          "ou_plan8_create", "ou_plan8_step", "ou_plan8_graph_step",
                          "ou_plan8_destroy", "optimizer_update_32bit_clip_noalloc",
                          "ou_clip_noalloc_max_elements", "ou_graph_create", "ou_graph_step",
                          "ou_graph_destroy"}
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    assert set(names) <= exported
    # nothing else is exported besides the test hooks
    assert exported - set(names) == {"ou__select_single", "ou__force_single", "ou__force_multi",
                                     "ou__step_scalars", "ou__force_8bit", "ou__validate_only",
                                     "ou__force_xcd", "ou__stream_probe", "ou__narrow",
                                     "ou__sqrt", "ou__recip8", "ou__quant8", "ou__valu_probe",
                                     "ou__select_multi"}


def test_header_is_plain_c_and_matches_ctypes_layout(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "optimizer_update.h"\n'
        'int main(void){printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(ou_hparams), '
        'offsetof(ou_hparams, skip_zeros), offsetof(ou_hparams, step), sizeof(ou_segment), '
        'offsetof(ou_segment, n), offsetof(ou_segment, dtype), sizeof(ou_segment8), '
        'offsetof(ou_segment8, n), offsetof(ou_segment8, dtype)); return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                    str(src), "-o", str(exe)], check=True)
    got = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True,
                                       check=True).stdout.split()))
    H, S, S8 = _lib.ou_hparams, _lib.ou_segment, _lib.ou_segment8
    assert got == [ctypes.sizeof(H), H.skip_zeros.offset, H.step.offset, ctypes.sizeof(S),
                   S.n.offset, S.dtype.offset, ctypes.sizeof(S8), S8.n.offset, S8.dtype.offset]


def _call(L, kind=0, dtype=0, p=0x10000, g=0x20000, s1=0x30000, s2=0x40000, n=16, b1=0.9,
          b2=0.999, b3=0.9999, alpha=5.0, eps=1e-8, wd=0.0, step=1, lr=1e-3, skip=0):
    return L.optimizer_update_32bit(kind, dtype, p, g, s1, s2, n, b1, b2, b3, alpha, eps, wd,
                                    step, lr, skip, None)


def _segs(*rows):
    arr = (_lib.ou_segment * len(rows))()
    for i, r in enumerate(rows):
        arr[i] = _lib.ou_segment(*r)
    return arr


@pytest.mark.parametrize("case,kw,code", [
    ("unknown kind", dict(kind=6), OU_EINVAL),
    ("negative kind", dict(kind=-1), OU_EINVAL),
    ("adam null state2", dict(s2=0), OU_EINVAL),
    ("lion beta2 = 1", dict(kind=5, b2=1.0), OU_EINVAL),
    ("momentum state1 overlaps param", dict(kind=2, s1=0x10000 + 32), OU_EOVERLAP),
    ("decay-after with momentum", dict(kind=2 | 0x100), OU_EINVAL),
    ("decay-after with rmsprop", dict(kind=3 | 0x100), OU_EINVAL),
    ("decay-after with adagrad", dict(kind=4 | 0x100), OU_EINVAL),
    ("unknown flag bit", dict(kind=0 | 0x200), OU_EINVAL),
    ("decay-after, unknown kind", dict(kind=6 | 0x100), OU_EINVAL),
    ("decay-after adam, bad beta", dict(kind=0 | 0x100, b1=1.0), OU_EINVAL),
    ("unknown dtype", dict(dtype=3), OU_EINVAL),
    ("negative n", dict(n=-1), OU_EINVAL),
    ("step 0", dict(step=0), OU_EINVAL),
    ("beta1 = 1", dict(b1=1.0), OU_EINVAL),
    ("beta2 < 0", dict(b2=-0.1), OU_EINVAL),
    ("beta2 nan", dict(b2=float("nan")), OU_EINVAL),
    ("ademamix beta3 = 1", dict(kind=1, b3=1.0), OU_EINVAL),
    ("ademamix alpha inf", dict(kind=1, alpha=float("inf")), OU_EINVAL),
    ("eps < 0", dict(eps=-1e-8), OU_EINVAL),
    ("lr inf", dict(lr=float("inf")), OU_EINVAL),
    ("wd nan", dict(wd=float("nan")), OU_EINVAL),
    ("null param", dict(p=0), OU_EINVAL),
    ("null grad", dict(g=0), OU_EINVAL),
    ("fp32 param 2-byte aligned", dict(p=0x10002), OU_EALIGN),
    ("fp16 grad odd address", dict(dtype=1, g=0x20001), OU_EALIGN),
    ("state not 4-byte aligned", dict(s2=0x40002), OU_EALIGN),
    ("param overlaps grad", dict(p=0x20000 - 32), OU_EOVERLAP),
    ("grad overlaps state1", dict(g=0x30000 + 4), OU_EOVERLAP),
    ("ademamix slow plane overlaps state2", dict(kind=1, s2=0x30000 + 4 * 16), OU_EOVERLAP),
    ("state1 is state2", dict(s2=0x30000), OU_EOVERLAP),
])
def test_single_entry_validation(L, case, kw, code):
    assert _call(L, **kw) == code, case
    assert L.ou_last_error().decode(), "an error message is set"


@pytest.mark.parametrize("kind", [0x100, 0x101, 0x105])
def test_decay_after_flag_passes_validation(L, kind):
    assert _call(L, kind=kind, s2=0x40000 if kind != 0x105 else 0) == OU_OK
    h = ctypes.c_void_p()
    st = L.ou_plan_create(kind, _segs((0x100000, 0x200000, 0x300000, 0x400000, 1024, 0, 0)), 1,
                          ctypes.byref(h))
    assert st == OU_OK and not h.value
    assert L.ou_plan_create(0x102, _segs((0x100000, 0x200000, 0x300000, 0, 1024, 0, 0)), 1,
                            ctypes.byref(h)) == OU_EINVAL


@pytest.mark.parametrize("kind", [2, 3, 4, 5])
def test_one_state_kinds_ignore_state2(L, kind):
    # state2 is not checked: NULL, misaligned or overlapping, it passes validation
    for s2 in (0, 0x40002, 0x30000, 0x10000):
        assert _call(L, kind=kind, s2=s2) == OU_OK
    assert _call(L, kind=kind, s1=0x30002) == OU_EALIGN
    assert _call(L, kind=kind, s1=0x20000 + 8) == OU_EOVERLAP


def test_adjacent_buffers_are_not_overlap_and_n0_is_noop(L):
    # n = 0 returns before any device work, whatever the pointers
    assert _call(L, n=0) == OU_OK
    assert _call(L, n=0, p=0, g=0, s1=0, s2=0) == OU_OK
    # touching ranges pass validation
    assert _call(L, p=0x10000, g=0x10000 + 64, s1=0x10000 + 128, s2=0x10000 + 192) == OU_OK
    h = ctypes.c_void_p()
    seg = _segs((0x10000, 0x10000 + 64, 0x10000 + 128, 0x10000 + 192, 16, 0, 0))
    assert L.ou_plan_create(0, seg, 1, ctypes.byref(h)) == OU_OK and not h.value


def test_plan_and_multi_validation(L):
    h = ctypes.c_void_p()
    ok = (0x100000, 0x200000, 0x300000, 0x400000, 1024, 0, 0)
    cases = {
        "overlapping params across segments": ([ok, (0x100000 + 4 * 512, 0x500000, 0x600000, 0x700000, 1024, 0, 0)], OU_EOVERLAP),
        "grad shared with another segment's state": ([ok, (0x800000, 0x300000, 0x900000, 0xa00000, 8, 0, 0)], OU_EOVERLAP),
        "bad dtype": ([(0x100000, 0x200000, 0x300000, 0x400000, 16, 7, 0)], OU_EINVAL),
        "reserved not zero": ([(0x100000, 0x200000, 0x300000, 0x400000, 16, 0, 1)], OU_EINVAL),
        "misaligned bf16": ([(0x100001, 0x200000, 0x300000, 0x400000, 16, 2, 0)], OU_EALIGN),
    }
    for name, (rows, code) in cases.items():
        assert L.ou_plan_create(0, _segs(*rows), len(rows), ctypes.byref(h)) == code, name
        assert not h.value, name
        hp = _lib.ou_hparams(0.9, 0.999, 0.9999, 5.0, 1e-8, 0.0, 1e-3, 0, 1)
        assert L.optimizer_update_32bit_multi(0, _segs(*rows), len(rows), ctypes.byref(hp), None) == code, name
    # two segments sharing one read-only gradient buffer are allowed by validation
    shared = [ok, (0x800000, 0x200000, 0x900000, 0xa00000, 1024, 0, 0)]
    assert L.ou_plan_create(0, _segs(*shared), 2, ctypes.byref(h)) == OU_OK
    hp = _lib.ou_hparams(0.9, 0.999, 0.9999, 5.0, 1e-8, 0.0, 1e-3, 0, 1)
    assert L.optimizer_update_32bit_multi(0, _segs(*shared), 2, ctypes.byref(hp), None) == OU_OK
    assert L.ou_plan_create(6, _segs(ok), 1, ctypes.byref(h)) == OU_EINVAL
    # a one-state plan ignores state2: NULL, or overlapping anything, passes validation
    for s2 in (0, 0x100000):
        st = L.ou_plan_create(4, _segs((0x100000, 0x200000, 0x300000, s2, 1024, 0, 0)), 1,
                              ctypes.byref(h))
        assert st == OU_OK
    assert L.ou_plan_create(0, _segs(ok), 1, None) == OU_EINVAL
    bad_hp = _lib.ou_hparams(0.9, 0.999, 0.9999, 5.0, 1e-8, 0.0, 1e-3, 0, 0)
    assert L.optimizer_update_32bit_multi(0, _segs(ok), 1, ctypes.byref(bad_hp), None) == OU_EINVAL
    assert L.ou_plan_step(None, bad_hp, None) == OU_EINVAL
    assert L.ou_plan_graph_step(None, ctypes.byref(bad_hp), None) == OU_EINVAL
    assert L.ou_plan_describe(None, None, None, None) == OU_EINVAL
    assert L.ou_plan_step_clip(None, ctypes.byref(bad_hp), 1.0, None) == OU_EINVAL
    assert L.ou_plan_graph_step_clip(None, ctypes.byref(bad_hp), 1.0, None) == OU_EINVAL
    assert L.ou_plan_clip_factors(None, None, 0) == OU_EINVAL
    L.ou_plan_destroy(None)


def _clip(L, max_unorm=1.0, ws=0x800000, wsb=None, n=4096, p=0x10000, kind=0, **kw):
    if wsb is None:
        wsb = L.ou_clip_workspace_bytes(n)
    return L.optimizer_update_32bit_clip(kind, 0, p, 0x20000, 0x30000, 0x40000, n, 0.9, 0.999, 0.9999,
                                         5.0, 1e-8, 0.0, kw.get("step", 1), 1e-3, 0, max_unorm,
                                         ws, wsb, None)


def _clip_noalloc(L, max_unorm=1.0, n=4096, p=0x10000, kind=0, dtype=0, s2=0x40000):
    return L.optimizer_update_32bit_clip_noalloc(kind, dtype, p, 0x20000, 0x30000, s2, n, 0.9, 0.999,
                                                 0.9999, 5.0, 1e-8, 0.0, 1, 1e-3, 0, max_unorm, None)


def test_graph_entry_validation(L):
    """ou_graph_create and ou_graph_step reject what they must before any
    device work: a null output handle, negative counts, null arrays or
    plans, a null graph or hparams."""
    vp = ctypes.c_void_p
    h = vp()
    none = (vp * 1)()
    assert L.ou_graph_create(none, 0, none, 0, None) == OU_EINVAL
    assert L.ou_graph_create(none, -1, none, 0, ctypes.byref(h)) == OU_EINVAL
    assert L.ou_graph_create(None, 1, none, 0, ctypes.byref(h)) == OU_EINVAL
    assert L.ou_graph_create(none, 1, none, 0, ctypes.byref(h)) == OU_EINVAL      # plan 0 is null
    assert L.ou_graph_create(none, 0, none, 1, ctypes.byref(h)) == OU_EINVAL      # 8-bit plan 0 is null
    assert L.ou_graph_create(none, 0, none, 0, ctypes.byref(h)) == OU_OK and h.value
    hp = _lib.ou_hparams(0.9, 0.999, 0.9999, 5.0, 1e-8, 0.0, 1e-3, 0, 1)
    assert L.ou_graph_step(None, ctypes.byref(hp), None) == OU_EINVAL
    assert L.ou_graph_step(h, None, None) == OU_EINVAL
    L.ou_graph_destroy(h)
    L.ou_graph_destroy(None)


def test_clip_noalloc_validation(L):
    """The allocation-free clipped step checks what the workspace form
    checks, minus the workspace, and refuses tensors beyond its static
    scratch (2^30 elements) before touching a device."""
    big = 1 << 30
    assert L.ou_clip_noalloc_max_elements() == big
    assert _clip_noalloc(L) == OU_OK
    assert _clip_noalloc(L, n=0) == OU_OK
    assert _clip_noalloc(L, max_unorm=0.0) == OU_OK
    assert _clip_noalloc(L, max_unorm=-1.0) == OU_EINVAL
    assert _clip_noalloc(L, max_unorm=float("nan")) == OU_EINVAL
    assert _clip_noalloc(L, kind=2) == OU_EINVAL                  # one-state kind with clipping
    assert _clip_noalloc(L, p=0x10002) == OU_EALIGN
    assert _clip_noalloc(L, s2=0x10000 + 64) == OU_EOVERLAP       # state2 inside param
    spread = dict(p=0x10_0000_0000, s2=0x40_0000_0000)
    args = (0, 0, spread["p"], 0x20_0000_0000, 0x30_0000_0000, spread["s2"])
    hp = (0.9, 0.999, 0.9999, 5.0, 1e-8, 0.0, 1, 1e-3, 0, 1.0, None)
    assert L.optimizer_update_32bit_clip_noalloc(*args, big, *hp) == OU_OK
    assert L.optimizer_update_32bit_clip_noalloc(*args, big + 1, *hp) == OU_EINVAL
    assert b"static scratch" in L.ou_last_error()
    # the workspace form has no such limit
    assert L.optimizer_update_32bit_clip(*args, big + 1, *hp[:-1], 0x50_0000_0000,
                                         L.ou_clip_workspace_bytes(big + 1), None) == OU_OK


def test_clip_entry_validation(L):
    assert L.ou_clip_workspace_bytes(0) == 256
    assert L.ou_clip_workspace_bytes(1) == 256 + 16
    assert L.ou_clip_workspace_bytes(2048) == 256 + 16
    assert L.ou_clip_workspace_bytes(2049) == 256 + 32
    assert L.ou_clip_workspace_bytes(1 << 30) == 256 + 16 * (1 << 19)
    assert _clip(L, max_unorm=-1.0) == OU_EINVAL
    assert _clip(L, max_unorm=float("nan")) == OU_EINVAL
    assert _clip(L, max_unorm=float("inf")) == OU_EINVAL
    assert _clip(L, ws=0) == OU_EINVAL
    assert _clip(L, ws=0x800008) == OU_EALIGN
    assert _clip(L, wsb=100) == OU_EINVAL
    assert _clip(L, ws=0x40000 + 64) == OU_EOVERLAP          # workspace inside state2
    assert _clip(L, ws=0x10000 - 64) == OU_EOVERLAP          # workspace runs into param
    assert _clip(L, step=0) == OU_EINVAL
    assert _clip(L) == OU_OK                                # passes validation
    assert _clip(L, n=0) == OU_OK                           # nothing to do
    assert _clip(L, max_unorm=0.0, n=0, ws=0) == OU_OK        # plain step, no workspace
    for kind in (2, 3, 4, 5, 0x105):                         # clipping: two-state kinds only
        assert _clip(L, kind=kind) == OU_EINVAL
        assert _clip(L, kind=kind, max_unorm=0.0, n=0, ws=0) == OU_OK


def test_status_strings(L):
    for code, name in _lib.STATUS.items():
        assert L.ou_status_string(code).decode().startswith(name)
    assert L.ou_status_string(42).decode() == "unknown status"


@pytest.mark.parametrize("cu,lds_cu,lds_blk", [(80, 65536, 65536), (256, 163840, 163840),
                                                (304, 65536, 65536), (256, 0, 0)])
def test_dispatch_with_mocked_device(L, cu, lds_cu, lds_blk):
    """Launch selection from fabricated device properties: the grid covers
    the tensor, blocks are whole waves, small tensors get one block, the
    occupancy cap of grids that oversubscribe the CUs reserves LDS so that
    exactly the kind's number of one-wave blocks fit per CU (by the bytes a
    tile reads per element: 20 B fp32 AdEMAMix 6, 16 B fp32 Adam and 16-bit
    AdEMAMix 7, 8 otherwise; none when the device reports no LDS size), and
    the choice depends only on the arguments."""
    out = (ctypes.c_int64 * 5)()
    for kind, dtype in ((k, d) for k in (0, 1, 2, 5) for d in (0, 1, 2)):
        per_cu = {(0, 0): 7, (1, 0): 6, (1, 1): 7, (1, 2): 7}.get((kind, dtype), 8)
        for n in (1, 2, 31, 64, 255, 256, 1023, 1024, 1025, 4095, 4096, 4097, 65539, 1 << 20,
                  (1 << 28) + 3, 1 << 30):
            for aligned in (0, 1):
                assert L.ou__select_single(cu, lds_cu, lds_blk, kind, dtype, n, aligned, out) == 0
                block, epl, unroll, grid, lds = list(out)
                assert block % 64 == 0 and 64 <= block <= 1024
                assert epl in (4, 8) and unroll in (1, 2, 4)
                units = -(-n // epl) if aligned else n
                # every lane's first pass covers the tensor (the kernels loop
                # grid-stride for the rest, so this is about efficiency)
                assert grid * block * unroll >= units
                if units <= 1024:
                    assert grid * block >= units and grid <= 16 and lds == 0
                if lds:
                    assert per_cu * lds <= lds_cu < (per_cu + 1) * lds and lds <= lds_blk
                    assert grid >= 32 * cu and block == 64
                elif lds_cu and grid >= 32 * cu:
                    raise AssertionError("large grids get the occupancy cap")
                again = (ctypes.c_int64 * 5)()
                L.ou__select_single(cu, lds_cu, lds_blk, kind, dtype, n, aligned, again)
                assert list(again) == list(out)


@pytest.mark.parametrize("cu,lds_cu,lds_blk", [(80, 65536, 65536), (256, 163840, 163840), (256, 0, 0)])
def test_plan_shape_selection(L, cu, lds_cu, lds_blk):
    """A plan's dtype group: collections of 2^24 elements or more take
    one-wave blocks of 512-element work items in runs of 64 with the
    single-tensor cap for the kind and storage (6, 7 or 8 blocks per CU by the
    bytes read per element; none when the device reports no LDS size);
    smaller ones 4-wave blocks of 256-element items, no cap, runs of 16.  The
    clipped step's pass 1 keeps 5 blocks per CU once its grid of 2,048-element
    chunks is 20 times the CU count."""
    out = (ctypes.c_int64 * 7)()
    for kind, dtype in ((k, d) for k in (0, 1, 2, 5) for d in (0, 1, 2)):
        per_cu = {(0, 0): 7, (1, 0): 6, (1, 1): 7, (1, 2): 7}.get((kind, dtype), 8)
        for total in (1, 4096, 3440640, (1 << 24) - 1, 1 << 24, 287866880):
            assert L.ou__select_multi(cu, lds_cu, lds_blk, kind, dtype, total, out) == 0
            waves, epl, unroll, lds, run, chunk, lds1 = list(out)
            assert epl == 4 and chunk % (64 * epl * unroll) == 0 and waves * 64 <= 512
            if total >= 1 << 24:
                assert (waves, unroll, run, chunk) == (1, 2, 64, 512)
                if lds_cu:
                    assert per_cu * lds <= lds_cu < (per_cu + 1) * lds and lds <= lds_blk
                else:
                    assert lds == 0
            else:
                assert (waves, unroll, lds, run, chunk) == (4, 1, 0, 16, 256)
            chunks = -(-total // 2048)
            if lds_cu and chunks >= 20 * cu:
                assert 5 * lds1 <= lds_cu < 6 * lds1
            else:
                assert lds1 == 0
    assert L.ou__select_multi(cu, lds_cu, lds_blk, 0, 0, -1, out) == OU_EINVAL


def test_step_scalars_match_oracle_bitwise(L):
    """The library's host-side per-step scalars equal the oracle's, bit for
    bit (both compute bc = fl32(1 - fl64(beta^t)), d = fl32(1 - fl64(lr wd))
    and 1 - beta in binary32, independently)."""
    orc = O.load()
    out = (ctypes.c_float * 12)()
    rng = np.random.default_rng(0)
    betas = [0.9, 0.999, 0.9999, 0.5, 0.0, 0.875, 1 - 2 ** -10, 0.95, 0.99]
    for _ in range(300):
        b1, b2, b3 = (float(rng.choice(betas)) for _ in range(3))
        lr = float(10 ** rng.uniform(-6, 0))
        wd = float(rng.choice([0.0, 0.01, 0.1, 1e-4]))
        step = int(rng.choice([1, 2, 3, 10, 100, 1000, 12345, 10 ** 6]))
        hp = _lib.ou_hparams(b1, b2, b3, 5.0, 1e-8, wd, lr, 0, step)
        assert L.ou__step_scalars(ctypes.byref(hp), out) == 0
        ref = orc.step_scalars(O.HParams(lr=lr, beta1=b1, beta2=b2, beta3=b3, weight_decay=wd), step)
        lib_vals = dict(zip(["omb1", "omb2", "omb3", "bc1", "bc2", "decay"],
                            [out[3], out[4], out[5], out[9], out[10], out[11]]))
        for k, v in lib_vals.items():
            assert np.float32(v).tobytes() == np.float32(ref[k]).tobytes(), (k, v, ref[k], b1, b2, step)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        _lib.load(str(tmp_path / "liboptimizer_update.so"))


def test_product_path_never_touches_the_oracle():
    """The package and the benchmark's timed path do not import or load the
    oracle; only the benchmark's cpu_baseline leg does."""
    pkg = os.path.join(ROOT, "optimizer_update_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"import oracle|from oracle|liboracle|oracle\.c\b|oracle_update",
                                     text), os.path.join(dirpath, f)
    bench = open(os.path.join(ROOT, "bench.py")).read()
    imports = re.findall(r"^\s*import oracle.*$|^\s*from oracle.*$", bench, flags=re.M)
    assert len(imports) == 1
    body = bench[bench.index("def cpu_baseline"):]
    assert "import oracle" in body.split("\ndef ")[0]


def test_kernel_hash_ignores_comments_only():
    """The benchmark keys its committed counter records by a hash of the
    kernels' code: comments, blank lines and indentation do not change it,
    any token of code does, and a comment marker inside a literal is code."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    a = 'int x = 1; // one\n/* block\n comment */\n\n    float y = 2.0f;\nconst char* s = "a//b/*c*/";\n'
    b = 'int x = 1;\nfloat y = 2.0f;   // two\n  const char* s = "a//b/*c*/";'
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) == 'int x = 1;\nfloat y = 2.0f;\nconst char* s = "a//b/*c*/";'
    assert bench.code_text(a.replace("2.0f", "3.0f")) != bench.code_text(a)
    assert bench.code_text("char c = '\\''; // q\nchar d = '/';") == "char c = '\\'';\nchar d = '/';"
    for f in bench.KERNEL_SOURCES + bench.KERNEL8_SOURCES:
        src = open(os.path.join(ROOT, f)).read()
        code = re.sub(r'"(?:\\.|[^"\\])*"', '""', bench.code_text(src))   # literals out
        assert code.count("{") == code.count("}") and code.count("(") == code.count(")"), f


def test_binding_rejects_host_tensors():
    import torch

    import optimizer_update_amd as ou
    p = torch.zeros(8)
    with pytest.raises(ValueError):
        ou.optimizer_update_32bit("adam", p, p.clone(), p.clone(), p.clone(), step=1, lr=1e-3)


# ------------------------------------------------------- 8-bit block-wise states

def _call8(L, kind=0, dtype=0, p=0x10000, g=0x20000, c1=0x30000, c2=0x40000, a1=0x50000,
           a2=0x60000, n=1000, b1=0.9, step=1):
    return L.optimizer_update_8bit_blockwise(kind, dtype, p, g, c1, c2, a1, a2, n, b1, 0.999, 0.9999,
                                             5.0, 1e-8, 0.0, step, 1e-3, 0, None)


@pytest.mark.parametrize("case,kw,code", [
    ("one-state kind", dict(kind=2), OU_EINVAL),
    ("lion", dict(kind=5), OU_EINVAL),
    ("unknown kind", dict(kind=7), OU_EINVAL),
    ("bad dtype", dict(dtype=3), OU_EINVAL),
    ("null absmax1", dict(a1=0), OU_EINVAL),
    ("null state2", dict(c2=0), OU_EINVAL),
    ("absmax misaligned", dict(a2=0x60002), OU_EALIGN),
    ("fp32 param misaligned", dict(p=0x10002), OU_EALIGN),
    ("codes overlap param", dict(c1=0x10000 + 100), OU_EOVERLAP),
    ("ademamix slow codes overlap state2", dict(kind=1, c2=0x30000 + 1500), OU_EOVERLAP),
    ("absmax1 overlaps absmax2", dict(a2=0x50000 + 8), OU_EOVERLAP),
    ("ademamix absmax planes overlap absmax2", dict(kind=1, a2=0x50000 + 4 * 5), OU_EOVERLAP),
    ("step 0", dict(step=0), OU_EINVAL),
    ("beta1 = 1", dict(b1=1.0), OU_EINVAL),
])
def test_8bit_entry_validation(L, case, kw, code):
    assert _call8(L, **kw) == code, case


def test_8bit_valid_calls_pass_validation(L):
    # unaligned codes are allowed (element-by-element path); n = 0 is a no-op
    for kw in (dict(), dict(kind=1), dict(kind=0x100), dict(c1=0x30001, c2=0x40003), dict(dtype=2)):
        assert _call8(L, **kw) == OU_OK, kw
    assert _call8(L, n=0, p=0, g=0, c1=0, c2=0, a1=0, a2=0) == OU_OK
    h = ctypes.c_void_p()
    seg = (_lib.ou_segment8 * 1)(_lib.ou_segment8(0x100000, 0x200000, 0x300000, 0x400000, 0x500000,
                                                  0x600000, 4096, 0, 0))
    assert L.ou_plan8_create(0, seg, 1, ctypes.byref(h)) == OU_OK and not h.value
    assert L.ou_plan8_create(3, seg, 1, ctypes.byref(h)) == OU_EINVAL
    bad = (_lib.ou_segment8 * 1)(_lib.ou_segment8(0x100000, 0x200000, 0x300000, 0x400000, 0x500000,
                                                  0x500000, 4096, 0, 0))
    assert L.ou_plan8_create(0, bad, 1, ctypes.byref(h)) == OU_EOVERLAP
    assert L.ou_plan8_step(None, None, None) == OU_EINVAL
    assert L.ou_plan8_graph_step(None, None, None) == OU_EINVAL


def test_8bit_qmap_matches_the_oracle(L):
    """The library builds the 8-bit type at compile time, the oracle at run
    time, each from the definition: the magnitudes agree bitwise."""
    import numpy as np
    import oracle as O
    orc = O.load()
    for signed, count in ((1, 128), (0, 256)):
        out = (ctypes.c_float * count)()
        assert L.ou_8bit_qmap(signed, out, count) == OU_OK
        got = np.frombuffer(out, dtype=np.float32)
        assert got.tobytes() == orc.qmap(bool(signed)).tobytes()
        assert L.ou_8bit_qmap(signed, out, count - 1) == OU_EINVAL


def test_8bit_quantizer_exhaustive(tmp_path):
    """The kernels' quantizer (qmap.hpp: key table of the binary64 ratio
    estimate, then one exact comparison), compiled for the host: for a set of
    absmax values from subnormal to the largest binary32, every value within
    2^-26 of absmax and a sample below, with the reciprocal exact and moved
    2^-21 either way, it returns the index of the magnitude nearest to
    |value| / absmax in exact arithmetic (ties to the smaller; NaN, absmax 0
    and infinite absmax -> 0), and the signed code's bit 7 for value < 0."""
    src = os.path.join(os.path.dirname(__file__), "native", "qindex_check.cpp")
    inc = os.path.join(os.path.dirname(os.path.dirname(__file__)), "optimizer_update_amd", "csrc")
    exe = tmp_path / "qindex_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fopenmp", "-I", inc, src,
                    "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr


def test_step_constant_division_exhaustive(tmp_path):
    """The kernels divide by the bias corrections through a binary64 product
    (stepdiv.hpp), compiled here for the host: for bias corrections formed
    as the library forms them and for the ends of [2^-24, 1], it equals the
    correctly rounded binary32 quotient for every binary32 numerator (a
    sample of them for most divisors)."""
    src = os.path.join(os.path.dirname(__file__), "native", "stepdiv_check.cpp")
    inc = os.path.join(os.path.dirname(os.path.dirname(__file__)), "optimizer_update_amd", "csrc")
    exe = tmp_path / "stepdiv_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fopenmp", "-I", inc, src,
                    "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr


def test_stream_probe_validation(L):
    """The bandwidth probe's argument checks (test hook)."""
    for mode in (0, 1, 2):
        assert L.ou__stream_probe(mode, 0x10000, 0x20000, 0x30000, 0x40000, 1 << 20, None) == OU_OK
        assert L.ou__stream_probe(mode, 0x10000, 0x20000, 0x30000, 0x40000, 6, None) == OU_EINVAL
        assert L.ou__stream_probe(mode, 0x10000, 0x20000, 0x30000, 0x40000, 0, None) == OU_EINVAL
        assert L.ou__stream_probe(mode, 0, 0x20000, 0x30000, 0x40000, 16, None) == OU_EINVAL
        assert L.ou__stream_probe(mode, 0x10004, 0x20000, 0x30000, 0x40000, 16, None) == OU_EALIGN
    assert L.ou__stream_probe(3, 0x10000, 0x20000, 0x30000, 0x40000, 16, None) == OU_EINVAL


def test_valu_probe_validation(L):
    """The VALU probe takes op 0 (FMA chains) or 1 (add chains), at least one
    block and one round, and an aligned output; the rest is OU_EINVAL or
    OU_EALIGN before any launch."""
    for op in (0, 1):
        assert L.ou__valu_probe(op, 2048, 16, 0x10000, None) == OU_OK
    assert L.ou__valu_probe(2, 2048, 16, 0x10000, None) == OU_EINVAL
    assert L.ou__valu_probe(-1, 2048, 16, 0x10000, None) == OU_EINVAL
    assert L.ou__valu_probe(0, 0, 16, 0x10000, None) == OU_EINVAL
    assert L.ou__valu_probe(0, 2048, 0, 0x10000, None) == OU_EINVAL
    assert L.ou__valu_probe(0, 2048, 16, 0, None) == OU_EINVAL
    assert L.ou__valu_probe(0, 2048, 16, 0x10002, None) == OU_EALIGN


def test_narrow_hook_validation(L):
    """The storage-rounding hook's argument checks (test hook)."""
    assert L.ou__narrow(1, 0x10000, 0x20000, 16, None) == OU_OK
    assert L.ou__narrow(2, 0x10000, 0x20002, 16, None) == OU_OK
    assert L.ou__narrow(0, 0x10000, 0x20000, 16, None) == OU_EINVAL
    assert L.ou__narrow(1, 0x10000, 0x20000, 0, None) == OU_EINVAL
    assert L.ou__narrow(1, 0x10002, 0x20000, 16, None) == OU_EALIGN
    assert L.ou__narrow(2, 0x10000, 0x20001, 16, None) == OU_EALIGN
    assert L.ou__narrow(18, 0x10000, 0x20000, 16, None) == OU_OK
    assert L.ou__narrow(17, 0x10000, 0x20000, 15, None) == OU_EINVAL
    assert L.ou__narrow(18, 0x10000, 0x20002, 16, None) == OU_EALIGN
    assert L.ou__narrow(16, 0x10000, 0x20000, 16, None) == OU_EINVAL


def test_sqrt_hook_validation(L):
    """The square-root, reciprocal and quantizer hooks' argument checks (test hooks)."""
    assert L.ou__sqrt(0x10000, 0x20000, 16, None) == OU_OK
    assert L.ou__sqrt(0x10000, 0x20000, 0, None) == OU_EINVAL
    assert L.ou__sqrt(0, 0x20000, 16, None) == OU_EINVAL
    assert L.ou__sqrt(0x10002, 0x20000, 16, None) == OU_EALIGN
    assert L.ou__recip8(0x10000, 0x20000, 16, None) == OU_OK
    assert L.ou__recip8(0x10000, 0x20000, -1, None) == OU_EINVAL
    assert L.ou__recip8(0x10000, 0, 16, None) == OU_EINVAL
    assert L.ou__recip8(0x10000, 0x20001, 16, None) == OU_EALIGN
    assert L.ou__quant8(0x10000, 0x20000, 0x30000, 0x40000, 16, None) == OU_OK
    assert L.ou__quant8(0x10000, 0x20000, 0x30000, 0x40000, 0, None) == OU_EINVAL
    assert L.ou__quant8(0x10000, 0x20000, 0, 0x40000, 16, None) == OU_EINVAL
    assert L.ou__quant8(0x10000, 0x20002, 0x30000, 0x40000, 16, None) == OU_EALIGN


# ---- validation against a brute-force reference (property-based) -----------

from hypothesis import HealthCheck, given, settings  # noqa: E402
from hypothesis import strategies as st  # noqa: E402

_SLOT = 256    # bytes between neighbouring slots: buffers of up to 512 B reach over two
_BASE = 0x100000


def _addr(slot, off):
    return _BASE + slot * _SLOT + off


_SEGMENT = st.tuples(st.integers(0, 31), st.integers(0, 31), st.integers(0, 31), st.integers(0, 31),
                     st.integers(1, 64), st.sampled_from([0, 1, 2]),
                     st.sampled_from([0, 0, 0, 0, 1, 2]))   # slots p g s1 s2, n, dtype, misalignment


def _expected(kind, segments):
    """The documented rules, checked pair by pair: a misaligned pointer gives
    OU_EALIGN (segments are checked in order, before any overlap); then any two
    byte ranges that intersect, one of them written, give OU_EOVERLAP."""
    two = kind in (0, 1)
    ranges = []
    for sp, sg, s1, s2, n, dtype, mis in segments:
        sb = 4 if dtype == 0 else 2
        p, g, a1, a2 = _addr(sp, mis), _addr(sg, 0), _addr(s1, 0), _addr(s2, 0)
        if p % sb or g % sb or a1 % 4 or (two and a2 % 4):
            return OU_EALIGN
        ranges += [(p, p + n * sb, True), (g, g + n * sb, False),
                   (a1, a1 + (2 if kind == 1 else 1) * n * 4, True)]
        if two:
            ranges.append((a2, a2 + n * 4, True))
    for i in range(len(ranges)):
        for j in range(i + 1, len(ranges)):
            (lo1, hi1, w1), (lo2, hi2, w2) = ranges[i], ranges[j]
            if (w1 or w2) and lo1 < hi2 and lo2 < hi1:
                return OU_EOVERLAP
    return OU_OK


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(kind=st.sampled_from([0, 1, 2]), segments=st.lists(_SEGMENT, min_size=1, max_size=5))
def test_collection_validation_matches_pairwise_rules(L, kind, segments):
    """ou_plan_create and optimizer_update_32bit_multi return what the
    pairwise reference gives, on random layouts where overlaps and
    misalignments are common (a sort-and-sweep against an O(n^2) check)."""
    rows = [(_addr(sp, mis), _addr(sg, 0), _addr(s1, 0), _addr(s2, 0), n, dtype, 0)
            for sp, sg, s1, s2, n, dtype, mis in segments]
    want = _expected(kind, segments)
    h = ctypes.c_void_p()
    assert L.ou_plan_create(kind, _segs(*rows), len(rows), ctypes.byref(h)) == want
    assert not h.value
    hp = _lib.ou_hparams(0.9, 0.999, 0.9999, 5.0, 1e-8, 0.0, 1e-3, 0, 1)
    assert L.optimizer_update_32bit_multi(kind, _segs(*rows), len(rows), ctypes.byref(hp), None) == want


def test_ranges_past_the_end_of_the_address_space(L):
    """A buffer that would run past 2^64 is rejected (OU_EINVAL), not wrapped
    into a small range that escapes the overlap check."""
    top = (1 << 64) - 64
    assert _call(L, p=top, n=32) == OU_EINVAL
    assert _call(L, s2=top & ~3, n=32) == OU_EINVAL
    h = ctypes.c_void_p()
    assert L.ou_plan_create(0, _segs((0x100000, top, 0x300000, 0x400000, 1024, 0, 0)), 1,
                            ctypes.byref(h)) == OU_EINVAL
    assert _call(L, p=top - 4 * 32, n=32) == OU_OK


_SEGMENT8 = st.tuples(st.lists(st.integers(0, 63), min_size=6, max_size=6), st.integers(1, 300),
                      st.sampled_from([0, 1, 2]), st.sampled_from([0] * 12 + [1, 2]),
                      st.sampled_from([0] * 12 + [1, 2]))  # slots p g c1 c2 a1 a2, n, dtype, p / a1 offsets


def _expected8(kind, segments):
    """The 8-bit segment rules pair by pair: param/grad aligned to their
    element size and absmax to 4 bytes (codes have no alignment), else
    OU_EALIGN; then intersecting byte ranges with one of them written give
    OU_EOVERLAP (codes k*n and n bytes, absmax 4 B per 256-element block)."""
    k = 2 if kind == 1 else 1
    ranges = []
    for slots, n, dtype, mp, ma in segments:
        sb = 4 if dtype == 0 else 2
        p, g, c1, c2, a1, a2 = (_addr(s, 0) for s in slots)
        p += mp
        a1 += ma
        if p % sb or g % sb or a1 % 4 or a2 % 4:
            return OU_EALIGN
        nb = -(-n // 256)
        ranges += [(p, p + n * sb, True), (g, g + n * sb, False), (c1, c1 + k * n, True), (c2, c2 + n, True),
                   (a1, a1 + k * nb * 4, True), (a2, a2 + nb * 4, True)]
    for i in range(len(ranges)):
        for j in range(i + 1, len(ranges)):
            (lo1, hi1, w1), (lo2, hi2, w2) = ranges[i], ranges[j]
            if (w1 or w2) and lo1 < hi2 and lo2 < hi1:
                return OU_EOVERLAP
    return OU_OK


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(kind=st.sampled_from([0, 1]), segments=st.lists(_SEGMENT8, min_size=1, max_size=4))
def test_8bit_collection_validation_matches_pairwise_rules(L, kind, segments):
    """ou_plan8_create returns what the pairwise reference gives."""
    arr = (_lib.ou_segment8 * len(segments))()
    for i, (slots, n, dtype, mp, ma) in enumerate(segments):
        p, g, c1, c2, a1, a2 = (_addr(s, 0) for s in slots)
        arr[i] = _lib.ou_segment8(p + mp, g, c1, c2, a1 + ma, a2, n, dtype, 0)
    h = ctypes.c_void_p()
    assert L.ou_plan8_create(kind, arr, len(segments), ctypes.byref(h)) == _expected8(kind, segments)
    assert not h.value


def test_no_buffer_store_wider_than_8_bytes():
    """Kernels store at most 8 bytes per lane through buffer descriptors.
    After a wider buffer store with a scalar offset the compiler inserts no
    wait state before an instruction that overwrites the data registers,
    and on gfx950 such a write reached the store (a wrong first word in
    some lanes, varying from run to run); 16-byte stores go through global
    addresses, which get the wait state."""
    import glob
    for path in glob.glob(os.path.join(ROOT, "optimizer_update_amd", "csrc", "*.hip")) + \
            glob.glob(os.path.join(ROOT, "optimizer_update_amd", "csrc", "*.hpp")):
        code = open(path).read()
        for wide in ("raw_buffer_store_b96", "raw_buffer_store_b128", "struct_buffer_store_b96",
                     "struct_buffer_store_b128", "raw_ptr_buffer_store"):
            assert wide not in code, f"{os.path.basename(path)} uses {wide}"
