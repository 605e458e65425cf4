"""GPU: the update kernels' storage rounding (elem.hpp's narrow, through the
ou__narrow test hook) on every binary32 bit pattern, against the oracle.

The oracle's conversions are themselves checked on every pattern against
the x86 F16C conversion and an exact-midpoint bfloat16 rule
(tests/native/conv_check.c)."""
import numpy as np
import pytest
import torch

import oracle as O
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _nan16(h: np.ndarray, exp_mask: int, man_mask: int) -> np.ndarray:
    return ((h & exp_mask) == exp_mask) & ((h & man_mask) != 0)


def test_kernel_rounding_exhaustive():
    """All 2^32 patterns in 16 chunks of 2^28: binary16 and bfloat16 codes
    equal the oracle's bitwise, one value at a time (the 32-bit kernels) and
    by packed pairs (the 8-bit kernels); a NaN gives a NaN (payloads are not
    part of the contract)."""
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    L = H.lib()
    orc = O.load()
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.int16, device="cuda")
    for lo in range(-(1 << 31), 1 << 31, chunk):
        x_dev = torch.arange(lo, lo + chunk, dtype=torch.int32, device="cuda").view(torch.float32)
        x = np.arange(lo, lo + chunk, dtype=np.int32).view(np.float32)
        nan = np.isnan(x)
        for dtype, exp_mask, man_mask in ((O.F16, 0x7c00, 0x03ff), (O.BF16, 0x7f80, 0x007f)):
            want = orc.f32_to_storage(x, dtype)
            for mode in (0, 16):
                st = L.ou__narrow(dtype + mode, x_dev.data_ptr(), out.data_ptr(), chunk, H.stream_handle())
                assert st == 0, H.last_error(L)
                got = out.cpu().numpy().view(np.uint16)
                same = (got == want) | (nan & _nan16(got, exp_mask, man_mask))
                assert same.all(), (dtype, mode, lo, int(np.argmin(same)), int((~same).sum()))
        del x_dev


def test_kernel_sqrt_exhaustive():
    """The 8-bit update kernels' square root (short form for waves whose inputs
    are all >= 2^-96, the full sequence otherwise) on all 2^32 patterns, in
    16 chunks of 2^28: bitwise equal to numpy's IEEE binary32 square root; a
    NaN (every negative input included) gives a NaN."""
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    L = H.lib()
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.float32, device="cuda")
    with np.errstate(invalid="ignore"):
        for lo in range(-(1 << 31), 1 << 31, chunk):
            x_dev = torch.arange(lo, lo + chunk, dtype=torch.int32, device="cuda").view(torch.float32)
            st = L.ou__sqrt(x_dev.data_ptr(), out.data_ptr(), chunk, H.stream_handle())
            assert st == 0, H.last_error(L)
            got = out.cpu().numpy()
            want = np.sqrt(np.arange(lo, lo + chunk, dtype=np.int32).view(np.float32))
            same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
            assert same.all(), (lo, int(np.argmin(same)), int((~same).sum()))


def test_kernel_block_reciprocal_exhaustive():
    """The 8-bit kernels' reciprocal of a block maximum (binary64 estimate,
    two Newton steps, one rounding) on every binary32 l in [+0, +inf], in 8
    chunks of 2^28: bitwise equal to numpy's IEEE binary32 1 / l for l > 0
    finite, and 0 for +0 and +inf."""
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    L = H.lib()
    chunk = 1 << 28
    out = torch.empty(chunk, dtype=torch.float32, device="cuda")
    top = 0x7f800000   # +inf
    with np.errstate(divide="ignore", over="ignore"):
        for lo in range(0, top + 1, chunk):
            cnt = min(chunk, top + 1 - lo)
            x_dev = torch.arange(lo, lo + cnt, dtype=torch.int32, device="cuda").view(torch.float32)
            st = L.ou__recip8(x_dev.data_ptr(), out.data_ptr(), cnt, H.stream_handle())
            assert st == 0, H.last_error(L)
            got = out[:cnt].cpu().numpy()
            x = np.arange(lo, lo + cnt, dtype=np.int32).view(np.float32)
            want = np.where((x > 0) & np.isfinite(x), np.float32(1.0) / x, np.float32(0.0)).astype(np.float32)
            same = got.view(np.uint32) == want.view(np.uint32)
            assert same.all(), (lo, int(np.argmin(same)), int((~same).sum()))
