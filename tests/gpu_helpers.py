"""Helpers of the GPU parity tests: comparison rule, buffers, raw C-ABI calls."""
from __future__ import annotations

import ctypes

import numpy as np
import torch

import oracle as O
import workloads as W

KIND = {"adam": O.ADAM, "ademamix": O.ADEMAMIX}
DT = {"fp32": O.F32, "fp16": O.F16, "bf16": O.BF16}
REL_TOL_F32 = 2e-6      # fp32 storage and every fp32 state
ULP_TOL_16 = 1          # fp16/bf16 parameters


def _ordered16(bits: np.ndarray) -> np.ndarray:
    """Monotone integer image of 16-bit float bit patterns (+0 and -0 adjacent)."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7fff) - 1, b)


def _nan16(bits: np.ndarray, storage: str) -> np.ndarray:
    if storage == "fp16":
        return ((bits & 0x7c00) == 0x7c00) & ((bits & 0x3ff) != 0)
    return ((bits & 0x7f80) == 0x7f80) & ((bits & 0x7f) != 0)


def compare(got: np.ndarray, ref: np.ndarray, storage: str) -> dict:
    """The parity rule.  fp32: bitwise equal, or both NaN, or ref != 0 and
    |got - ref| <= 2e-6 |ref|.  fp16/bf16: at most 1 ulp apart on the
    monotone integer image (both NaN counts as equal).  Returns counts and
    the worst error; 'ok' says whether the tolerance holds, 'bitwise' whether
    every element is bit-identical (NaN payloads aside)."""
    assert got.shape == ref.shape and got.dtype == ref.dtype, (got.shape, ref.shape, got.dtype, ref.dtype)
    if got.size == 0:
        return {"ok": True, "bitwise": True, "n_diff": 0, "worst": 0.0}
    if storage == "fp32" or got.dtype == np.float32:
        gb, rb = got.view(np.uint32), ref.view(np.uint32)
        both_nan = np.isnan(got) & np.isnan(ref)
        same = (gb == rb) | both_nan
        with np.errstate(invalid="ignore", divide="ignore"):
            rel = np.abs(got.astype(np.float64) - ref.astype(np.float64)) / np.abs(ref.astype(np.float64))
        ok = same | ((ref != 0) & (rel <= REL_TOL_F32))
        worst = float(np.nanmax(np.where(same, 0.0, rel))) if not same.all() else 0.0
    else:
        both_nan = _nan16(got, storage) & _nan16(ref, storage)
        same = (got == ref) | both_nan
        ulp = np.abs(_ordered16(got) - _ordered16(ref))
        ok = same | (ulp <= ULP_TOL_16)
        worst = float(np.max(np.where(same, 0, ulp)))
    return {"ok": bool(ok.all()), "bitwise": bool(same.all()), "n_diff": int((~same).sum()),
            "worst": worst, "first_bad": int(np.argmin(ok)) if not ok.all() else -1}


def assert_parity(got: np.ndarray, ref: np.ndarray, storage: str, what: str,
                  bitwise: bool = True) -> dict:
    r = compare(got, ref, storage)
    assert r["ok"], f"{what}: outside tolerance: {r}"
    if bitwise:
        assert r["bitwise"], f"{what}: not bitwise identical to the oracle: {r}"
    return r


def lib():
    from optimizer_update_amd import _lib
    return _lib.load()


def raw_update(L, kind: str, storage: str, p: torch.Tensor, g: torch.Tensor, s1: torch.Tensor,
               s2: torch.Tensor, n: int, hp: O.HParams, step: int, stream: int) -> int:
    """optimizer_update_32bit through the C ABI with raw pointers."""
    return L.optimizer_update_32bit(KIND[kind], DT[storage], p.data_ptr(), g.data_ptr(),
                                    s1.data_ptr(), s2.data_ptr(), n, hp.beta1, hp.beta2, hp.beta3,
                                    hp.alpha, hp.eps, hp.weight_decay, step, hp.lr,
                                    int(hp.skip_zeros), stream)


def pkg_hp(hp: O.HParams):
    from optimizer_update_amd import HParams
    return HParams(**hp.__dict__)


def padded_offsets(sizes, align_elems: int = 64) -> tuple[list[int], int]:
    """Offsets of segments packed into one buffer, each start rounded up to
    align_elems elements (so every segment starts 256-byte aligned)."""
    offs, cur = [], 0
    for n in sizes:
        offs.append(cur)
        cur += -(-n // align_elems) * align_elems
    return offs, max(cur, 1)


def stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def last_error(L) -> str:
    return L.ou_last_error().decode(errors="replace")


def to_dev(a: np.ndarray, storage: str) -> torch.Tensor:
    return W.to_torch(a, storage, device="cuda")


def ctypes_ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())
