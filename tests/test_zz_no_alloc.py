"""GPU: the allocation-free clipped step (optimizer_update_32bit_clip_noalloc).

It runs the clipped step of optimizer_update_32bit_clip with the library's
static device scratch in place of a caller workspace.  Called through the C
ABI, it must give the workspace form's bytes exactly (parameters and both
states), on two calls in a row, the second on a smaller tensor (so the
scratch still holds the first call's partial norms beyond the second's
chunks), with the clip active and not, for Adam and AdEMAMix, fp32 and
bf16 storage.  Memory the test allocates is allocated before the calls.
"""
import numpy as np
import pytest
import torch

import optimizer_update_amd as ou
from optimizer_update_amd import _lib

pytestmark = pytest.mark.gpu

KIND = {"adam": _lib.OU_ADAM, "ademamix": _lib.OU_ADEMAMIX}
DT = {"fp32": (_lib.OU_F32, torch.float32), "bf16": (_lib.OU_BF16, torch.bfloat16)}


def _inputs(kind, storage, n, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    t = DT[storage][1]
    p = torch.empty(n, device="cuda").uniform_(-1, 1, generator=gen).to(t)
    g = (torch.randn(n, device="cuda", generator=gen) * 1e-2).to(t)
    s1n, s2n = ou.state_sizes(kind, n)
    s1 = (torch.randn(s1n, device="cuda", generator=gen) * 1e-3)
    s2 = (torch.rand(s2n, device="cuda", generator=gen) * 1e-4)
    return p, g, s1, s2


def _call(lib, fn, kind, storage, bufs, step, max_unorm, ws=None):
    p, g, s1, s2 = bufs
    args = [KIND[kind], DT[storage][0], p.data_ptr(), g.data_ptr(), s1.data_ptr(), s2.data_ptr(), p.numel(),
            0.9, 0.999, 0.9999, 5.0, 1e-8, 0.01, step, 1e-3, 0, max_unorm]
    if ws is not None:
        args += [ws.data_ptr(), ws.numel()]
    st = fn(*args, torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.ou_last_error().decode()


def _bytes(t):
    return t.view(torch.uint8).cpu().numpy() if t.dtype != torch.float32 else t.cpu().numpy().view(np.uint8)


@pytest.mark.parametrize("kind,storage", [("adam", "fp32"), ("ademamix", "bf16"), ("adam", "bf16")])
@pytest.mark.parametrize("max_unorm", [1e-4, 10.0])
def test_noalloc_matches_workspace_form(kind, storage, max_unorm):
    lib = _lib.load()
    sizes = ((3 << 20) + 1237, 70001)        # the second call is the smaller one
    cases = []
    for i, n in enumerate(sizes):
        a = _inputs(kind, storage, n, seed=17 + i)
        b = tuple(x.clone() for x in a)
        ws = ou.clip_workspace(n, "cuda")
        cases.append((a, b, ws))
    torch.cuda.synchronize()
    for step in (1, 2):
        for a, b, ws in cases:                # big, then small, in one stream's order
            print(f"noalloc {kind} {storage} max_unorm={max_unorm} n={a[0].numel()} step={step}", flush=True)
            _call(lib, lib.optimizer_update_32bit_clip_noalloc, kind, storage, a, step, max_unorm)
            _call(lib, lib.optimizer_update_32bit_clip, kind, storage, b, step, max_unorm, ws)
        torch.cuda.synchronize()
        for a, b, ws in cases:
            for x, y, name in zip(a, b, ("param", "grad", "state1", "state2")):
                assert np.array_equal(_bytes(x), _bytes(y)), (name, a[0].numel(), step)
    # the clip was active (or not) as intended on the workspace form
    s = ou.clip_scale(cases[0][2])
    assert (s < 1.0) if max_unorm < 1 else (s == 1.0), s


def test_noalloc_limits():
    lib = _lib.load()
    assert lib.ou_clip_noalloc_max_elements() == 1 << 30
    assert ou.clip_noalloc_max_elements() == 1 << 30
    # max_unorm = 0 is the plain step, through the Python wrapper too
    a = _inputs("adam", "fp32", 5000, seed=3)
    b = tuple(x.clone() for x in a)
    ou.optimizer_update_32bit_clip_noalloc("adam", *a, step=1, lr=1e-3, max_unorm=0.0, weight_decay=0.01)
    ou.optimizer_update_32bit("adam", *b, step=1, lr=1e-3, weight_decay=0.01)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
