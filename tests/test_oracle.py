"""CPU tests of the oracle against its pins (no GPU)."""
import os
import warnings

import numpy as np
import pytest

import oracle as O
from tests import oracle_pins as P


@pytest.fixture(scope="module")
def orc():
    return O.load()


@pytest.mark.parametrize("pin", P.ALL, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)   # fp16 overflow in numpy's own cast
        pin(orc)


def test_conversion_strided_sweep(orc):
    """Every 61st binary32 bit pattern (2^32 / 61 ~ 7e7 values, every
    exponent and sign, all residues of the dropped bits) through both
    storage conversions, against numpy float16 and torch bfloat16."""
    stride, chunk = 61, 1 << 24
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)
        for start in range(0, 1 << 32, stride * chunk):
            bits = np.arange(start, min(start + stride * chunk, 1 << 32), stride, dtype=np.uint64)
            P.check_conversions(orc, bits.astype(np.uint32))


def test_conversion_exhaustive_native(tmp_path):
    """Every binary32 bit pattern through the oracle's storage conversions
    (tests/native/conv_check.c, built with oracle/oracle.c): binary16
    against the x86 F16C conversion, bfloat16 against the nearer bfloat16
    neighbour in exact binary64 arithmetic (ties to even)."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    exe = tmp_path / "conv_check"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-mf16c",
                    os.path.join(root, "tests", "native", "conv_check.c"),
                    os.path.join(root, "oracle", "oracle.c"), "-lm", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr


@pytest.mark.parametrize("plant", range(1, 31))
def test_planted_mistake_is_caught(plant, tmp_path):
    """A copy of the oracle with one planted mistake (dropped bias
    correction, eps inside the root, decay after the update, decay sign,
    corrected slow EMA, alpha on the wrong EMA, swapped betas, decay on
    skipped elements, dropped square, written gradient, bf16 truncation,
    no fp16 subnormals, step off by one, reversed slow plane; for clipping:
    norm of the new parameter, squared update norm, clipping below the
    bound; one-state kinds: Lion's moment updated before its sign, eps
    inside RMSprop's root, Adagrad without the square, momentum with
    dampening; 8-bit: truncating quantizer, absmax of the old states,
    parameter moved with the quantized moments, first moment's sign
    dropped, blocks of 512, top magnitude left at its bin centre, the
    decoder ignoring the sign bit, the ratio normalised by a rounded
    reciprocal against rounded midpoints) must fail at least one pin that does not
    retype the formulas."""
    path = O.build(str(tmp_path / f"liboracle_plant{plant}.so"), plant=plant)
    bad = O.Oracle(path)
    assert bad.planted == plant
    failed = []
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)
        for pin in P.INDEPENDENT:
            try:
                pin(bad)
            except AssertionError:
                failed.append(pin.__name__)
    assert failed, f"planted mistake {plant} passed every pin"


def test_unknown_kind_or_dtype_rejected(orc):
    lib = orc._lib
    args = (None, None, None, None, 0, 0.9, 0.999, 0.9, 0.0, 1e-8, 0.0, 1, 1e-3, 0, 1)
    assert lib.oracle_update_f32(7, 0, *args) == -1
    assert lib.oracle_update_f32(0, 9, *args) == -1
    assert lib.oracle_update_f32(0, 0, *args) == 0      # n = 0 is a no-op


def test_sweep_matches_page_matrix():
    import json
    import workloads as W
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "golden", "coverage_matrix.json")) as f:
        cm = json.load(f)
    assert tuple(cm["n"] + cm["n_boundary_controls"]) == W.SWEEP_N
    assert tuple(cm["direct_cells_n"] + cm["direct_boundary_controls"]) == W.DIRECT_N
    assert tuple(cm["steps"]) == W.SNAPSHOT_STEPS
