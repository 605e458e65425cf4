"""Build liboptimizer_update.so (HIP, gfx950) in-tree with hipcc, and the
CPython module _fast that calls its per-step entry points without ctypes.

The flags fix the arithmetic: no contraction into fused multiply-adds,
correctly rounded binary32 division and square root, denormals kept, and no
packed-fp32 instructions.
"""
from __future__ import annotations

import os
import subprocess
import sysconfig
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIBRARY = os.path.join(HERE, "liboptimizer_update.so")
FAST = os.path.join(HERE, "_fast" + sysconfig.get_config_var("EXT_SUFFIX"))
SOURCES = [os.path.join(CSRC, "kernels.hip"), os.path.join(CSRC, "host.hip"),
           os.path.join(CSRC, "kernels8.hip"), os.path.join(CSRC, "host8.hip"),
           os.path.join(CSRC, "host_graph.hip"), os.path.join(CSRC, "probes.hip"),
           os.path.join(CSRC, "host_probes.hip")]
HEADERS = [os.path.join(CSRC, "elem.hpp"), os.path.join(CSRC, "internal.h"),
           os.path.join(CSRC, "host_internal.h"), os.path.join(CSRC, "qmap.hpp"),
           os.path.join(CSRC, "stepdiv.hpp"), os.path.join(CSRC, "ou_testing.h"),
           os.path.join(CSRC, "stream.hpp"),
           os.path.join(os.path.dirname(HERE), "include", "optimizer_update.h")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-command-line-argument",
]


def build(out_path: str = LIBRARY, extra_flags: list[str] | None = None, quiet: bool = True) -> str:
    """Compile the library (always; atomically replaces ``out_path``)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=os.path.dirname(out_path))
    os.close(fd)
    cmd = [hipcc, *HIPCC_FLAGS, *(extra_flags or []), "-o", tmp, *SOURCES]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
        if not quiet:
            print(r.stderr)
        os.replace(tmp, out_path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    build_fast()
    return out_path


def build_fast(out_path: str = FAST) -> str:
    """Compile the CPython module (gcc, linked to the library next to it)."""
    cc = os.environ.get("CC", "gcc")
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=os.path.dirname(out_path))
    os.close(fd)
    cmd = [cc, "-O2", "-std=c11", "-shared", "-fPIC", "-Wall", "-Werror",
           "-I", sysconfig.get_paths()["include"], os.path.join(CSRC, "pyfast.c"),
           "-L", HERE, "-loptimizer_update", "-Wl,-rpath,$ORIGIN", "-o", tmp]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("building _fast failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
        os.chmod(tmp, 0o755)
        os.replace(tmp, out_path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return out_path


if __name__ == "__main__":
    print(build(quiet=False))
