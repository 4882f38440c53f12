"""Build step of libdeltalog: compiles the HIP sources for gfx950 with hipcc
and links ``libdeltalog.so`` next to this file (and ``libdlceiling.so``, the
benchmark's pattern-ceiling helper, from ``csrc/dl_ceiling.hip``).

    python recurrent_state_update_amd/_build.py

(run as a file, not as a module of the package: importing the package loads
the built library, which may be the stale one this step replaces).

Extra ``-D`` defines (for example a different value-tile width) can be passed
through ``build(defines=[...], out=...)`` to produce a variant library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdeltalog.so")
# the benchmark's pattern-ceiling helper, a library of its own (not part of
# the decode path)
CEILING_LIB = os.path.join(PKG, "libdlceiling.so")
SOURCES = ["dl_api.hip", "dl_device.hip", "dl_gdn.hip", "dl_kda.hip", "dl_rwkv6.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-fp32 instructions are switched off for all device code.
CFLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, obj: str, defines: list[str]) -> None:
    cmd = [HIPCC, *CFLAGS, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")


def build(defines: list[str] | None = None, out: str = LIB, build_dir: str | None = None,
          jobs: int = 4) -> str:
    """Compile every source (in parallel) and link the shared library."""
    defines = defines or []
    build_dir = build_dir or os.path.join(ROOT, "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = []
        for s in SOURCES:
            obj = os.path.join(build_dir, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            futs.append(ex.submit(_compile, os.path.join(CSRC, s), obj, defines))
        for f in futs:
            f.result()
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build_ceiling(out: str = CEILING_LIB) -> str:
    """Compile and link libdlceiling.so (csrc/dl_ceiling.hip), which bench.py
    loads to measure the HBM rate of the step kernel's own access pattern."""
    tmp = out + ".tmp"
    cmd = [HIPCC, *CFLAGS, "-shared", os.path.join(CSRC, "dl_ceiling.hip"), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on dl_ceiling.hip:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(defines=sys.argv[1:]))
    print(build_ceiling())
