"""Build libfa355.so (the HIP kernels and the C ABI) for gfx950, in-tree, the
unfused comparator's libfa355_unfused.so (the only one linked with rocBLAS),
and the fa355_ceilings calibration program.

Usage: ``python -m exact_io_aware_12_amd.build`` (or ``__graft_entry__.build()``).
Always recompiles. Needs only hipcc; no GPU is touched.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libfa355.so")
# The unfused comparator: its own library, the only one linked with rocBLAS.
LIB_UNFUSED = os.path.join(PKG, "libfa355_unfused.so")
# The race-check build of libfa355.so (FA_STRICT_SYNC: every global -> LDS
# copy awaited as soon as it is issued), compared bit for bit with the normal
# build by the GPU tests.
LIB_STRICT = os.path.join(PKG, "libfa355_strict.so")
# Calibration program (unit ceilings measured on the device), not linked into
# the library.
CEILINGS = os.path.join(PKG, "fa355_ceilings")
SOURCES = ["fa_fwd.hip", "fa_bwd.hip", "fa_decode.hip", "fa_fa1.hip", "fa_api.cpp"]
SOURCES_UNFUSED = ["fa_unfused.hip", "fa_unfused_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 VALU instructions are kept out of every kernel.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-fvisibility=hidden",
          "-Wno-unused-command-line-argument"]


def _compile(src: str, obj: str, extra: list[str]) -> None:
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if obj.endswith(".strict.o"):
        cmd.insert(-4, "-DFA_STRICT_SYNC")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
    if any("warning" in ln for ln in noise):
        sys.stderr.write("\n".join(noise) + "\n")


def _link(objs: list[str], out: str, libs: list[str]) -> None:
    cmd = [HIPCC, *COMMON, "-shared", *objs, "-o", out + ".tmp", *libs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(out + ".tmp", out)


def build(extra: list[str] | None = None) -> str:
    extra = list(extra or [])
    tmp = tempfile.mkdtemp(prefix="fa355_build_")
    try:
        jobs = [(s, os.path.join(tmp, s + ".o")) for s in SOURCES + SOURCES_UNFUSED]
        jobs += [(s, os.path.join(tmp, s + ".strict.o")) for s in SOURCES]
        with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 4)) as ex:
            list(ex.map(lambda j: _compile(j[0], j[1], extra), jobs))
        objs = dict(jobs[:len(SOURCES) + len(SOURCES_UNFUSED)])
        _link([objs[s] for s in SOURCES], LIB, [])
        _link([os.path.join(tmp, s + ".strict.o") for s in SOURCES], LIB_STRICT, [])
        # rocBLAS serves the two plain GEMMs of the unfused comparator only.
        _link([objs[s] for s in SOURCES_UNFUSED], LIB_UNFUSED, ["-L/opt/rocm/lib", "-lrocblas"])
        cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, os.path.join(CSRC, "ceilings.hip"), "-o",
               CEILINGS + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for ceilings.hip:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(CEILINGS + ".tmp", CEILINGS)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(sys.argv[1:]))
