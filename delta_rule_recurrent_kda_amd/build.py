"""Build libkda.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkda.so")
# bandwidth probes for the benchmark's measured ceilings (not part of the scan library)
PROBE_SRC = os.path.join(CSRC, "bw_probe.hip")
PROBE_LIB = os.path.join(PKG, "libkda_probe.so")
SOURCES = [os.path.join(CSRC, "kda_fwd.hip"), os.path.join(CSRC, "kda_wy.hip"), os.path.join(CSRC, "kda_fused.hip"), os.path.join(CSRC, "kda_noalloc.hip"),
           os.path.join(CSRC, "kda_bwd.hip"),
           os.path.join(CSRC, "kda_conv.hip"),
           os.path.join(CSRC, "kda_api.cpp")]
HEADERS = [os.path.join(CSRC, "kda_internal.h"), os.path.join(CSRC, "kda_device.h"),
           os.path.join(ROOT, "include", "kda.h")]
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
               # packed fp32 VALU ops stay off on this target
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.sep not in c or os.path.exists(c)):
            return c
    raise RuntimeError("hipcc not found")


def _hipcc_shared(out: str, sources, verbose: bool) -> None:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *sources]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Build libkda.so and the benchmark's bandwidth probes (libkda_probe.so)."""
    _hipcc_shared(LIB, SOURCES, verbose)
    _hipcc_shared(PROBE_LIB, [PROBE_SRC], verbose)
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB) or not os.path.exists(PROBE_LIB):
        return True
    if os.path.getmtime(PROBE_SRC) > os.path.getmtime(PROBE_LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
