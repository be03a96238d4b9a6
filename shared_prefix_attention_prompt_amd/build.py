"""Builds libaugtree.so (the gfx950 HIP kernels + C ABI) in place, next to this file, and the
standalone issue-rate probe ``probe_rates`` (csrc/probe_rates.hip; not part of the library).

Every source is compiled with hipcc for gfx950 only, in parallel, then linked into one
shared library. Intermediate objects go to ``_build/`` beside the sources.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libaugtree.so")
PROBE = os.path.join(HERE, "probe_rates")
SOURCES = ["api.hip", "attn_fwd.hip", "attn_bwd.hip", "aux.hip", "planner.hip"]
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         # packed fp32 VALU forms stay disabled: plain float code only
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src: str) -> str:
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    return out


def _probe() -> str:
    tmp = PROBE + ".tmp"
    cmd = [HIPCC, *FLAGS, os.path.join(CSRC, "probe_rates.hip"), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for probe_rates.hip:\n{res.stderr}")
    os.replace(tmp, PROBE)
    return PROBE


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES) + 1, max(1, (os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        probe = ex.submit(_probe)
        objs = list(ex.map(_compile, SOURCES))
        probe.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
