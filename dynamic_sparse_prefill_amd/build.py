"""Build libcrisp.so (HIP for gfx950) in-tree with hipcc.

    python -m dynamic_sparse_prefill_amd.build      # or build() from Python

Every .hip source is compiled for gfx950 only; the host layer (crisp.cpp) is
compiled by hipcc as well so that it links against the HIP runtime.  Packed
fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcrisp.so")
ROOT = os.path.dirname(HERE)

SOURCES = ["crisp.cpp", "attn.hip", "proxy.hip", "select.hip"]
PROBE_LIB = os.path.join(HERE, "libcrisp_probe.so")   # attainable-peak probe used by the benchmark
PROBE_SOURCES = ["probe.hip"]
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
          f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False, jobs: int = 4) -> str:
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else ["-x", "hip"]
        cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len(procs) >= jobs:
            _wait(procs.pop(0), verbose)
    for p in procs:
        _wait(p, verbose)
    main_objs = [o for o, s in zip(objs, SOURCES + PROBE_SOURCES) if s in SOURCES]
    probe_objs = [o for o, s in zip(objs, SOURCES + PROBE_SOURCES) if s in PROBE_SOURCES]
    for lib, lobjs in ((LIB, main_objs), (PROBE_LIB, probe_objs)):
        tmp = lib + ".tmp"
        cmd = [hipcc(), *DEVICE_FLAGS, "-shared", "-fPIC", "-o", tmp, *lobjs]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout)
        os.replace(tmp, lib)
    return LIB


def _wait(item, verbose):
    src, p = item
    out, _ = p.communicate()
    lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l and "--hip-link" not in l]
    if p.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n" + "\n".join(lines))
    if verbose and lines:
        print("\n".join(lines), flush=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
