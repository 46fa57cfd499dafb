"""Build libpaged_decode.so (and the bench's libpd_probe.so) for gfx950 with
hipcc (ahead of time, in-tree).

    python -m paged_kv_attention_14_amd.build

Every HIP source is compiled with packed-FP32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``): plain float code is
used instead.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpaged_decode.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
# Measurement aid for bench.py (the streaming-read ceiling), kept out of the
# decode library.
PROBE_SOURCE = "read_probe.hip"
PROBE_PATH = os.path.join(PKG, "libpd_probe.so")

SOURCES = ["decode_kernels.hip", "kv_write_kernels.hip", "check_kernels.hip",
           "paged_decode_abi.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; return its path."""
    cc = hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd.insert(1, "-xhip")
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB_PATH + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(tmp, LIB_PATH)
    build_probe(cc, verbose)
    return LIB_PATH


def build_probe(cc: str, verbose: bool = False) -> str:
    """Compile the streaming-read probe library bench.py uses."""
    tmp = PROBE_PATH + ".tmp"
    cmd = [cc, *compile_flags(), "-shared", os.path.join(CSRC, PROBE_SOURCE), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBE_PATH)
    return PROBE_PATH


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv or "--verbose" in sys.argv)
    print("built", path)
