"""Build libexact_attn.so in-tree with hipcc for gfx950.

Usage: python -m exact_io_aware_71_amd.build   (or call build()).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libexact_attn.so")
SOURCES = ["api.hip", "fwd.hip", "bwd.hip", "decode.hip"]
# Benchmark calibration (a streaming HBM read), kept out of the attention library.
CALIB_LIB = os.path.join(PKG, "libexact_calib.so")
CALIB_SOURCE = "calib.hip"

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # Keep packed fp32 VALU ops out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-parameter", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, extra_flags=None) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    flags = HIPCC_FLAGS + list(extra_flags or [])
    procs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src.replace(".hip", ".o"))
        cmd = [hipcc] + [f for f in flags if f != "-shared"] + ["-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = False
    for cmd, p in procs:
        out, _ = p.communicate()
        if verbose or p.returncode != 0:
            sys.stderr.write(" ".join(cmd) + "\n" + _filter(out))
        failed |= p.returncode != 0
    if failed:
        raise RuntimeError("hipcc failed to compile the attention kernels")
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        sys.stderr.write(p.stdout)
        raise RuntimeError("hipcc failed to link libexact_attn.so")
    os.replace(tmp, LIB)
    tmp = CALIB_LIB + ".tmp"
    cmd = [hipcc] + flags + ["-o", tmp, os.path.join(CSRC, CALIB_SOURCE)]
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if p.returncode != 0:
        sys.stderr.write(_filter(p.stdout))
        raise RuntimeError("hipcc failed to build libexact_calib.so")
    os.replace(tmp, CALIB_LIB)
    return LIB


def _filter(out: str) -> str:
    # The host pass does not know the packed-fp32 target feature; that warning is noise.
    return "".join(l for l in out.splitlines(True) if "packed-fp32-ops" not in l)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
