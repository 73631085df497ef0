"""Build libdeltalog.so in-tree with hipcc for gfx950.

Usage: python -m linear_attention_recurrent_amd.build [--verbose] [--trace]

Each translation unit is compiled to an object (in parallel), then linked into
linear_attention_recurrent_amd/libdeltalog.so.  The benchmark's read-rate probe
is linked on its own into linear_attention_recurrent_amd/libdlprobe.so.  With
--trace, the library is also built with per-workgroup timestamps in the decode
kernel (DL_TRACE) as linear_attention_recurrent_amd/libdeltalog_trace.so, which
nothing loads by default (bench.py --trace does).  Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdeltalog.so")
SOURCES = ["decode.hip", "merge_mfma.hip", "eager.hip", "prefill.hip", "api.cpp"]
PROBE_LIB = os.path.join(PKG, "libdlprobe.so")
TRACE_LIB = os.path.join(PKG, "libdeltalog_trace.so")
PROBE_SOURCES = ["read_probe.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libdeltalog.so)")


def common_flags() -> list:
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # no packed fp32 instructions anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the feature
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, save_temps: bool = False, trace: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    probe_objs = []
    trace_objs = []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if save_temps:
            cmd += ["--save-temps"]
        (probe_objs if src in PROBE_SOURCES else objs).append(obj)
        cmds.append(cmd)
        if trace and src == "decode.hip":
            tobj = os.path.join(BUILD, "decode_trace.o")
            cmds.append([cc] + common_flags() + ["-DDL_TRACE", "-c", os.path.join(CSRC, src), "-o", tobj])
    if trace:
        trace_objs = [os.path.join(BUILD, "decode_trace.o")] + [o for o in objs if not o.endswith("decode.o")]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    libs = [(LIB, objs), (PROBE_LIB, probe_objs)] + ([(TRACE_LIB, trace_objs)] if trace else [])
    for lib, lib_objs in libs:
        tmp = lib + ".tmp"
        _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + lib_objs, verbose)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv, save_temps="--save-temps" in sys.argv, trace="--trace" in sys.argv))
