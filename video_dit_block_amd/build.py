"""Build libvsa.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m video_dit_block_amd.build`` (or ``__graft_entry__.build()``).
Every call recompiles all sources; objects go to ``_build/`` at the repository
root and the library to ``video_dit_block_amd/libvsa.so``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libvsa.so")
# measurement aid of the benchmark (a bf16 MFMA ceiling loop), not the VSA path
PROBE_LIB = os.path.join(PKG, "libvsa_probe.so")

SOURCES = ["api.hip", "tile.hip", "select.hip", "fwd.hip", "coarse.hip", "lut.hip", "validate.hip"]
PROBE_SOURCES = ["mfma_peak.hip"]

ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 VALU instructions (v_pk_*_f32) in any kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libvsa")


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source, link libvsa.so and the benchmark's probe library;
    returns the path of libvsa.so."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = {}
    cmds = []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs[src] = obj
        cmds.append([cc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
        for cmd, fut in zip(cmds, [ex.submit(_run, c) for c in cmds]):
            if verbose:
                print(" ".join(cmd))
            fut.result()
    for lib, srcs in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        tmp = lib + ".tmp"
        link = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[objs[s] for s in srcs],
                "-o", tmp]
        if verbose:
            print(" ".join(link))
        _run(link)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
