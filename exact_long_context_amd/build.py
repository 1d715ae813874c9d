"""Build librocring.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python exact_long_context_amd/build.py

Run it by path (or load it by file): importing the package itself needs the library.

Every source is compiled with packed-fp32 instruction selection switched off (the
host pass of hipcc warns that it does not know that feature; that is harmless),
then linked into ``exact_long_context_amd/librocring.so``.  Objects go to
``exact_long_context_amd/_build/``.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "librocring.so")

SOURCES = [
    "ra_api.cpp",
    "ra_ring.cpp",
    "ra_step_bf16.hip",
    "ra_step_f32.hip",
    "ra_finalize.hip",
    "ra_merge.hip",
    "ra_decode.hip",
    "ra_bwd.hip",
    "ra_bwd_bf16.hip",
]

ARCH = "gfx950"

# Per-source extra compiler flags (none needed at present).
EXTRA_FLAGS: dict[str, list[str]] = {}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-I", CSRC,
    ]


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link the library; returns the library path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [hipcc] + compile_flags() + EXTRA_FLAGS.get(src, []) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        while sum(p.poll() is None for _, p in procs) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        out = "\n".join(ln for ln in out.splitlines() if "packed-fp32-ops" not in ln)
        if p.returncode != 0:
            failed.append(f"--- {src} ---\n{out}")
        elif verbose and out.strip():
            print(out)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n".join(failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    # the library must load with every symbol resolved (a kernel whose host launch stub
    # was not emitted shows up here, not at first use); checked in a child process so
    # that this process maps no HIP runtime of its own
    chk = subprocess.run([sys.executable, "-c", "import ctypes, sys; ctypes.CDLL(sys.argv[1])", tmp],
                         stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if chk.returncode != 0:
        raise RuntimeError("built library does not load:\n" + chk.stdout.decode(errors="replace"))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
