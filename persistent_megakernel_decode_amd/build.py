"""Build libmk.so (the megakernel, scheduler and C ABI) in-tree with hipcc for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
SOURCES = ["mk_kernel.hip", "mk_kernel_trace.hip", "mk_api.cpp", "mk_sched.cpp", "mk_emu.cpp"]
HEADERS = ["mk_internal.h", "mk_attn_plan.h", "mk_sched.h", os.path.join("..", "..", "include", "mk.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-x", "hip",
    # packed fp32 VALU ops are kept out of every kernel (they are not needed and are avoided on this part)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every loop starts on a 64-byte boundary: without it the persistent kernel's speed moved by
    # up to 2 % with unrelated code changes (the hot loops' placement in the instruction stream)
    "-falign-loops=64",
    "-Wno-unused-command-line-argument",
]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(os.path.join(CSRC, f)) > t for f in SOURCES + HEADERS)


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile libmk.so.  With force=False an up-to-date library is kept."""
    if not force and not stale():
        return LIB
    tmp = LIB + ".tmp"
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    # one hipcc per source, in parallel (the two kernel translation units dominate), then link
    procs = [subprocess.Popen([HIPCC, *FLAGS, "-c", src, "-o", obj], stdout=subprocess.PIPE,
                              stderr=subprocess.STDOUT, text=True) for src, obj in zip(sources(), objs)]
    results = [(p.communicate()[0], p.returncode) for p in procs]
    link = subprocess.run([HIPCC, *[f for f in FLAGS if f not in ("-x", "hip")], *objs, "-o", tmp],
                          capture_output=True, text=True)
    results.append((link.stdout + link.stderr, link.returncode))
    out = "\n".join(l for o, _ in results for l in o.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if any(rc != 0 for _, rc in results):
        raise RuntimeError(f"hipcc failed:\n{out}")
    if verbose and out:
        print(out, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
