"""Build the HIP library (libdsa.so, gfx950) in-tree with hipcc.

Usage: python -m sparse_attention_07_amd.build  [--save-temps]
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdsa.so")
# (source, object, extra defines): indexer.hip is built once per part (the
# planning kernel and dispatcher, then one index format each)
SOURCES = [("api.hip", "api", []), ("mla.hip", "mla", []), ("quant.hip", "quant", [])] + [
    ("indexer.hip", f"indexer{i}", [f"-DDSA_IDX_PART={i}"]) for i in range(5)]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU ops are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the device-only feature flag; that warning is noise
    noise = ("packed-fp32-ops", "warning generated", "warnings generated")
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if l.strip() and not any(n in l for n in noise)]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source to an object (in parallel: each translation unit
    holds its own kernels and their launchers), then link the shared library."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, o + ".o") for _, o, _ in SOURCES]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    cmds = [[HIPCC, *compile_flags, *defs, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
            for (src, _, defs), obj in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    extra = ["-save-temps"] if "--save-temps" in sys.argv else []
    print(build(verbose=True, extra=extra))
