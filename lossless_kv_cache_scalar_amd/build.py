"""Compile libskv.so for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC_DIR = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_lib", "libskv.so")

# -ffp-contract=off: the frequency model's fp32 operations must not be fused
# beyond the explicit fma the format specifies (encoder and decoder, GPU and
# CPU, take the same integer decisions).  Denormals are kept.  Packed fp32
# instructions are disabled.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(SRC_DIR, "*.hip")))


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"  # host pass only
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l and l.strip()]
    return res.returncode, msgs


def build(verbose: bool = False) -> str:
    """Each source compiled to an object in parallel, then one link."""
    os.makedirs(os.path.dirname(OUT), exist_ok=True)
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(os.path.dirname(OUT), "obj")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + SRC_DIR]
    objs, cmds = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmds.append([hipcc, *compile_flags, *inc, "-c", src, "-o", obj])
    msgs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        for (rc, m), cmd in zip(ex.map(_run, cmds), cmds):
            msgs += m
            if rc != 0:
                raise RuntimeError("hipcc failed on " + cmd[-3] + ":\n" + "\n".join(m))
    tmp = OUT + ".tmp"
    rc, m = _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    msgs += m
    if rc != 0:
        raise RuntimeError("hipcc link failed:\n" + "\n".join(m))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, OUT)
    return OUT


def is_built() -> bool:
    return os.path.exists(OUT)


if __name__ == "__main__":
    print(build(verbose=True))
