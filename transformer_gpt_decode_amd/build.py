"""Build libgptdecode.so (the HIP decode library) in-tree with hipcc for gfx950.

No fast-math: the attention and argmax code rely on IEEE -inf/NaN behaviour.
Packed fp32 instructions are disabled (-packed-fp32-ops).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libgptdecode.so")
SRC = os.path.join(HERE, "csrc", "runtime.hip")
FLAGS = ["-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]


def build(verbose: bool = False, extra=()) -> str:
    cmd = ["hipcc", *FLAGS, *extra, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=[a for a in sys.argv[1:] if a != "-v"])
