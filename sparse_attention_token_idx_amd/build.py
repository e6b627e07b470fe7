"""Build libdsaidx.so in-tree for gfx950 with hipcc (run by __graft_entry__.build())."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libdsaidx.so")
SOURCES = ["api.cpp", "project.hip", "scores.hip", "topk.hip", "decode.hip", "fp8.hip", "mla.hip", "rope.hip"]

# Packed fp32 arithmetic is switched off for the device code (see the design notes); the
# host pass only warns that it does not know the feature.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def build(verbose=False):
    cmd = ["/opt/rocm/bin/hipcc", *FLAGS, "-o", SO + ".tmp"]
    for s in SOURCES:
        if s.endswith(".cpp"):
            cmd += ["-x", "hip", os.path.join(CSRC, s)]
        else:
            cmd += [os.path.join(CSRC, s)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    lines = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError("hipcc failed building libdsaidx.so")
    if verbose and lines:
        print("\n".join(lines))
    os.replace(SO + ".tmp", SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
