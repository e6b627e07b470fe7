"""Build libdsaidx.so in-tree for gfx950 with hipcc (run by __graft_entry__.build()).

Each source compiles to its own object in parallel (every kernel is launched from the file
that defines it, so no relocatable device code is needed), then hipcc links the library.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
SO = os.path.join(HERE, "libdsaidx.so")
SOURCES = ["api.cpp", "project.hip", "topk.hip", "decode.hip", "fp8.hip", "mla.hip", "rope.hip", "prefill.hip"]

# Packed fp32 arithmetic is switched off for the device code (see the design notes); the
# host pass only warns that it does not know the feature.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def _filter(text):
    return [l for l in text.splitlines() if "packed-fp32-ops" not in l]


def _compile(src, extra):
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    cmd = ["/opt/rocm/bin/hipcc", *FLAGS, *extra, "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r.returncode, _filter(r.stdout + r.stderr), cmd


def build(verbose=False, extra=(), jobs=None):
    os.makedirs(OBJ, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, list(extra)), SOURCES))
    failed = False
    for src, obj, rc, lines, cmd in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            failed = True
            sys.stderr.write("\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("hipcc failed building libdsaidx.so")
    link = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", *extra, "-o", SO + ".tmp",
            *[obj for _, obj, _, _, _ in results]]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("linking libdsaidx.so failed")
    os.replace(SO + ".tmp", SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
