"""Build libdsaidx.so in-tree for gfx950 with hipcc (run by __graft_entry__.build()).

Each source compiles to its own object in parallel (every kernel is launched from the file
that defines it, so no relocatable device code is needed), then hipcc links the library.

build(sanitize=True) makes a second library under _build_san/ whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer checks (device code is built as usual).  It
does not link the sanitizer runtime: load it into a process that preloads clang's ASan runtime
(sanitizer_runtime()), with DSA_IDX_LIB naming the library for the Python binding.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
SO = os.path.join(HERE, "libdsaidx.so")
OBJ_SAN = os.path.join(HERE, "_build_san")
SO_SAN = os.path.join(OBJ_SAN, "libdsaidx.so")
SOURCES = ["api.cpp", "project.hip", "topk.hip", "decode.hip", "fp8.hip", "mla.hip", "prefill.hip", "calib.hip"]

# Packed fp32 arithmetic is switched off for the device code (see the design notes); the
# host pass only warns that it does not know the feature.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


# Host-only sanitizer flags (each -fsanitize= applies to the host pass only).
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def sanitizer_runtime():
    """Path of the ASan runtime (with UBSan) of the hipcc toolchain, for LD_PRELOAD."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def _filter(text):
    return [l for l in text.splitlines() if "packed-fp32-ops" not in l]


def _compile(src, extra, objdir):
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = ["/opt/rocm/bin/hipcc", *FLAGS, *extra, "-c", "-x", "hip", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    return src, obj, r.returncode, _filter(r.stdout + r.stderr), cmd


def build(verbose=False, extra=(), jobs=None, sanitize=False):
    objdir, so = (OBJ_SAN, SO_SAN) if sanitize else (OBJ, SO)
    extra = list(extra) + (SAN_FLAGS if sanitize else [])
    os.makedirs(objdir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, extra, objdir), SOURCES))
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
    link = ["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", so + ".tmp",
            *[obj for _, obj, _, _, _ in results]]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("linking libdsaidx.so failed")
    os.replace(so + ".tmp", so)
    return so


if __name__ == "__main__":
    print(build(verbose=True, sanitize="--sanitize" in sys.argv[1:]))
