"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

Holds random-number generation only (no indexer arithmetic).  The native part
is ``gen.c`` (SplitMix64 counter streams + Box-Muller), built with gcc into
``libsynth.so`` next to it.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_SRC = os.path.join(_HERE, "gen.c")

# Stream ids: one unrelated counter stream per (seed, tensor, layer).
Q, K, W, X, CQ, WQ, WK, WW, GAMMA, BETA, KCACHE, SEQLEN = range(1, 13)


def build(force=False):
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        subprocess.check_call(["gcc", "-O2", "-std=gnu11", "-fopenmp", "-fPIC", "-shared",
                               _SRC, "-o", _SO + ".tmp", "-lm"])
        os.replace(_SO + ".tmp", _SO)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, i64, f64 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_normal_bf16.argtypes = [u64, u64, u64, f64, f64, i64, vp]
        L.synth_normal_bf16_range.argtypes = [u64, u64, u64, f64, f64, i64, i64, vp]
        L.synth_uniform_f64.argtypes = [u64, u64, u64, i64, vp]
        L.synth_uniform_int.argtypes = [u64, u64, u64, i64, i64, i64, vp]
        for f in (L.synth_normal_bf16, L.synth_normal_bf16_range, L.synth_uniform_f64,
                  L.synth_uniform_int):
            f.restype = None
        _lib = L
    return _lib


def normal_bf16(shape, mean, var, tensor, layer=0, seed=0, first=0):
    """bf16 bit patterns (uint16) of N(mean, var) samples; ``var`` is the variance.  The
    samples are elements first, first + 1, ... of the stream, so a slice of a large tensor
    can be drawn on its own."""
    out = np.empty(shape, dtype=np.uint16)
    lib().synth_normal_bf16_range(seed, tensor, layer, float(mean), float(np.sqrt(var)),
                                  int(first), out.size, out.ctypes.data)
    return out


def uniform_f64(n, tensor, layer=0, seed=0):
    out = np.empty(n, dtype=np.float64)
    lib().synth_uniform_f64(seed, tensor, layer, n, out.ctypes.data)
    return out


def uniform_int(n, lo, hi, tensor, layer=0, seed=0):
    """Integers uniform on [lo, hi] inclusive."""
    out = np.empty(n, dtype=np.int64)
    lib().synth_uniform_int(seed, tensor, layer, lo, hi, n, out.ctypes.data)
    return out
