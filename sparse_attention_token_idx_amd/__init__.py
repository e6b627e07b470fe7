"""Python binding of libdsaidx, the MI355X (gfx950) DSA lightning indexer forward pass.

Every function here is argument marshalling only: it checks dtypes and shapes, allocates
outputs and workspace with torch (torch supplies device memory and the current stream),
and calls the C-ABI entry point of the same name in ``libdsaidx.so``.  All computation
runs in the library's HIP kernels; there is no CPU or PyTorch fallback, and importing
fails loudly when the library has not been built.

bf16 tensors are ``torch.bfloat16``; index outputs are int32 and scores float32.
"""
import ctypes
import os

import torch

__all__ = ["version", "workspace_size", "project", "score_topk", "score_topk_varlen", "decode",
           "prefill_scores", "prefill_select", "score_row", "quantize_keys", "decode_fp8",
           "prefill_chunk", "sparse_mla", "OP_SPARSE_MLA", "HEADS", "DIM", "QLAT", "QOUT", "HIDDEN", "MAX_TOPK", "OP_PROJECT",
           "OP_SCORE_TOPK", "OP_SCORE_TOPK_VARLEN", "OP_DECODE", "OP_DECODE_FP8",
           "OP_PREFILL_CHUNK", "OP_PREFILL_ROWS", "OP_V32_SCORE_TOPK_VARLEN", "OP_V32_PREFILL_CHUNK",
           "prefill_rows_workspace", "decode_noalloc", "workspace_status", "set_wait_budget", "phase_timing", "phase_times", "PHASES", "EINVAL", "EUNSUPPORTED", "ESTALL", "arch_supported", "DsaIdxError", "lib"]

HEADS, DIM, QLAT, QOUT, HIDDEN, MAX_TOPK = 32, 128, 1536, 4096, 7168, 2048
OP_PROJECT, OP_SCORE_TOPK, OP_SCORE_TOPK_VARLEN, OP_DECODE, OP_DECODE_FP8 = 0, 1, 2, 3, 4
OP_PREFILL_CHUNK = 5
OP_SPARSE_MLA = 6
OP_V32_PROJECT, OP_V32_SCORE_TOPK = 7, 8
OP_V32_SCORE_TOPK_VARLEN, OP_V32_PREFILL_CHUNK, OP_PREFILL_ROWS = 9, 10, 11
EINVAL, EUNSUPPORTED, ESTALL = -1, -2, -5
MLA_HEADS, MLA_KV, MLA_V = 96, 576, 512
V32_HEADS, V32_QOUT, V32_THETA = 64, 8192, 10000.0   # the 64-head (DeepSeek-V3.2-shaped) indexer

_HERE = os.path.dirname(os.path.abspath(__file__))
# DSA_IDX_LIB names another build of the same library (e.g. the host-sanitizer build).
LIB_PATH = os.environ.get("DSA_IDX_LIB") or os.path.join(_HERE, "libdsaidx.so")


class DsaIdxError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with status {code}: {msg}")
        self.code = code


class _Weights(ctypes.Structure):
    _fields_ = [("W_q", ctypes.c_void_p), ("W_k", ctypes.c_void_p), ("W_w", ctypes.c_void_p),
                ("ln_gamma", ctypes.c_void_p), ("ln_beta", ctypes.c_void_p),
                ("ln_eps", ctypes.c_float)]


_lib = None


def lib():
    """The loaded libdsaidx (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950); there is no fallback path")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.dsa_idx_version.restype = ctypes.c_char_p
        L.dsa_idx_version.argtypes = []
        L.dsa_idx_last_error.restype = ctypes.c_char_p
        L.dsa_idx_last_error.argtypes = []
        L.dsa_idx_workspace_size.restype = i32
        L.dsa_idx_workspace_size.argtypes = [i32, i64, i32, i32, i32, ctypes.POINTER(sz)]
        L.dsa_idx_project.restype = i32
        L.dsa_idx_project.argtypes = [ctypes.POINTER(_Weights), vp, i64, vp, i64, i64, vp, vp, vp,
                                      vp, vp, sz, vp]
        L.dsa_idx_score_topk.restype = i32
        L.dsa_idx_score_topk.argtypes = [vp, vp, vp, i64, i32, vp, vp, vp, sz, vp]
        L.dsa_idx_score_topk_varlen.restype = i32
        L.dsa_idx_score_topk_varlen.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, vp, vp, vp,
                                                sz, vp]
        L.dsa_idx_prefill_scores.restype = i32
        L.dsa_idx_prefill_scores.argtypes = [vp, vp, vp, vp, i32, i32, i64, vp, sz, vp]
        L.dsa_idx_prefill_select.restype = i32
        L.dsa_idx_prefill_select.argtypes = [vp, i32, i32, i64, i32, vp, vp, vp, sz, vp]
        L.dsa_idx_prefill_chunk.restype = i32
        L.dsa_idx_prefill_chunk.argtypes = [vp, vp, vp, i64, i64, i32, vp, vp, vp, sz, vp]
        L.dsa_idx_v32_project.restype = i32
        L.dsa_idx_v32_project.argtypes = [ctypes.POINTER(_Weights), vp, i64, vp, i64, i64, i64,
                                          ctypes.c_float, vp, vp, vp, vp, sz, vp]
        L.dsa_idx_v32_score_topk.restype = i32
        L.dsa_idx_v32_score_topk.argtypes = [vp, vp, vp, i64, i32, vp, vp, vp, sz, vp]
        L.dsa_idx_v32_score_topk_varlen.restype = i32
        L.dsa_idx_v32_score_topk_varlen.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, vp, vp, vp,
                                                    sz, vp]
        L.dsa_idx_v32_prefill_chunk.restype = i32
        L.dsa_idx_v32_prefill_chunk.argtypes = [vp, vp, vp, i64, i64, i32, vp, vp, vp, sz, vp]
        L.dsa_idx_v32_decode.restype = i32
        L.dsa_idx_v32_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
        L.dsa_idx_v32_decode_fp8.restype = i32
        L.dsa_idx_v32_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
        L.dsa_idx_sparse_mla.restype = i32
        L.dsa_idx_sparse_mla.argtypes = [vp, vp, vp, vp, i64, i32, ctypes.c_float, vp, vp, vp, sz, vp]
        L.dsa_idx_decode_noalloc.restype = i32
        L.dsa_idx_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp]
        L.dsa_idx_decode.restype = i32
        L.dsa_idx_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
        L.dsa_idx_quantize_keys.restype = i32
        L.dsa_idx_quantize_keys.argtypes = [vp, i64, i64, vp, vp, vp, vp]
        L.dsa_idx_workspace_status.restype = i32
        L.dsa_idx_workspace_status.argtypes = [vp, sz, vp]
        L.dsa_idx_set_wait_budget.restype = i32
        L.dsa_idx_set_wait_budget.argtypes = [i32]
        L.dsa_idx_phase_timing.restype = i32
        L.dsa_idx_phase_timing.argtypes = [i32]
        L.dsa_idx_phase_times.restype = i32
        L.dsa_idx_phase_times.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int), i32]
        L.dsa_idx_arch_supported.restype = i32
        L.dsa_idx_arch_supported.argtypes = [ctypes.c_char_p]
        L.dsa_idx_decode_fp8.restype = i32
        L.dsa_idx_decode_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, sz, vp]
        L.dsa_idx_mfma_calibrate.restype = i32
        L.dsa_idx_mfma_calibrate.argtypes = [i64, i32, vp, sz, ctypes.POINTER(i64), vp]
        _lib = L
    return _lib


def version():
    return lib().dsa_idx_version().decode()


def arch_supported(arch_name):
    """Raise DsaIdxError unless the library runs on a device of this gcnArchName."""
    _check("dsa_idx_arch_supported", lib().dsa_idx_arch_supported(arch_name.encode()))


def _check(fn, code):
    if code != 0:
        raise DsaIdxError(fn, code, lib().dsa_idx_last_error().decode())


def workspace_size(op, total_tokens=0, B=0, max_seqlen=0, topk=MAX_TOPK):
    n = ctypes.c_size_t(0)
    _check("dsa_idx_workspace_size",
           lib().dsa_idx_workspace_size(op, int(total_tokens), int(B), int(max_seqlen), int(topk),
                                        ctypes.byref(n)))
    return n.value


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t, name, dtype, shape=None, contiguous=True):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return None
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes < {nbytes}")
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def project(x, c_q, weights, q=None, k_out=None, k_slot=None, w=None, stream=None):
    """q [T,32,128], k [T,128] (or rows k_slot of k_out), w [T,32] of one indexer layer.

    x [T,>=7168] and c_q [T,>=1536] are bf16 with unit stride along the row;
    weights = dict(W_q, W_k, W_w, gamma, beta, eps).  Returns (q, k_out, w).
    """
    T = x.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, contiguous=False)
    _need(c_q, "c_q", torch.bfloat16, contiguous=False)
    if x.stride(1) != 1 or c_q.stride(1) != 1 or c_q.shape[0] != T:
        raise ValueError("x and c_q need unit column stride and equal row counts")
    W = weights
    _need(W["W_q"], "W_q", torch.bfloat16, (QLAT, QOUT))
    _need(W["W_k"], "W_k", torch.bfloat16, (HIDDEN, DIM))
    _need(W["W_w"], "W_w", torch.bfloat16, (HIDDEN, HEADS))
    _need(W["gamma"], "gamma", torch.bfloat16, (DIM,))
    _need(W["beta"], "beta", torch.bfloat16, (DIM,))
    q = torch.empty((T, HEADS, DIM), dtype=torch.bfloat16, device=dev) if q is None else q
    w = torch.empty((T, HEADS), dtype=torch.bfloat16, device=dev) if w is None else w
    if k_out is None:
        k_out = torch.empty((T, DIM), dtype=torch.bfloat16, device=dev)
    _need(q, "q", torch.bfloat16, (T, HEADS, DIM))
    _need(w, "w", torch.bfloat16, (T, HEADS))
    _need(k_out, "k_out", torch.bfloat16)
    if k_out.dim() != 2 or k_out.shape[1] != DIM:
        raise ValueError("k_out must be [rows, 128]")
    if k_slot is not None:
        _need(k_slot, "k_slot", torch.int64, (T,))
    elif k_out.shape[0] < T:
        raise ValueError("k_out has fewer than T rows")
    wt = _Weights(_ptr(W["W_q"]), _ptr(W["W_k"]), _ptr(W["W_w"]), _ptr(W["gamma"]),
                  _ptr(W["beta"]), float(W["eps"]))
    nbytes = workspace_size(OP_PROJECT, T)
    ws = _workspace(nbytes, dev, None)
    _check("dsa_idx_project",
           lib().dsa_idx_project(ctypes.byref(wt), _ptr(x), x.stride(0), _ptr(c_q), c_q.stride(0),
                                 T, _ptr(q), _ptr(k_out), _ptr(k_slot), _ptr(w), _ptr(ws), nbytes,
                                 _stream(stream)))
    return q, k_out, w


def score_topk(q, k, w, topk=MAX_TOPK, with_scores=True, ws=None, out=None, stream=None):
    """Causal top-k of one sequence: q [T,32,128], k [T,128], w [T,32] -> idx [T,topk] int32,
    scores [T,topk] float32 (or None)."""
    T = q.shape[0]
    _need(q, "q", torch.bfloat16, (T, HEADS, DIM))
    _need(k, "k", torch.bfloat16, (T, DIM))
    _need(w, "w", torch.bfloat16, (T, HEADS))
    if out is None:
        idx = torch.empty((T, topk), dtype=torch.int32, device=q.device)
        sc = torch.empty((T, topk), dtype=torch.float32, device=q.device) if with_scores else None
    else:
        idx, sc = out
    nbytes = workspace_size(OP_SCORE_TOPK, T, topk=topk)
    ws = _workspace(nbytes, q.device, ws)
    _check("dsa_idx_score_topk",
           lib().dsa_idx_score_topk(_ptr(q), _ptr(k), _ptr(w), T, topk, _ptr(idx), _ptr(sc),
                                    _ptr(ws), nbytes, _stream(stream)))
    return idx, sc


def v32_project(x, c_q, weights, pos0=0, theta=V32_THETA, q=None, k=None, w=None, stream=None):
    """The 64-head indexer's projections with the rotary step, tokens at positions pos0 ..:
    q [T,64,128], k [T,128], w [T,64]; weights = dict(W_q [1536,8192], W_k [7168,128],
    W_w [7168,64], gamma, beta, eps)."""
    T = x.shape[0]
    dev = x.device
    _need(x, "x", torch.bfloat16, contiguous=False)
    _need(c_q, "c_q", torch.bfloat16, contiguous=False)
    if x.stride(1) != 1 or c_q.stride(1) != 1 or c_q.shape[0] != T:
        raise ValueError("x and c_q need unit column stride and equal row counts")
    W = weights
    _need(W["W_q"], "W_q", torch.bfloat16, (QLAT, V32_QOUT))
    _need(W["W_k"], "W_k", torch.bfloat16, (HIDDEN, DIM))
    _need(W["W_w"], "W_w", torch.bfloat16, (HIDDEN, V32_HEADS))
    _need(W["gamma"], "gamma", torch.bfloat16, (DIM,))
    _need(W["beta"], "beta", torch.bfloat16, (DIM,))
    q = torch.empty((T, V32_HEADS, DIM), dtype=torch.bfloat16, device=dev) if q is None else q
    k = torch.empty((T, DIM), dtype=torch.bfloat16, device=dev) if k is None else k
    w = torch.empty((T, V32_HEADS), dtype=torch.bfloat16, device=dev) if w is None else w
    _need(q, "q", torch.bfloat16, (T, V32_HEADS, DIM))
    _need(k, "k", torch.bfloat16, (T, DIM))
    _need(w, "w", torch.bfloat16, (T, V32_HEADS))
    wt = _Weights(_ptr(W["W_q"]), _ptr(W["W_k"]), _ptr(W["W_w"]), _ptr(W["gamma"]),
                  _ptr(W["beta"]), float(W["eps"]))
    nbytes = workspace_size(OP_V32_PROJECT, T)
    ws = _workspace(nbytes, dev, None)
    _check("dsa_idx_v32_project",
           lib().dsa_idx_v32_project(ctypes.byref(wt), _ptr(x), x.stride(0), _ptr(c_q), c_q.stride(0),
                                     T, int(pos0), float(theta), _ptr(q), _ptr(k), _ptr(w), _ptr(ws),
                                     nbytes, _stream(stream)))
    return q, k, w


def v32_score_topk(q, k, w, topk=MAX_TOPK, with_scores=True, ws=None, out=None, stream=None):
    """Causal top-k of one sequence for the 64-head indexer: q [T,64,128], k [T,128],
    w [T,64] -> idx [T,topk] int32, scores [T,topk] float32 (or None)."""
    T = q.shape[0]
    _need(q, "q", torch.bfloat16, (T, V32_HEADS, DIM))
    _need(k, "k", torch.bfloat16, (T, DIM))
    _need(w, "w", torch.bfloat16, (T, V32_HEADS))
    if out is None:
        idx = torch.empty((T, topk), dtype=torch.int32, device=q.device)
        sc = torch.empty((T, topk), dtype=torch.float32, device=q.device) if with_scores else None
    else:
        idx, sc = out
    nbytes = workspace_size(OP_V32_SCORE_TOPK, T, topk=topk)
    ws = _workspace(nbytes, q.device, ws)
    _check("dsa_idx_v32_score_topk",
           lib().dsa_idx_v32_score_topk(_ptr(q), _ptr(k), _ptr(w), T, topk, _ptr(idx), _ptr(sc),
                                        _ptr(ws), nbytes, _stream(stream)))
    return idx, sc


def v32_score_topk_varlen(q, k, w, cu_seqlens, max_seqlen, topk=MAX_TOPK, with_scores=True, ws=None,
                          out=None, stream=None):
    """Packed sequences for the 64-head indexer: q [total,64,128], k [total,128], w [total,64],
    cu_seqlens int32 [B+1] on the device; indices relative to each sequence's start."""
    total = q.shape[0]
    _need(q, "q", torch.bfloat16, (total, V32_HEADS, DIM))
    _need(k, "k", torch.bfloat16, (total, DIM))
    _need(w, "w", torch.bfloat16, (total, V32_HEADS))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    B = cu_seqlens.numel() - 1
    if out is None:
        idx = torch.empty((total, topk), dtype=torch.int32, device=q.device)
        sc = torch.empty((total, topk), dtype=torch.float32, device=q.device) if with_scores else None
    else:
        idx, sc = out
    nbytes = workspace_size(OP_V32_SCORE_TOPK_VARLEN, total, B, max_seqlen, topk)
    ws = _workspace(nbytes, q.device, ws)
    _check("dsa_idx_v32_score_topk_varlen",
           lib().dsa_idx_v32_score_topk_varlen(_ptr(q), _ptr(k), _ptr(w), _ptr(cu_seqlens), B,
                                               int(max_seqlen), total, topk, _ptr(idx), _ptr(sc),
                                               _ptr(ws), nbytes, _stream(stream)))
    return idx, sc


def score_topk_varlen(q, k, w, cu_seqlens, max_seqlen, topk=MAX_TOPK, with_scores=True, ws=None,
                      out=None, stream=None):
    """Packed sequences delimited by cu_seqlens (int32 [B+1] on the device); indices are
    relative to each sequence's start."""
    total = q.shape[0]
    _need(q, "q", torch.bfloat16, (total, HEADS, DIM))
    _need(k, "k", torch.bfloat16, (total, DIM))
    _need(w, "w", torch.bfloat16, (total, HEADS))
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    B = cu_seqlens.numel() - 1
    if out is None:
        idx = torch.empty((total, topk), dtype=torch.int32, device=q.device)
        sc = torch.empty((total, topk), dtype=torch.float32, device=q.device) if with_scores else None
    else:
        idx, sc = out
    nbytes = workspace_size(OP_SCORE_TOPK_VARLEN, total, B, max_seqlen, topk)
    ws = _workspace(nbytes, q.device, ws)
    _check("dsa_idx_score_topk_varlen",
           lib().dsa_idx_score_topk_varlen(_ptr(q), _ptr(k), _ptr(w), _ptr(cu_seqlens), B,
                                           int(max_seqlen), total, topk, _ptr(idx), _ptr(sc),
                                           _ptr(ws), nbytes, _stream(stream)))
    return idx, sc


def prefill_rows_workspace(total, cu_seqlens=None, max_seqlen=0, device="cuda"):
    """A workspace for prefill_scores / prefill_select (about 2 total^2 bytes for one
    sequence: every causal score is stored)."""
    B = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    nbytes = workspace_size(OP_PROJECT if total == 0 else OP_PREFILL_ROWS, total, B, max_seqlen)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)


def workspace_status(ws, stream=None):
    """Synchronizes `stream` and raises DsaIdxError (ESTALL) if a prefill call on this
    workspace reported that a score kernel's ring wait gave up."""
    nb = ws.numel() * ws.element_size()
    _check("dsa_idx_workspace_status", lib().dsa_idx_workspace_status(_ptr(ws), nb, _stream(stream)))


PHASES = ("sample", "threshold", "filter", "select", "fallback")


def phase_timing(enable):
    """Diagnostic: switch the event timing of the prefill top-k phases on (forgetting older
    records) or off."""
    _check("dsa_idx_phase_timing", lib().dsa_idx_phase_timing(1 if enable else 0))


def phase_times():
    """Synchronizes the recorded phase events; {phase: (total ms, launches)} since the last read."""
    n = len(PHASES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    _check("dsa_idx_phase_times", lib().dsa_idx_phase_times(ms, cnt, n))
    return {PHASES[i]: (ms[i], cnt[i]) for i in range(n)}


def set_wait_budget(polls):
    """Diagnostic: polls per ring wait of the prefill score kernels; returns the previous value."""
    return lib().dsa_idx_set_wait_budget(int(polls))


CALIB_SINK = 262144


def mfma_calibrate(iters, random_operands=True, sink=None, stream=None):
    """Calibration, not part of the indexer: launches the library's sustained-MFMA kernel
    (iters rounds of 16 independent bf16 products per wave, on register operands) on `stream`
    and returns (bf16 flop executed, sink).  Asynchronous; time it with events."""
    if sink is None:
        sink = torch.empty(CALIB_SINK, dtype=torch.float32, device="cuda")
    _need(sink, "sink", torch.float32)
    flop = ctypes.c_int64(0)
    _check("dsa_idx_mfma_calibrate", lib().dsa_idx_mfma_calibrate(int(iters), 1 if random_operands else 0,
                                                                  _ptr(sink), sink.numel(), ctypes.byref(flop),
                                                                  _stream(stream)))
    return flop.value, sink


def prefill_scores(q, k, w, ws, cu_seqlens=None, max_seqlen=0, stream=None):
    """Every causal fp32 score I[t, s], s <= t, into the workspace `ws` (prefill_rows_workspace;
    see score_row for the layout).  This stores the whole triangle; score_topk does not."""
    total = q.shape[0]
    _need(q, "q", torch.bfloat16, (total, HEADS, DIM))
    _need(k, "k", torch.bfloat16, (total, DIM))
    _need(w, "w", torch.bfloat16, (total, HEADS))
    B = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    nb = ws.numel() * ws.element_size()
    _check("dsa_idx_prefill_scores",
           lib().dsa_idx_prefill_scores(_ptr(q), _ptr(k), _ptr(w), _ptr(cu_seqlens), B,
                                        int(max_seqlen), total, _ptr(ws), nb, _stream(stream)))


def prefill_select(total, ws, topk=MAX_TOPK, with_scores=True, cu_seqlens=None, max_seqlen=0,
                   out=None, stream=None):
    """The row top-k of the score rows that prefill_scores left in `ws`."""
    B = 1 if cu_seqlens is None else cu_seqlens.numel() - 1
    if out is None:
        idx = torch.empty((total, topk), dtype=torch.int32, device=ws.device)
        sc = torch.empty((total, topk), dtype=torch.float32, device=ws.device) if with_scores else None
    else:
        idx, sc = out
    nb = ws.numel() * ws.element_size()
    _check("dsa_idx_prefill_select",
           lib().dsa_idx_prefill_select(_ptr(cu_seqlens), B, int(max_seqlen), total, topk,
                                        _ptr(idx), _ptr(sc), _ptr(ws), nb, _stream(stream)))
    return idx, sc


def score_row(ws, t, max_len, B=1, seq_base=0):
    """View of the t+1 causal scores of row t (of a sequence whose rows start at float offset
    seq_base of the row area) inside a prefill workspace; max_len is the T or max_seqlen of the
    call, B its sequence count (1 for the dense call)."""
    hdr = 256 + (8 * (B + 1) + 255) // 256 * 256
    dummy = (4 * ((max_len + 127) // 128) * 128 + 255) // 256 * 256
    q, r = divmod(t, 128)
    off = seq_base + 8192 * q * (q + 1) + 128 * r * (q + 1)
    rows = ws[hdr + dummy:].view(torch.float32)
    return rows[off:off + t + 1]


def prefill_chunk(q, k, w, prefix, topk=MAX_TOPK, with_scores=True, ws=None, out=None,
                  stream=None):
    """C query tokens at positions prefix .. prefix + C - 1 against the whole causal prefix:
    q [C,32,128], w [C,32], k [prefix + C, 128] (the cached keys, then the chunk's own) ->
    idx [C,topk] int32 (absolute positions), scores [C,topk] float32 (or None).  With
    q [C,64,128] and w [C,64], the 64-head indexer."""
    C = q.shape[0]
    heads = V32_HEADS if q.dim() == 3 and q.shape[1] == V32_HEADS else HEADS
    _need(q, "q", torch.bfloat16, (C, heads, DIM))
    _need(k, "k", torch.bfloat16, (prefix + C, DIM))
    _need(w, "w", torch.bfloat16, (C, heads))
    if out is None:
        idx = torch.empty((C, topk), dtype=torch.int32, device=q.device)
        sc = torch.empty((C, topk), dtype=torch.float32, device=q.device) if with_scores else None
    else:
        idx, sc = out
    nbytes = workspace_size(OP_V32_PREFILL_CHUNK if heads == V32_HEADS else OP_PREFILL_CHUNK, C, 0, prefix, topk)
    ws = _workspace(nbytes, q.device, ws)
    fn = "dsa_idx_v32_prefill_chunk" if heads == V32_HEADS else "dsa_idx_prefill_chunk"
    _check(fn, getattr(lib(), fn)(_ptr(q), _ptr(k), _ptr(w), C, int(prefix), topk, _ptr(idx),
                                  _ptr(sc), _ptr(ws), nbytes, _stream(stream)))
    return idx, sc


def sparse_mla(q, kv, idx, row0=None, scale=192.0 ** -0.5, with_lse=True, ws=None, out=None,
               stream=None):
    """Sparse MLA over the selected tokens: q [T,96,576] bf16 (absorbed queries), kv [*,576]
    bf16 (latent cache rows), idx [T,topk] int32 (-1: none), row0 int64 [T] or None ->
    o [T,96,512] bf16, lse [T,96] float32 (or None)."""
    T = q.shape[0]
    _need(q, "q", torch.bfloat16, (T, MLA_HEADS, MLA_KV))
    _need(kv, "kv", torch.bfloat16)
    if kv.dim() != 2 or kv.shape[1] != MLA_KV:
        raise ValueError("kv must be [rows, 576]")
    _need(idx, "idx", torch.int32)
    if idx.dim() != 2 or idx.shape[0] != T:
        raise ValueError("idx must be [T, topk]")
    topk = idx.shape[1]
    if row0 is not None:
        _need(row0, "row0", torch.int64, (T,))
    if out is None:
        o = torch.empty((T, MLA_HEADS, MLA_V), dtype=torch.bfloat16, device=q.device)
        lse = torch.empty((T, MLA_HEADS), dtype=torch.float32, device=q.device) if with_lse else None
    else:
        o, lse = out
    nbytes = workspace_size(OP_SPARSE_MLA, T, 0, 0, topk)
    ws = _workspace(nbytes, q.device, ws)
    _check("dsa_idx_sparse_mla",
           lib().dsa_idx_sparse_mla(_ptr(q), _ptr(kv), _ptr(idx), _ptr(row0), T, topk, float(scale),
                                    _ptr(o), _ptr(lse), _ptr(ws), nbytes, _stream(stream)))
    return o, lse


def decode(q, w, k_cache, start, seqlens, max_seqlen, topk=MAX_TOPK, with_scores=True, ws=None,
           out=None, stream=None):
    """One query per sequence against its cached keys: q [B,32,128], w [B,32],
    k_cache [*,128], start int64 [B], seqlens int32 [B] (own key included).  With q [B,64,128]
    and w [B,64], the 64-head indexer."""
    B = q.shape[0]
    heads = V32_HEADS if q.dim() == 3 and q.shape[1] == V32_HEADS else HEADS
    _need(q, "q", torch.bfloat16, (B, heads, DIM))
    _need(w, "w", torch.bfloat16, (B, heads))
    _need(k_cache, "k_cache", torch.bfloat16)
    _need(start, "start", torch.int64, (B,))
    _need(seqlens, "seqlens", torch.int32, (B,))
    if out is None:
        idx = torch.empty((B, topk), dtype=torch.int32, device=q.device)
        sc = torch.empty((B, topk), dtype=torch.float32, device=q.device) if with_scores else None
    else:
        idx, sc = out
    nbytes = workspace_size(OP_DECODE, 0, B, max_seqlen, topk)
    ws = _workspace(nbytes, q.device, ws)
    fn = "dsa_idx_v32_decode" if heads == V32_HEADS else "dsa_idx_decode"
    _check(fn, getattr(lib(), fn)(_ptr(q), _ptr(w), _ptr(k_cache), _ptr(start), _ptr(seqlens), B,
                                  int(max_seqlen), topk, _ptr(idx), _ptr(sc), _ptr(ws), nbytes,
                                  _stream(stream)))
    return idx, sc


def decode_noalloc(q, w, k_cache, start, seqlens, max_seqlen, topk=MAX_TOPK, with_scores=True, out=None,
                   stream=None):
    """decode (32 heads) through the entry point that allocates no device memory: its scratch is
    a static array inside the library.  Pass `out` (idx, scores) to allocate nothing here either."""
    B = q.shape[0]
    _need(q, "q", torch.bfloat16, (B, HEADS, DIM))
    _need(w, "w", torch.bfloat16, (B, HEADS))
    _need(k_cache, "k_cache", torch.bfloat16)
    _need(start, "start", torch.int64, (B,))
    _need(seqlens, "seqlens", torch.int32, (B,))
    if out is None:
        idx = torch.empty((B, topk), dtype=torch.int32, device=q.device)
        sc = torch.empty((B, topk), dtype=torch.float32, device=q.device) if with_scores else None
    else:
        idx, sc = out
    _check("dsa_idx_decode_noalloc",
           lib().dsa_idx_decode_noalloc(_ptr(q), _ptr(w), _ptr(k_cache), _ptr(start), _ptr(seqlens), B,
                                        int(max_seqlen), topk, _ptr(idx), _ptr(sc), _stream(stream)))
    return idx, sc


def quantize_keys(k, k8_out=None, scale_out=None, slot=None, stream=None):
    """FP8 cache rows of bf16 keys k [N,>=128] (unit column stride): codes uint8 [*,128] and
    scales float32 [*] (powers of two); row slot[i] (int64) or i.  Returns (k8_out, scale_out)."""
    N = k.shape[0]
    _need(k, "k", torch.bfloat16, contiguous=False)
    if k.dim() != 2 or k.stride(1) != 1 or k.shape[1] < DIM:
        raise ValueError("k must be [N, >=128] with unit column stride")
    if k8_out is None:
        k8_out = torch.empty((N, DIM), dtype=torch.uint8, device=k.device)
        scale_out = torch.empty((N,), dtype=torch.float32, device=k.device)
    _need(k8_out, "k8_out", torch.uint8)
    _need(scale_out, "scale_out", torch.float32)
    if k8_out.dim() != 2 or k8_out.shape[1] != DIM or scale_out.shape[0] != k8_out.shape[0]:
        raise ValueError("k8_out must be [rows, 128] and scale_out [rows]")
    if slot is not None:
        _need(slot, "slot", torch.int64, (N,))
    elif k8_out.shape[0] < N:
        raise ValueError("k8_out has fewer than N rows")
    _check("dsa_idx_quantize_keys",
           lib().dsa_idx_quantize_keys(_ptr(k), k.stride(0), N, _ptr(slot), _ptr(k8_out),
                                       _ptr(scale_out), _stream(stream)))
    return k8_out, scale_out


def decode_fp8(q, w, k8_cache, k_scale, start, seqlens, max_seqlen, topk=MAX_TOPK, with_scores=True,
               ws=None, out=None, stream=None):
    """As decode, against an FP8 cache: k8_cache uint8 [*,128], k_scale float32 [*].  With
    q [B,64,128] and w [B,64], the 64-head indexer."""
    B = q.shape[0]
    heads = V32_HEADS if q.dim() == 3 and q.shape[1] == V32_HEADS else HEADS
    _need(q, "q", torch.bfloat16, (B, heads, DIM))
    _need(w, "w", torch.bfloat16, (B, heads))
    _need(k8_cache, "k8_cache", torch.uint8)
    _need(k_scale, "k_scale", torch.float32)
    _need(start, "start", torch.int64, (B,))
    _need(seqlens, "seqlens", torch.int32, (B,))
    if out is None:
        idx = torch.empty((B, topk), dtype=torch.int32, device=q.device)
        sc = torch.empty((B, topk), dtype=torch.float32, device=q.device) if with_scores else None
    else:
        idx, sc = out
    nbytes = workspace_size(OP_DECODE_FP8, 0, B, max_seqlen, topk)
    ws = _workspace(nbytes, q.device, ws)
    fn = "dsa_idx_v32_decode_fp8" if heads == V32_HEADS else "dsa_idx_decode_fp8"
    _check(fn, getattr(lib(), fn)(_ptr(q), _ptr(w), _ptr(k8_cache), _ptr(k_scale), _ptr(start),
                                  _ptr(seqlens), B, int(max_seqlen), topk, _ptr(idx), _ptr(sc),
                                  _ptr(ws), nbytes, _stream(stream)))
    return idx, sc
