"""The C-ABI library without a GPU: it loads, exports every declared symbol, sizes
workspaces, and rejects bad arguments before touching any device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsaidx.h")


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_token_idx_amd as m
    if not os.path.exists(m.LIB_PATH):
        from sparse_attention_token_idx_amd import build
        build.build()
    return m


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(dsa_idx_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(dsa):
    L = dsa.lib()
    names = declared_functions()
    assert set(names) == {"dsa_idx_version", "dsa_idx_last_error", "dsa_idx_workspace_size",
                          "dsa_idx_project", "dsa_idx_score_topk", "dsa_idx_score_topk_varlen",
                          "dsa_idx_prefill_scores", "dsa_idx_prefill_select", "dsa_idx_decode",
                          "dsa_idx_quantize_keys", "dsa_idx_decode_fp8", "dsa_idx_prefill_chunk",
                          "dsa_idx_sparse_mla", "dsa_idx_v32_project", "dsa_idx_v32_score_topk",
                          "dsa_idx_v32_score_topk_varlen", "dsa_idx_v32_prefill_chunk",
                          "dsa_idx_v32_decode", "dsa_idx_v32_decode_fp8", "dsa_idx_workspace_status",
                          "dsa_idx_set_wait_budget", "dsa_idx_phase_timing", "dsa_idx_phase_times",
                          "dsa_idx_decode_noalloc", "dsa_idx_arch_supported", "dsa_idx_mfma_calibrate"}
    for n in names:
        assert getattr(L, n) is not None


def test_version(dsa):
    assert "gfx950" in dsa.version()


def test_architecture_check(dsa):
    """The device check on architecture names (no device needed): gfx950 with any feature
    suffix runs; other gfx9 parts, near-miss names and the empty name are refused."""
    for name in ("gfx950", "gfx950:sramecc+:xnack-", "gfx950:xnack+"):
        dsa.arch_supported(name)
    for name in ("gfx942", "gfx942:sramecc+:xnack-", "gfx90a", "gfx9500", "gfx95", "gfx1100", "",
                 ":gfx950", "GFX950"):
        with pytest.raises(dsa.DsaIdxError) as e:
            dsa.arch_supported(name)
        assert e.value.code == dsa.EUNSUPPORTED and "gfx950 only" in str(e.value)
    assert dsa.lib().dsa_idx_arch_supported(None) == dsa.EINVAL


def test_workspace_sizes(dsa):
    # more than 64 tokens: W_q transposed (4096 x 1536 bf16)
    # more than 64 tokens, at most 32,768: then the [k | w] partial sums of its K slices (enough
    # slices that 64-row tiles x slices reach 1,024 workgroups, at most 56)
    def kw_slices(T):
        tiles = (T + 63) // 64
        return next((d for d in (1, 2, 4, 7, 8, 14, 16, 28, 56) if tiles * d >= 1024), 56)
    assert kw_slices(8192) == 8 and kw_slices(100) == 56 and kw_slices(32768) == 2
    for T in (100, 8192, 20000, 32768):
        assert dsa.workspace_size(dsa.OP_PROJECT, T) == 4096 * 1536 * 2 + 4 * kw_slices(T) * T * 160
    assert dsa.workspace_size(dsa.OP_PROJECT, 32769) == 4096 * 1536 * 2
    # a few tokens (at most 64) split K: fp32 partial sums, 6 slices of q and 56 of [k | w]
    assert dsa.workspace_size(dsa.OP_PROJECT, 64) == 4 * 64 * (6 * 4096 + 56 * 160)
    assert dsa.workspace_size(dsa.OP_PROJECT, 1) == 4 * (6 * 4096 + 56 * 160)
    # raw causal score rows: a 256-byte status header, the sequence bases (256-byte aligned), a
    # dummy row of 128*ceil(max/128) floats, and the triangular score rows (row t holds
    # 128*(t//128 + 1) floats)
    def tri(t):
        q, r = divmod(t, 128)
        return 8192 * q * (q + 1) + 128 * r * (q + 1)
    assert tri(1000) == sum(128 * (t // 128 + 1) for t in range(1000))
    r256 = lambda b: (b + 255) // 256 * 256
    assert dsa.workspace_size(dsa.OP_PREFILL_ROWS, 1000, 0, 0) == 256 + 256 + r256(4 * 1024) + 4 * tri(1000)
    # ragged: bound from sequences of max length (here 2 of length 8 -> (8+128)^2/2 floats each)
    vb = ((2 * 136 * 136 // 2 + 127) // 128) * 128
    assert dsa.workspace_size(dsa.OP_PREFILL_ROWS, 16, 2, 8) == 256 + 256 + 512 + 4 * vb
    # prefill top-k: the layout of the plan (a status header; per row of a filter chunk of at most
    # 65,536 rows a threshold, per (row, key segment) a count and a list of 6,144 (score, index)
    # pairs followed by 64 sentinel pairs
    # pairs; sample rows of ceil(n / 32 / 128) * 128 floats for a sub-chunk of at most 512 MB; a
    # fallback list; and 128 fallback scratch rows of the longest row, padded to 64)
    def plan(rows, heads=32, varlen=False, B=1, max_len=None, pos0=0):
        bq = 16 if heads == 64 else 32
        max_len = rows if max_len is None else max_len
        pos0 = 0 if varlen else pos0
        nkeys = pos0 + max_len
        cmax = 65536 if heads == 32 else 32768
        cf = -(-rows // -(-rows // cmax)) if rows else 0     # equal filter chunks
        lists = 0

        def dealt(n, p0, seg):
            # the busiest CU when the workgroups, row blocks (longest first) fastest and key
            # segments second, go to the 8 XCDs in turn and, in each, to the one of its 32 CUs
            # that frees first (each costing its key tiles + 2)
            busy = [[0] * 32 for _ in range(8)]
            nrb, mt = -(-n // bq), (p0 + n - 1) // 128 + 1
            i = 0
            for y in range(-(-mt // seg) if seg else 1):
                for x in range(nrb):
                    r0 = (nrb - 1 - x) * bq
                    nkt = (p0 + r0 + min(bq, n - r0) - 1) // 128 + 1
                    if y * seg < nkt:
                        cu = busy[i % 8]
                        cu[cu.index(min(cu))] += min(seg or nkt, nkt - y * seg) + 2
                    i += 1
            return max(max(cu) for cu in busy)

        for f0 in range(0, rows, cf):
            f1 = min(rows, f0 + cf)
            nseg = 1
            if not varlen:
                n, p0 = f1 - f0, pos0 + f0
                nrb, mt = -(-n // bq), (p0 + n - 1) // 128 + 1
                st = 0
                if 128 < nrb and 2 * nrb <= 3 * 256 and p0 < n:
                    # one or two rounds of workgroups: the longest row block in two segments (of
                    # at least 8 tiles) when that leaves the busiest CU less busy
                    half = -(-mt // 2)
                    st = half if half >= 8 and dealt(n, p0, half) < dealt(n, p0, 0) else 0
                else:
                    min_seg = 8 if nrb <= 128 else 64      # launches of few row blocks: short segments
                    if nrb < 2048 and mt > min_seg:
                        want = -(-2048 // nrb)
                        st = max(min_seg, -(-mt // want), -(-mt // 512))
                        st = st if st < mt else 0
                if st:
                    nseg = -(-mt // st)
            lists = max(lists, (cf if varlen else f1 - f0) * nseg)
        ms = -(-max(nkeys // 32, 1) // 128) * 128
        cs = max(bq, (512 * 2 ** 20 // (4 * ms)) // bq * bq)
        cs = min(cs, cf)
        ld = -(-max(nkeys, 1) // 64) * 64
        parts = [256, 4 * cf, 4 * lists, 8 * lists * (6144 + 64), 4 * cs * ms, 8 * cf, 4 * 128, 8 * 128,
                 4 * 128 * ld, 4 * max(ms, ld) + 4 * 128]
        return sum(r256(x) for x in parts)
    for T in (1, 300, 1000, 2560, 4096, 5000, 8192, 12000, 65536, 100000, 131073):
        assert dsa.workspace_size(dsa.OP_SCORE_TOPK, T, topk=2048) == plan(T), T
        assert dsa.workspace_size(dsa.OP_V32_SCORE_TOPK, T, topk=2048) == plan(T, heads=64), T
    assert dsa.workspace_size(dsa.OP_SCORE_TOPK_VARLEN, 16, 2, 8, topk=5) == plan(16, varlen=True, B=2, max_len=8)
    assert dsa.workspace_size(dsa.OP_V32_SCORE_TOPK_VARLEN, 177278, 16, 32768, topk=5) == \
        plan(177278, heads=64, varlen=True, B=16, max_len=32768)
    assert dsa.workspace_size(dsa.OP_PREFILL_CHUNK, 300, 0, 1000, 8) == plan(300, pos0=1000)
    assert dsa.workspace_size(dsa.OP_V32_PREFILL_CHUNK, 4096, 0, 10 ** 6, 8) == plan(4096, heads=64, pos0=10 ** 6)
    assert dsa.workspace_size(dsa.OP_PREFILL_CHUNK, 1000, 0, 0, 8) == dsa.workspace_size(dsa.OP_SCORE_TOPK, 1000, topk=8)
    assert dsa.workspace_size(dsa.OP_PREFILL_CHUNK, 0, 0, 5000, 8) == 0
    # no T x T matrix: the top-k workspace grows at most linearly in T, and a 1,048,576-token
    # sequence needs a few GB where its score triangle alone would take 2.2 TB
    big = [dsa.workspace_size(dsa.OP_SCORE_TOPK, T, topk=2048) for T in (2 ** 16, 2 ** 18, 2 ** 20, 2 ** 22)]
    assert all(b2 <= 4 * b1 for b1, b2 in zip(big, big[1:]))
    assert big[2] < 5 * 2 ** 30 and 4 * tri(2 ** 20) > 2 * 10 ** 12
    # decode: 256-byte aligned parts over the padded positions P = B * 64 * ceil(max / 64):
    # B + 1 cache offsets, B plans (8 bytes), P / 64 + 1 piece counts, P candidate slots of
    # 8 bytes, P fp32 scores, 8,192 sampled score keys per sequence; FP8 adds the quantised
    # queries (B x 4096 bytes) and their folded head weights (B x 32 fp32)
    def dec(B, m, fp8=False):
        P = B * 64 * ((m + 63) // 64)
        n = (r256(8 * (B + 1)) + r256(8 * B) + r256(4 * (P // 64 + 1)) + r256(8 * P) + r256(4 * P)
             + r256(4 * 8192 * B))
        return n + (r256(B * 2 * 4096) + r256(2 * 128 * B) if fp8 else 0)   # room for 64 heads
    assert dec(64, 131072) == 101189120 + 2097152 and dec(3, 100) == 5376 + 98304
    assert dsa.workspace_size(dsa.OP_DECODE, 0, 64, 131072, 2048) == dec(64, 131072)
    assert dsa.workspace_size(dsa.OP_DECODE, 0, 3, 100, 8) == dec(3, 100)
    assert dsa.workspace_size(dsa.OP_DECODE_FP8, 0, 3, 100, 8) == dec(3, 100, True)
    # sparse MLA: the splits' fp32 partial outputs and (max, sum) per (split, query, head), only
    # when a query's selections are split over several workgroups (few queries)
    assert dsa.workspace_size(dsa.OP_SPARSE_MLA, 5000, 0, 0, 2048) == 0
    n64 = dsa.workspace_size(dsa.OP_SPARSE_MLA, 64, 0, 0, 2048)
    assert n64 > 0 and n64 % (64 * 96 * (512 * 2 + 8)) == 0
    with pytest.raises(dsa.DsaIdxError) as e:
        dsa.workspace_size(dsa.OP_SCORE_TOPK, 10, topk=0)
    assert e.value.code == -2
    with pytest.raises(dsa.DsaIdxError) as e:
        dsa.workspace_size(99, 10)
    assert e.value.code == -1


def _vp(x):
    return ctypes.c_void_p(x)


def test_rejections_before_device(dsa):
    L = dsa.lib()
    A = 0x10000   # a fake, aligned "device" address: never dereferenced on these paths
    # topk out of range
    assert L.dsa_idx_score_topk(_vp(A), _vp(A), _vp(A), 10, 0, _vp(A), None, _vp(A), 1 << 30, None) == -2
    assert b"topk" in L.dsa_idx_last_error()
    assert L.dsa_idx_score_topk(_vp(A), _vp(A), _vp(A), 10, 2049, _vp(A), None, _vp(A), 1 << 30, None) == -2
    # negative T, null pointers, misalignment, small workspace
    assert L.dsa_idx_score_topk(_vp(A), _vp(A), _vp(A), -1, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert L.dsa_idx_score_topk(None, _vp(A), _vp(A), 10, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert L.dsa_idx_score_topk(_vp(A + 2), _vp(A), _vp(A), 10, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert L.dsa_idx_score_topk(_vp(A), _vp(A), _vp(A), 10, 8, _vp(A), None, _vp(A), 10, None) == -3
    assert b"workspace" in L.dsa_idx_last_error()
    # T = 0 is a no-op that succeeds without a device
    assert L.dsa_idx_score_topk(None, None, None, 0, 8, None, None, None, 0, None) == 0
    # varlen
    assert L.dsa_idx_score_topk_varlen(_vp(A), _vp(A), _vp(A), None, 2, 8, 10, 8, _vp(A), None,
                                       _vp(A), 1 << 30, None) == -1
    assert L.dsa_idx_score_topk_varlen(_vp(A), _vp(A), _vp(A), _vp(A), -1, 8, 10, 8, _vp(A), None,
                                       _vp(A), 1 << 30, None) == -1
    # the two prefill halves
    assert L.dsa_idx_prefill_scores(_vp(A), _vp(A), _vp(A), None, 1, 0, 10, _vp(A), 10, None) == -3
    assert L.dsa_idx_prefill_scores(None, _vp(A), _vp(A), None, 1, 0, 10, _vp(A), 1 << 30, None) == -1
    assert L.dsa_idx_prefill_scores(_vp(A), _vp(A), _vp(A), None, 1, 0, -5, _vp(A), 1 << 30, None) == -1
    assert L.dsa_idx_prefill_select(None, 1, 0, 10, 0, _vp(A), None, _vp(A), 1 << 30, None) == -2
    assert L.dsa_idx_prefill_select(None, 1, 0, 10, 8, None, None, _vp(A), 1 << 30, None) == -1
    assert L.dsa_idx_prefill_select(_vp(A), 2, 4, 10, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert b"B * max_seqlen" in L.dsa_idx_last_error()
    assert L.dsa_idx_prefill_select(None, 1, 0, 0, 8, None, None, None, 0, None) == 0
    # the MFMA calibration kernel: iteration count, sink size, null pointers
    import ctypes
    flop = ctypes.c_int64(0)
    assert L.dsa_idx_mfma_calibrate(0, 1, _vp(A), dsa.CALIB_SINK, ctypes.byref(flop), None) == -1
    assert L.dsa_idx_mfma_calibrate(10, 1, _vp(A), dsa.CALIB_SINK - 1, ctypes.byref(flop), None) == -1
    assert b"sink_floats" in L.dsa_idx_last_error()
    assert L.dsa_idx_mfma_calibrate(10, 1, None, dsa.CALIB_SINK, ctypes.byref(flop), None) == -1
    assert L.dsa_idx_mfma_calibrate(10, 1, _vp(A), dsa.CALIB_SINK, None, None) == -1
    # decode
    assert L.dsa_idx_decode(_vp(A), _vp(A), _vp(A), _vp(A), _vp(A), 4, 100, 0, _vp(A), None, _vp(A),
                            1 << 30, None) == -2
    assert L.dsa_idx_decode(_vp(A), _vp(A), _vp(A), None, _vp(A), 4, 100, 8, _vp(A), None, _vp(A),
                            1 << 30, None) == -1
    assert L.dsa_idx_decode(_vp(A), _vp(A), _vp(A), _vp(A), _vp(A), 4, 100, 8, _vp(A), None, _vp(A),
                            16, None) == -3
    assert L.dsa_idx_decode(None, None, None, None, None, 0, 0, 8, None, None, None, 0, None) == 0
    # FP8 cache
    assert L.dsa_idx_quantize_keys(_vp(A), 128, -1, None, _vp(A), _vp(A), None) == -1
    assert L.dsa_idx_quantize_keys(_vp(A), 100, 4, None, _vp(A), _vp(A), None) == -1
    assert L.dsa_idx_quantize_keys(_vp(A + 2), 128, 4, None, _vp(A), _vp(A), None) == -1
    assert L.dsa_idx_quantize_keys(None, 128, 0, None, None, None, None) == 0
    assert L.dsa_idx_decode_fp8(_vp(A), _vp(A), _vp(A), _vp(A), _vp(A), _vp(A), 4, 100, 0, _vp(A), None,
                                _vp(A), 1 << 30, None) == -2
    assert L.dsa_idx_decode_fp8(_vp(A), _vp(A), _vp(A), None, _vp(A), _vp(A), 4, 100, 8, _vp(A), None,
                                _vp(A), 1 << 30, None) == -1
    assert L.dsa_idx_decode_fp8(_vp(A), _vp(A), _vp(A), _vp(A), _vp(A), _vp(A), 4, 100, 8, _vp(A), None,
                                _vp(A), 16, None) == -3
    # chunked prefill
    chunk = lambda *a: L.dsa_idx_prefill_chunk(*a)
    assert chunk(_vp(A), _vp(A), _vp(A), 10, 100, 0, _vp(A), None, _vp(A), 1 << 30, None) == -2
    assert chunk(_vp(A), _vp(A), _vp(A), -1, 100, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert chunk(_vp(A), _vp(A), _vp(A), 10, -1, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert chunk(_vp(A), None, _vp(A), 10, 100, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert chunk(_vp(A), _vp(A + 8), _vp(A), 10, 100, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert chunk(_vp(A), _vp(A), _vp(A), 10, 100, 8, _vp(A), None, _vp(A), 16, None) == -3
    assert chunk(_vp(A), _vp(A), _vp(A), 4096, (1 << 24) - 4095, 8, _vp(A), None, _vp(A), 1 << 62,
                 None) == -2
    assert b"keys above 16777216" in L.dsa_idx_last_error()
    assert chunk(None, None, None, 0, 100, 8, None, None, None, 0, None) == 0
    # sparse MLA
    mla = lambda *a: L.dsa_idx_sparse_mla(*a)
    f = ctypes.c_float
    assert mla(_vp(A), _vp(A), _vp(A), None, 4, 0, f(0.1), _vp(A), None, _vp(A), 1 << 30, None) == -2
    assert mla(_vp(A), _vp(A), _vp(A), None, -1, 8, f(0.1), _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert mla(_vp(A), None, _vp(A), None, 4, 8, f(0.1), _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert mla(_vp(A + 4), _vp(A), _vp(A), None, 4, 8, f(0.1), _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert mla(_vp(A), _vp(A), _vp(A), None, 4, 8, f(0.0), _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert mla(_vp(A), _vp(A), _vp(A), None, 64, 2048, f(0.1), _vp(A), None, _vp(A), 16, None) == -3
    assert mla(None, None, None, None, 0, 8, f(0.1), None, None, None, 0, None) == 0
    # 64-head indexer: the score call has the one-sequence rules, its workspace the same size
    v32 = lambda *a: L.dsa_idx_v32_score_topk(*a)
    assert v32(_vp(A), _vp(A), _vp(A), 100, 0, _vp(A), None, _vp(A), 1 << 30, None) == -2
    assert v32(_vp(A), _vp(A), _vp(A), -1, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert v32(_vp(A), None, _vp(A), 100, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert v32(_vp(A), _vp(A + 8), _vp(A), 100, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert v32(_vp(A), _vp(A), _vp(A), 100, 8, _vp(A), None, _vp(A), 16, None) == -3
    assert v32(None, None, None, 0, 8, None, None, None, 0, None) == 0
    vv = lambda *a: L.dsa_idx_v32_score_topk_varlen(*a)
    assert vv(_vp(A), _vp(A), _vp(A), None, 2, 100, 150, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert vv(_vp(A), _vp(A), _vp(A), _vp(A), -1, 100, 150, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert vv(_vp(A), _vp(A), _vp(A), _vp(A), 2, 100, 150, 0, _vp(A), None, _vp(A), 1 << 30, None) == -2
    assert vv(_vp(A), _vp(A), _vp(A), _vp(A), 2, 100, 150, 8, _vp(A), None, _vp(A), 16, None) == -3
    assert vv(None, None, None, None, 0, 0, 0, 8, None, None, None, 0, None) == 0
    vd = lambda *a: L.dsa_idx_v32_decode(*a)
    assert vd(_vp(A), _vp(A), _vp(A), _vp(A), _vp(A), 4, 100, 0, _vp(A), None, _vp(A), 1 << 30, None) == -2
    assert vd(_vp(A), _vp(A), _vp(A), _vp(A), _vp(A), -1, 100, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert vd(_vp(A), None, _vp(A), _vp(A), _vp(A), 4, 100, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert vd(_vp(A), _vp(A), _vp(A), _vp(A), _vp(A), 4, 100, 8, _vp(A), None, _vp(A), 16, None) == -3
    assert vd(None, None, None, None, None, 0, 0, 8, None, None, None, 0, None) == 0
    vc = lambda *a: L.dsa_idx_v32_prefill_chunk(*a)
    assert vc(_vp(A), _vp(A), _vp(A), 10, 100, 0, _vp(A), None, _vp(A), 1 << 30, None) == -2
    assert vc(_vp(A), _vp(A), _vp(A), 10, -1, 8, _vp(A), None, _vp(A), 1 << 30, None) == -1
    assert vc(_vp(A), _vp(A), _vp(A), 10, 100, 8, _vp(A), None, _vp(A), 16, None) == -3
    assert vc(None, None, None, 0, 100, 8, None, None, None, 0, None) == 0
    # the 64-head projection in one pass: W_q transposed (8,192 x 1,536 bf16) above 64 tokens, the
    # split-K partial sums of 8,192 + 192 columns at most 64 tokens, then (256-byte aligned) the
    # rotary table, (cos, sin) in fp32 for 32 pairs of every token
    r256 = lambda b: (b + 255) // 256 * 256
    assert dsa.workspace_size(dsa.OP_V32_PROJECT, 100) == r256(8192 * 1536 * 2 + 4 * 56 * 100 * 192) + 100 * 32 * 8
    assert dsa.workspace_size(dsa.OP_V32_PROJECT, 7) == r256(4 * 7 * (6 * 8192 + 56 * 192)) + 7 * 32 * 8


def test_v32_project_rejections(dsa):
    L = dsa.lib()
    A = 0x10000
    W = dsa._Weights(A, A, A, A, A, 1e-6)
    f = ctypes.c_float

    def call(wt=W, ldx=7168, ldc=1536, T=4, pos0=0, theta=1e4, q=_vp(A), k=_vp(A), w=_vp(A), x=_vp(A),
             ws=_vp(A), nbytes=1 << 30):
        return L.dsa_idx_v32_project(ctypes.byref(wt) if wt is not None else None, x, ldx, _vp(A), ldc, T,
                                     pos0, f(theta), q, k, w, ws, nbytes, None)
    assert call(wt=None) == -1
    assert call(T=-1) == -1
    assert call(pos0=-5) == -1
    assert call(theta=0.0) == -1
    assert call(ldx=7000) == -1
    assert call(ldc=1537) == -1
    assert call(k=None) == -1
    assert call(x=_vp(A + 8)) == -1
    assert call(wt=dsa._Weights(A, A, A, A, A, 0.0)) == -1
    assert call(T=4, ws=None, nbytes=0) == -3
    assert call(T=0) == 0


def test_project_rejections(dsa):
    L = dsa.lib()
    A = 0x10000
    W = dsa._Weights(A, A, A, A, A, 1e-6)
    args = lambda **kw: dict(dict(x=_vp(A), ldx=7168, c_q=_vp(A), ldc=1536, T=4, q=_vp(A),
                                  k=_vp(A), slot=None, w=_vp(A)), **kw)

    def call(wt=W, **kw):
        a = args(**kw)
        return L.dsa_idx_project(ctypes.byref(wt) if wt is not None else None, a["x"], a["ldx"],
                                 a["c_q"], a["ldc"], a["T"], a["q"], a["k"], a["slot"], a["w"],
                                 None, 0, None)
    assert call(wt=None) == -1
    assert call(T=-1) == -1
    assert call(ldx=7000) == -1
    assert call(ldx=7172) == -1          # not a multiple of 8
    assert call(ldc=1535) == -1
    assert call(q=None) == -1
    assert call(x=_vp(A + 8)) == -1       # misaligned
    W0 = dsa._Weights(A, A, A, A, A, 0.0)
    assert call(wt=W0) == -1             # eps must be positive
    assert call(T=0) == 0
    # T <= 64 needs the split-K workspace
    a = args(T=4)
    assert L.dsa_idx_project(ctypes.byref(W), a["x"], a["ldx"], a["c_q"], a["ldc"], 4, a["q"], a["k"],
                             None, a["w"], None, 0, None) == -3
