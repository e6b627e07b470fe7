"""GPU parity of chunked prefill: C query tokens at positions prefix .. prefix + C - 1 scored
against the whole causal prefix ("Kimi K3.1 Pro vs Gemma 4 31B" page, long-context row: the
indexer scores every earlier token of a window of up to 1,048,576 tokens).

Row i of a chunk is row prefix + i of the causal problem, so it is checked against the
oracle's row prefix + i (keys 0 .. prefix + i), and against the library's own one-sequence
call on prefix + C tokens, whose rows must be the same bits (same kernels, same per-key
arithmetic, only the position offset differs)."""
import numpy as np
import pytest
import torch

import oracle
from synth import workloads as wl
from tests.helpers import check_row, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import sparse_attention_token_idx_amd as m
    assert torch.cuda.is_available()
    return m


def _chunk(dsa, prefix, C, seed, topk=2048):
    inp = wl.chunk_inputs(prefix, C, seed=seed)
    print(f"chunk: prefix={prefix} C={C} seed={seed} topk={topk}", flush=True)
    idx, sc = dsa.prefill_chunk(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["w"]), prefix, topk=topk)
    torch.cuda.synchronize()
    return inp, idx.cpu().numpy(), sc.cpu().numpy()


def _oracle_rows(inp, prefix, rows, topk):
    rows = np.asarray(rows, dtype=np.int64)
    return oracle.rows(inp["q"][rows], inp["w"][rows], inp["k"], np.zeros_like(rows), prefix + rows,
                       topk=topk, full=True)


@pytest.mark.parametrize("prefix,C", [(0, 3000), (2048, 1000), (1000, 777), (4093, 130), (77, 1)])
def test_chunk_rows_equal_whole_sequence_rows(dsa, prefix, C):
    # the last C rows of a one-sequence call on prefix + C tokens, bit for bit; offsets that are
    # not multiples of the 32-row blocks or the 128-key tiles make blocks straddle a tile edge
    inp, idx, sc = _chunk(dsa, prefix, C, seed=prefix + C)
    full = wl.score_inputs(prefix + C, seed=prefix + C)
    assert np.array_equal(full["k"], inp["k"]) and np.array_equal(full["q"][prefix:], inp["q"])
    fi, fs = dsa.score_topk(to_dev(full["q"]), to_dev(full["k"]), to_dev(full["w"]), topk=2048)
    torch.cuda.synchronize()
    assert np.array_equal(idx, fi.cpu().numpy()[prefix:])
    assert np.array_equal(sc.view(np.uint32), fs.cpu().numpy()[prefix:].view(np.uint32))


def test_chunk_against_oracle_every_row(dsa):
    prefix, C = 1000, 777
    inp, idx, sc = _chunk(dsa, prefix, C, seed=11)
    rows = np.arange(C)
    ref = _oracle_rows(inp, prefix, rows, 2048)
    for j, i in enumerate(rows):
        check_row(prefix + i, idx[i], sc[i], ref, j, 2048)


@pytest.mark.parametrize("topk", [2048, 100])
def test_chunk_long_rows(dsa, topk):
    # rows of 69,990 .. 70,289 keys (the 16-wave row top-k), sampled rows against the oracle
    prefix, C = 69990, 300
    inp, idx, sc = _chunk(dsa, prefix, C, seed=12, topk=topk)
    rows = [0, 1, 31, 32, 33, 100, 127, 128, 200, 299]
    ref = _oracle_rows(inp, prefix, rows, topk)
    for j, i in enumerate(rows):
        check_row(prefix + i, idx[i], sc[i], ref, j, topk)


def test_chunk_across_the_row_length_switch(dsa):
    # rows of up to 65,536 keys take the 4-wave row top-k, longer ones the 16-wave one
    prefix, C = 65536 - 200, 400
    inp, idx, sc = _chunk(dsa, prefix, C, seed=13)
    rows = [0, 198, 199, 200, 201, 399]
    ref = _oracle_rows(inp, prefix, rows, 2048)
    for j, i in enumerate(rows):
        check_row(prefix + i, idx[i], sc[i], ref, j, 2048)


def test_chunk_long_rows_all_equal_scores(dsa):
    # w = 0: every score is 0, so each row keeps its 2,048 lowest positions (ties go low)
    prefix, C = 70000, 64
    inp = wl.chunk_inputs(prefix, C, seed=14)
    w = np.zeros_like(inp["w"])
    idx, sc = dsa.prefill_chunk(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(w), prefix, topk=2048)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    assert np.array_equal(idx, np.broadcast_to(np.arange(2048, dtype=np.int32), idx.shape))
    assert np.all(sc == 0)


def test_chunk_at_the_end_of_a_1m_window(dsa):
    # the last 512 queries of a 1,048,576-token window: rows of about 1M keys
    C = 512
    prefix = 1048576 - C
    inp, idx, sc = _chunk(dsa, prefix, C, seed=15)
    rows = [0, 255, 511]
    ref = _oracle_rows(inp, prefix, rows, 2048)
    for j, i in enumerate(rows):
        check_row(prefix + i, idx[i], sc[i], ref, j, 2048)
