"""GPU parity of call 2 (causal top-k) against the oracle: bit-exact indices
on identical score rows, ties to the lower position, -0 == +0, ascending
output, -1 padding."""
import numpy as np
import pytest

import oracle
import sparse_attention_index_amd as dsa
import synth
from gpu_util import check_topk_properties, dev, host, say

pytestmark = pytest.mark.gpu


def run_topk(scores_rows, n_valid, K, Lmax=None, sentinel=1e30, ws_fill=None):
    """scores_rows [R, L] float32 -> GPU idx [R, K] (rows as B=R, S=1).
    ws_fill: byte value the workspace holds before the call (its contents on
    entry must not matter)."""
    import torch
    R, L = scores_rows.shape
    Lmax = Lmax or L
    buf = np.full((R, 1, Lmax), np.float32(sentinel), np.float32)
    buf[:, 0, :L] = scores_rows
    for r, n in enumerate(n_valid):               # beyond the causal end: never read
        if 0 <= n <= Lmax:
            buf[r, 0, max(n, 0):] = np.float32(sentinel)
    pos = (np.asarray(n_valid, np.int64) - 1).astype(np.int32).reshape(R, 1)
    count = torch.empty((R, 1), dtype=torch.int32, device="cuda")
    d_sc, d_pos = dev(buf), dev(pos)
    ws = None
    if ws_fill is not None:
        ws = dsa.topk_workspace(d_sc, d_pos, K)
        ws.fill_(ws_fill)
    idx = dsa.topk(d_sc, d_pos, K, count=count, workspace=ws)
    torch.cuda.synchronize()
    return host(idx)[:, 0], host(count)[:, 0]


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "constant", "wide"])
@pytest.mark.parametrize("K", [1, 7, 32, 2048])
def test_topk_bit_exact_lds_rows(kind, K):
    L = 16384
    lens = [1, 2, 33, 100, 2047, 2048, 2049, 5000, 9999, 16383, 16384]
    sc = synth.topk_scores(1000 + K, len(lens), L, kind)
    say(f"topk lds rows kind={kind} K={K}")
    g, cnt = run_topk(sc, lens, K)
    o = oracle.topk(sc, lens, K)
    assert np.array_equal(g, o)
    assert np.array_equal(cnt, np.minimum(lens, K))


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "constant", "wide"])
@pytest.mark.parametrize("K", [1, 100, 2048])
def test_topk_bit_exact_long_rows(kind, K):
    """Rows past one selection block (16,384 scores): chunk lists, then one
    merge; lengths cover a one-score tail chunk, chunks past the causal end,
    a row that fits in its first chunk and rows shorter than K."""
    L = 131072
    lens = [131072, 16385, 40000, 70001, 12000, 1500, 0, 98305]
    sc = synth.topk_scores(2000 + K, len(lens), L, kind)
    say(f"topk long rows kind={kind} K={K}")
    g, cnt = run_topk(sc, lens, K, ws_fill=0xFF)
    o = oracle.topk(sc, lens, K)
    assert np.array_equal(g, o)
    assert np.array_equal(cnt, np.minimum(lens, K))
    check_topk_properties(sc, g, lens, K, kind)


@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_topk_multi_level_rows(kind):
    """2^21-score rows: 128 chunk lists, merged to 16, to 2, then the row."""
    L = 1 << 21
    lens = [L, 1_000_001]
    sc = synth.topk_scores(2500, len(lens), L, kind)
    say(f"topk 2M rows kind={kind}")
    g, cnt = run_topk(sc, lens, 2048, ws_fill=0x7F)
    o = oracle.topk(sc, lens, 2048)
    assert np.array_equal(g, o)
    assert np.array_equal(cnt, np.minimum(lens, 2048))


def test_topk_long_rows_many():
    """Many 32K rows of ragged lengths (two chunk lists per row)."""
    L = 32768
    g0 = np.random.default_rng(7)
    lens = g0.integers(0, L + 1, size=300).tolist()
    sc = synth.topk_scores(2600, len(lens), L, "ties")
    say("topk 300 rows of 32K")
    g, cnt = run_topk(sc, lens, 2048)
    o = oracle.topk(sc, lens, 2048)
    assert np.array_equal(g, o)


def test_topk_prefill_rows():
    """Prefill shape: row t keeps min(2048, t+1) of its t+1 causal scores."""
    T = 4096
    sc = synth.topk_scores(3000, T, T, "normal")
    n_valid = np.arange(1, T + 1)
    say("topk prefill 4096 rows")
    g, cnt = run_topk(sc, n_valid, 2048)
    o = oracle.topk(sc, n_valid, 2048)
    assert np.array_equal(g, o)
    assert np.array_equal(cnt, np.minimum(n_valid, 2048))


def test_topk_invalid_positions_give_empty_rows():
    import torch
    sc = np.zeros((3, 1, 64), np.float32)
    pos = np.array([[-1], [64], [-5]], np.int32)
    count = torch.full((3, 1), 9, dtype=torch.int32, device="cuda")
    idx = dsa.topk(dev(sc), dev(pos), 16, count=count)
    torch.cuda.synchronize()
    assert np.all(host(idx) == -1) and np.all(host(count) == 0)


def test_topk_is_deterministic():
    sc = synth.topk_scores(4000, 8, 16384, "ties")
    lens = [16384] * 8
    a, _ = run_topk(sc, lens, 2048)
    b, _ = run_topk(sc, lens, 2048)
    assert np.array_equal(a, b)
