"""The causal count of one decode step, pinned by the page's printed score
shape (page "Similarities", decode mode at position 1000: the scores are
[B, 128 heads, 1 query, 1001 keys]). A query at position p sees keys
0..p, its own key included, so the oracle's whole decode step at p = 1000
must score exactly 1001 keys, and with a top-k budget of 2048 select all of
them; an off-by-one in n_valid (p or p + 2 keys) fails here."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decode_score_shape.json")


def test_decode_at_position_1000_scores_1001_keys():
    ref = json.load(open(GOLDEN))
    p, keys, Hq = ref["position"], ref["keys"], ref["heads"]
    L, H = 1100, 4                                   # cache longer than the causal prefix
    g = np.random.Generator(np.random.PCG64(1001))
    q_raw = g.standard_normal((1, 1, H, 128)).astype(np.float32)
    k_raw = g.standard_normal((1, L, 128)).astype(np.float32)
    w = g.standard_normal((1, 1, H)).astype(np.float32)
    q_mla = g.standard_normal((1, 1, Hq, 576)).astype(np.float32)
    latent = g.standard_normal((1, L, 512)).astype(np.float32)
    kpe = g.standard_normal((1, L, 64)).astype(np.float32)
    cos, sin = oracle.rope_table(L)
    res = oracle.decode_path(q_raw, k_raw, np.array([[p]], np.int32), w, cos, sin, q_mla,
                             latent, kpe, 2048, 192 ** -0.5, bf16_input=False)
    sc = res["scores"][0, 0]
    assert int(np.isfinite(sc).sum()) == keys
    assert np.all(np.isfinite(sc[:keys])) and np.all(np.isnan(sc[keys:]))
    idx = res["idx"][0, 0]
    assert int((idx >= 0).sum()) == keys
    np.testing.assert_array_equal(idx[:keys], np.arange(keys))
    assert res["out"].shape == (1, 1, Hq, 512) and np.all(np.isfinite(res["out"]))
