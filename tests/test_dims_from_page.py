"""The dimensions the workloads use, pinned by the page's parameter table
(page "Sparse latent attention", table "Exact per-instance accounting").

Re-deriving every printed count from (model width 7168, query rank 1536,
latent 512, rotary key 64, 128 heads of 128+64 query / 128 value features,
64 indexer heads of 128 features sharing one 128-feature key per position)
fixes H_I = 64, d = 128, the single shared indexer key, and the 512 + 64
cached features that the kernels stream.
"""
import json
import os

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "attention_params.json")


def test_parameter_table_fixes_the_dimensions():
    ref = json.load(open(GOLDEN))
    dim, q_rank = 7168, 1536
    wl = synth.workload("decode16k")
    H_I, d = wl.H, synth.D_INDEX
    Hq, lat, rope = wl.Hq, synth.D_LATENT, synth.D_ROPE
    nope, v = synth.D_QK_HEAD - rope, 128
    got = {
        "query_compression": dim * q_rank + q_rank,                 # wq_a + q_norm
        "key_value_compression": dim * lat + lat,                   # latent part of wkv_a + kv_norm
        "query_heads": q_rank * Hq * (nope + rope),                 # wq_b
        "key_heads": Hq * nope * lat + dim * rope,                  # W_UK + rotary-key part of wkv_a
        "value_heads": Hq * v * lat,                                # W_UV
        "lightning_indexer": q_rank * H_I * d + dim * d + 2 * d + dim * H_I,
        "sparse_attention": Hq * v * dim,                           # wo
    }
    got["total"] = sum(got.values())
    for k, val in got.items():
        assert val == ref[k], k
