"""HIP-graph capture of the library's calls: each graph is replayed several
times, with eager work and synchronisations between the replays and the
outputs cleared before each one, and every replay must reproduce the eager
result bit for bit (every kernel here is deterministic)."""
import numpy as np
import pytest

import sparse_attention_index_amd as dsa
import synth
from gpu_util import say

pytestmark = pytest.mark.gpu


def capture(fn):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_matches(g, outs, ref, scratch=(), reps=3):
    """Replay g `reps` times; before each replay the outputs are set to a
    fill value and the scratch buffers (workspaces) to garbage."""
    import torch
    for i in range(reps):
        for o in outs:
            o.fill_(0 if o.dtype == torch.int32 else 7)
        for w in scratch:
            w.fill_(255)
        junk = torch.randn(1 << 16, device="cuda").sum()      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {i} differs"


def test_decode_step_graph_replays():
    import torch
    B, H, Hq, L, K = 2, 64, 128, 4096, 2048
    say(f"graph decode step B={B} L={L}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    rn = lambda *s: torch.randn(*s, generator=gen, device="cuda")  # noqa: E731
    pos = torch.tensor([[L - 1], [L - 700]], dtype=torch.int32, device="cuda")
    cos, sin = dsa.rope_table(L)
    k_all = rn(B, L, 128).to(torch.bfloat16)
    kc = torch.zeros(B, L, 128, dtype=torch.uint8, device="cuda")
    ks = torch.zeros(B, L, dtype=torch.float32, device="cuda")
    kpos = torch.arange(L, dtype=torch.int32, device="cuda").expand(B, L).contiguous()
    dsa.indexer_append(k_all, kpos, cos, sin, kc, ks)
    q_raw = rn(B, 1, H, 128).to(torch.bfloat16)
    k_new = rn(B, 1, 128).to(torch.bfloat16)
    w = rn(B, 1, H) * (64 ** -0.5) * (128 ** -0.5)
    q = rn(B, 1, Hq, 576).to(torch.bfloat16)
    lat = rn(B, L, 512).to(torch.bfloat16)
    pe = rn(B, L, 64).to(torch.bfloat16)
    scores = torch.empty(B, 1, L, dtype=torch.float32, device="cuda")
    idx = torch.empty(B, 1, K, dtype=torch.int32, device="cuda")
    out = torch.empty(B, 1, Hq, 512, dtype=torch.bfloat16, device="cuda")
    mws = torch.empty(max(1, dsa.sparse_mla_workspace_bytes(
        dsa.mla_args(q, lat, pe, idx, 0.07, out))), dtype=torch.uint8, device="cuda")
    tws = dsa.topk_workspace(scores, pos, K)

    def step():
        dsa.indexer(q_raw, w, pos, cos, sin, kc, ks, scores, k_raw=k_new)
        dsa.topk(scores, pos, K, idx=idx, workspace=tws)
        dsa.sparse_mla(q, lat, pe, idx, 0.07, out=out, workspace=mws)

    scores.fill_(7)                            # entries past a row's position are not written
    step()
    torch.cuda.synchronize()
    ref = [scores.clone(), idx.clone(), out.clone()]
    g = capture(step)
    replay_matches(g, [scores, idx, out], ref, scratch=[mws, tws])


def test_long_row_topk_graph_replays():
    import torch
    L, K = 131072, 2048
    say("graph top-k tournament")
    sc = torch.from_numpy(synth.topk_scores(21, 2, L, "ties")).cuda().view(2, 1, L)
    pos = torch.tensor([[L - 1], [70000]], dtype=torch.int32, device="cuda")
    idx = torch.empty(2, 1, K, dtype=torch.int32, device="cuda")
    ws = dsa.topk_workspace(sc, pos, K)
    dsa.topk(sc, pos, K, idx=idx, workspace=ws)
    torch.cuda.synchronize()
    ref = [idx.clone()]
    g = capture(lambda: dsa.topk(sc, pos, K, idx=idx, workspace=ws))
    replay_matches(g, [idx], ref, scratch=[ws])


def test_multi_head_prefill_graph_replays():
    import torch
    B, S, Hq, L, K = 1, 300, 16, 1000, 512
    say("graph multi-head prefill and projections")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(31)
    rn = lambda *s: torch.randn(*s, generator=gen, device="cuda")  # noqa: E731
    W = (rn(Hq, 256, 512) * 512 ** -0.5).to(torch.bfloat16)
    lat = rn(B, L, 512).to(torch.bfloat16)
    pe = rn(B, L, 64).to(torch.bfloat16)
    qn = rn(B, S, Hq, 128).to(torch.bfloat16)
    q192 = rn(B, S, Hq, 192).to(torch.bfloat16)
    x = rn(B, S, Hq, 512).to(torch.bfloat16)
    posn = np.broadcast_to(np.arange(L - S, L, dtype=np.int32), (B, S)).copy()
    idxn = synth.random_selection(32, B * S, K, (posn + 1).reshape(-1), 0.6).reshape(B, S, K)
    pos = torch.from_numpy(posn).cuda()
    idx = torch.from_numpy(idxn).cuda()
    kv = torch.empty(B, L, Hq, 256, dtype=torch.bfloat16, device="cuda")
    o = torch.empty(B, S, Hq, 128, dtype=torch.bfloat16, device="cuda")
    qa = torch.empty(B, S, Hq, 512, dtype=torch.bfloat16, device="cuda")
    oa = torch.empty(B, S, Hq, 128, dtype=torch.bfloat16, device="cuda")
    hws = torch.empty(dsa.sparse_mha_workspace_bytes(dsa.mha_args(q192, kv, pe, idx, 0.07, o, pos)),
                      dtype=torch.uint8, device="cuda")

    def calls():
        dsa.mla_kv_up(lat, W, out=kv)
        dsa.sparse_mha(q192, kv, pe, idx, 0.07, pos=pos, out=o, workspace=hws)
        dsa.mla_absorb_q(qn, W, out=qa)
        dsa.mla_absorb_o(x, W, out=oa)

    calls()
    torch.cuda.synchronize()
    ref = [kv.clone(), o.clone(), qa.clone(), oa.clone()]
    g = capture(calls)
    # the workspace is filled with garbage before each replay: its masks,
    # lists and zero block are rebuilt by every call
    replay_matches(g, [kv, o, qa, oa], ref, scratch=[hws])
