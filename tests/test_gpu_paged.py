"""Paged caches (block table): every call that reads or writes a
per-position cache gives, on a page pool addressed through a block table,
bit-for-bit the result it gives on the equivalent dense cache (the same
arithmetic on the same values, only the addresses differ), and both the
paged and the dense results are checked against the oracle directly. Positions on a page whose table entry
is outside the pool are "not present": the indexer scores them -inf, the
attention skips them, nothing is written there. (Paged variants are named
on the aipricedb page, indexer logit kernels paragraph; the layout is the
plain block-table reading.)"""
import numpy as np
import pytest

import oracle
import sparse_attention_index_amd as dsa
import synth
from gpu_util import (INDEXER_RTOL, MLA_ATOL, check_scores, dev, dev_bf16, host, host_bf16_as_f32,
                      say, score_errors)
from test_gpu_mla import oracle_on_selection

pytestmark = pytest.mark.gpu


def make_table(seed, B, Lmax, page, extra_pages=3, hole=None):
    """A random page permutation for B rows of Lmax positions; `hole` =
    (b, logical page) is left unmapped (-1)."""
    g = synth.rng(seed)
    max_pages = (Lmax + page - 1) // page
    num_pages = B * max_pages + extra_pages
    perm = g.permutation(num_pages)[:B * max_pages].astype(np.int32).reshape(B, max_pages)
    if hole is not None:
        perm[hole] = -1
    return perm, num_pages


def scatter_pool(dense, table, page, num_pages):
    """Dense [B, Lmax, ...] cache -> pool [num_pages, page, ...] per the table."""
    B, Lmax = dense.shape[:2]
    pool = np.zeros((num_pages, page) + dense.shape[2:], dense.dtype)
    for b in range(B):
        for lp in range(table.shape[1]):
            pg = table[b, lp]
            if pg < 0:
                continue
            lo, hi = lp * page, min(Lmax, (lp + 1) * page)
            pool[pg, :hi - lo] = dense[b, lo:hi]
    return pool


@pytest.mark.parametrize("S,page,Lmax", [(1, 64, 1000), (1, 16, 1000), (3, 128, 1000),
                                         (20, 32, 1000), (1, 64, 70000)])
def test_indexer_paged_matches_dense(S, page, Lmax):
    import torch
    B, H = 2, 64
    say(f"indexer paged S={S} page={page} Lmax={Lmax}")
    g = synth.rng(400 + S + page)
    q_raw = synth.bf16_bits_to_f32(synth.to_bf16_bits(g.standard_normal((B, S, H, 128), dtype=np.float32)))
    k_all = synth.bf16_bits_to_f32(synth.to_bf16_bits(g.standard_normal((B, Lmax, 128), dtype=np.float32)))
    w = (g.standard_normal((B, S, H), dtype=np.float32) * np.float32(64 ** -0.5 * 128 ** -0.5))
    pos = np.array([[Lmax - 1 - 7 * s for s in range(S)], [480 + s for s in range(S)]], np.int32)
    cos, sin = oracle.rope_table(Lmax)
    dcos, dsin = dev(cos), dev(sin)
    table, num_pages = make_table(401, B, Lmax, page, hole=(1, 3))
    paging = dsa.Paging(dev(table), page, num_pages)
    all_pos = dev(np.broadcast_to(np.arange(Lmax, dtype=np.int32), (B, Lmax)).copy())
    k_call = np.stack([k_all[b, pos[b]] for b in range(B)])
    results = {}
    for mode in ("dense", "paged"):
        if mode == "dense":
            kc = torch.zeros((B, Lmax, 128), dtype=torch.uint8, device="cuda")
            ks = torch.zeros((B, Lmax), dtype=torch.float32, device="cuda")
            pg = None
        else:
            kc = torch.zeros((num_pages, page, 128), dtype=torch.uint8, device="cuda")
            ks = torch.zeros((num_pages, page), dtype=torch.float32, device="cuda")
            pg = paging
        dsa.indexer_append(dev_bf(k_all), all_pos, dcos, dsin, kc, ks, paging=pg)
        sc = torch.full((B, S, pg.lmax if pg else Lmax), float("nan"), dtype=torch.float32,
                        device="cuda")
        dsa.indexer(dev_bf(q_raw), dev(w), dev(pos), dcos, dsin, kc, ks, sc,
                    k_raw=dev_bf(k_call), paging=pg)
        torch.cuda.synchronize()
        results[mode] = (host(kc), host(ks), host(sc)[..., :Lmax])
    dk, dks, dsc = results["dense"]
    pk, pks, psc = results["paged"]
    # the pool holds the dense rows at the mapped positions
    assert np.array_equal(scatter_pool(dk, table, page, num_pages), pk)
    assert np.array_equal(scatter_pool(dks, table, page, num_pages), pks)
    # scores: identical except the unmapped page (b = 1, positions 3p..4p-1)
    hole = np.zeros((B, Lmax), bool)
    hole[1, 3 * page:4 * page] = True
    for b in range(B):
        for s in range(S):
            n = pos[b, s] + 1
            d, p = dsc[b, s, :n], psc[b, s, :n]
            h = hole[b, :n]
            assert np.array_equal(d[~h], p[~h])
            assert np.all(p[h] == -np.inf)
    # the pool's codes and scales and the paged scores against the oracle
    # directly, and the dense scores too
    k8, ks8, _ = oracle.indexer_prepare(k_all, np.broadcast_to(np.arange(Lmax), (B, Lmax)), cos,
                                        sin, True)
    assert np.array_equal(scatter_pool(k8, table, page, num_pages), pk)
    assert np.array_equal(scatter_pool(ks8, table, page, num_pages), pks)
    q8, qs8, _ = oracle.indexer_prepare(q_raw, pos[..., None], cos, sin, True)
    o = oracle.indexer_scores(oracle.dequantize(q8, qs8), w, oracle.dequantize(k8, ks8), pos + 1)
    check_scores(dsc.reshape(B * S, Lmax), o.reshape(B * S, Lmax), (pos + 1).reshape(-1), "dense")
    worst = 0.0
    for b in range(B):
        for s in range(S):
            n = pos[b, s] + 1
            h = hole[b, :n]
            e = score_errors(psc[b, s, :n], o[b, s, :n])[~h]
            worst = max(worst, float(e.max()))
    assert worst <= INDEXER_RTOL
    say(f"  paged worst normalised score error {worst:.2e}")


def dev_bf(values_f32):
    import torch
    return torch.from_numpy(np.ascontiguousarray(values_f32)).to("cuda").to(torch.bfloat16)


@pytest.mark.parametrize("S,page,K", [(1, 64, 2048), (2, 32, 256), (40, 128, 512)])
def test_mla_paged_matches_dense(S, page, K):
    import torch
    B, Hq, L = 2, 128, 4096
    say(f"mla paged S={S} page={page} K={K}")
    g = synth.rng(410 + S)
    q = synth.to_bf16_bits(g.standard_normal((B, S, Hq, 576), dtype=np.float32))
    lat = synth.to_bf16_bits(g.standard_normal((B, L, 512), dtype=np.float32))
    kpe = synth.to_bf16_bits(g.standard_normal((B, L, 64), dtype=np.float32))
    idx = synth.random_selection(411, B * S, K, np.full(B * S, L), 1.0).reshape(B, S, K)
    table, num_pages = make_table(412, B, L, page, hole=(0, 5))
    scale = 192 ** -0.5
    dq, didx = dev_bf16(q), dev(idx)
    out_d, lse_d = dsa.sparse_mla(dq, dev_bf16(lat), dev_bf16(kpe), didx, scale, return_lse=True)
    pool = scatter_pool(np.concatenate([lat, kpe], axis=2), table, page, num_pages)
    dpool = dev_bf16(pool)
    out_p, lse_p = dsa.sparse_mla(dq, dpool[..., :512], dpool[..., 512:], didx, scale,
                                  return_lse=True, paging=dsa.Paging(dev(table), page, num_pages))
    torch.cuda.synchronize()
    # positions on the unmapped page are skipped: the dense reference drops them too
    idx_drop = np.where((idx >= 0) & (idx // page == 5) & (np.arange(B)[:, None, None] == 0),
                        -1, idx).astype(np.int32)
    out_r, lse_r = dsa.sparse_mla(dq, dev_bf16(lat), dev_bf16(kpe), dev(idx_drop), scale,
                                  return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(out_p.view(torch.int16)), host(out_r.view(torch.int16)))
    assert np.array_equal(host(lse_p), host(lse_r))
    # the paged output against the oracle on the selection without the
    # unmapped page, and the dense run on the full selection
    o, l = oracle_on_selection(q, lat, kpe, idx_drop, scale)
    ep = np.max(np.abs(host_bf16_as_f32(out_p) - o))
    assert ep <= MLA_ATOL
    assert np.allclose(host(lse_p), l, rtol=0, atol=1e-3)
    o, l = oracle_on_selection(q, lat, kpe, idx, scale)
    ed = np.max(np.abs(host_bf16_as_f32(out_d) - o))
    assert ed <= MLA_ATOL
    assert np.allclose(host(lse_d), l, rtol=0, atol=1e-3)
    say(f"  paged max abs err {ep:.3e}, dense {ed:.3e}")


def test_mla_append_paged_matches_dense():
    import torch
    B, S, Hq, L, page = 2, 3, 16, 256, 32
    say("mla_append paged")
    g = synth.rng(420)
    lat_new = synth.to_bf16_bits(g.standard_normal((B, S, 512), dtype=np.float32))
    kpe_new = synth.to_bf16_bits(g.standard_normal((B, S, 64), dtype=np.float32))
    q = synth.to_bf16_bits(g.standard_normal((B, S, Hq, 576), dtype=np.float32))
    pos = np.array([[0, 100, 255], [33, 34, 200]], np.int32)
    cos, sin = oracle.rope_table(L)
    table, num_pages = make_table(421, B, L, page, hole=(1, 1))
    lat_d = dev_bf16(np.zeros((B, L, 512), np.uint16))
    rope_d = dev_bf16(np.zeros((B, L, 64), np.uint16))
    q_d = dev_bf16(q)
    dsa.mla_append(dev_bf16(lat_new), dev_bf16(kpe_new), dev(pos), dev(cos), dev(sin), lat_d,
                   rope_d, q=q_d)
    pool = dev_bf16(np.zeros((num_pages, page, 576), np.uint16))
    q_p = dev_bf16(q)
    dsa.mla_append(dev_bf16(lat_new), dev_bf16(kpe_new), dev(pos), dev(cos), dev(sin),
                   pool[..., :512], pool[..., 512:], q=q_p,
                   paging=dsa.Paging(dev(table), page, num_pages))
    torch.cuda.synchronize()
    bits = lambda t: host(t.view(torch.int16)).view(np.uint16)
    dense = np.concatenate([bits(lat_d), bits(rope_d)], axis=2)
    dense[1, 32:64] = 0                                      # the unmapped page gets nothing
    assert np.array_equal(scatter_pool(dense, table, page, num_pages), bits(pool))
    assert np.array_equal(bits(q_p), bits(q_d))              # q is rotated either way
    # the paged pool and q against the oracle directly: latent rows copied,
    # rotary keys and the queries' rope parts rotated with the interleaved
    # pairing (page "RoPE coefficients"), bf16, nothing else written
    f = synth.bf16_bits_to_f32
    kpe_rot = synth.to_bf16_bits(oracle.rope(f(kpe_new), pos, cos, sin, rope_dim=64,
                                             interleaved=True, out_bf16=True))
    q_rot = q.copy()
    q_rot[..., 512:] = synth.to_bf16_bits(oracle.rope(f(q[..., 512:]), pos[..., None], cos, sin,
                                                      rope_dim=64, interleaved=True,
                                                      out_bf16=True))
    assert np.array_equal(bits(q_p), q_rot)
    expect = np.zeros((num_pages, page, 576), np.uint16)
    for b in range(B):
        for s in range(S):
            pg = table[b, pos[b, s] // page]
            if pg < 0:
                continue
            expect[pg, pos[b, s] % page, :512] = lat_new[b, s]
            expect[pg, pos[b, s] % page, 512:] = kpe_rot[b, s]
    assert np.array_equal(bits(pool), expect)
