"""GPU parity of the multi-head (non-absorbed) prefill form and of the MLA
projections against the oracle.

- dsa_mla_kv_up / dsa_mla_absorb_q / dsa_mla_absorb_o: bf16 inputs, float32
  accumulation, one bf16 rounding of the result. Bound per element:
  |g - o| <= 2^-8 |o| + 2^-14 sum_k |a_k||b_k| (the rounding, 2^-9 of the
  float32 value, doubled; plus float32 accumulation over K <= 512 terms,
  at most K 2^-24 = 2^-15 of sum |a||b|, doubled).
- dsa_sparse_mha: max-abs <= 2e-2 on the bf16 output, the bar of the
  absorbed form (same bf16 inputs and selection on both sides).
"""
import numpy as np
import pytest

import oracle
import sparse_attention_index_amd as dsa
import synth
from gpu_util import MLA_ATOL, dev, dev_bf16, host_bf16_as_f32, say

pytestmark = pytest.mark.gpu

SCALE = 192 ** -0.5


def bf(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def check_proj(g, o, bound, label):
    err = np.abs(g - o)
    lim = 2.0 ** -8 * np.abs(o) + 2.0 ** -14 * bound
    worst = float((err / lim).max()) if err.size else 0.0
    say(f"  {label}: max abs err {err.max():.3e}, worst err/bound {worst:.3f}")
    assert np.all(err <= lim), label


def sample_rows(n, k, seed):
    """k distinct rows of n: the first and last, tile edges, random others."""
    g = synth.rng(seed)
    fixed = [r for r in (0, 1, 127, 128, n - 129, n - 128, n - 2, n - 1) if 0 <= r < n]
    rest = g.choice(n, size=min(n, k), replace=False).tolist()
    return np.array(sorted(set(fixed + rest))[:max(k, len(fixed))], np.int64)


# ---------------------------------------------------------------- projections --

def make_w(g, Hq):
    # W ~ N(0, 1/512): up-projected features of N(0,1) latents are ~N(0,1)
    return synth.to_bf16_bits(g.standard_normal((Hq, 256, 512), dtype=np.float32) / np.sqrt(512))


PROJ_CASES = [
    # name, B, rows, Hq
    ("one-row", 1, 1, 1),
    ("ragged", 2, 300, 3),
    ("heads20", 1, 129, 20),
    ("decode-batch", 4, 1, 128),
]


@pytest.mark.parametrize("name,B,rows,Hq", PROJ_CASES, ids=[c[0] for c in PROJ_CASES])
def test_kv_up_parity(name, B, rows, Hq):
    say(f"kv_up {name}: B={B} rows={rows} Hq={Hq}")
    g = synth.rng(700 + rows + Hq)
    W = make_w(g, Hq)
    lat = synth.to_bf16_bits(g.standard_normal((B, rows, 512), dtype=np.float32))
    kv = host_bf16_as_f32(dsa.mla_kv_up(dev_bf16(lat), dev_bf16(W)))
    o = oracle.kv_up(bf(lat), bf(W))
    bound = oracle.kv_up(np.abs(bf(lat)), np.abs(bf(W)))
    check_proj(kv, o, bound, "kv_up")


@pytest.mark.parametrize("name,B,rows,Hq", PROJ_CASES, ids=[c[0] for c in PROJ_CASES])
def test_absorb_parity(name, B, rows, Hq):
    import torch
    say(f"absorb {name}: B={B} rows={rows} Hq={Hq}")
    g = synth.rng(800 + rows + Hq)
    W = make_w(g, Hq)
    qn = synth.to_bf16_bits(g.standard_normal((B, rows, Hq, 128), dtype=np.float32))
    x = synth.to_bf16_bits(g.standard_normal((B, rows, Hq, 512), dtype=np.float32))
    dW = dev_bf16(W)
    # the query absorption writes into the latent part of a 576-wide query
    q576 = torch.full((B, rows, Hq, 576), 3.0, dtype=torch.bfloat16, device="cuda")
    dsa.mla_absorb_q(dev_bf16(qn), dW, out=q576[..., :512])
    qa = host_bf16_as_f32(q576)
    assert np.all(qa[..., 512:] == 3.0)
    check_proj(qa[..., :512], oracle.absorb_q(bf(qn), bf(W)),
               oracle.absorb_q(np.abs(bf(qn)), np.abs(bf(W))), "absorb_q")
    o = host_bf16_as_f32(dsa.mla_absorb_o(dev_bf16(x), dW))
    check_proj(o, oracle.absorb_o(bf(x), bf(W)), oracle.absorb_o(np.abs(bf(x)), np.abs(bf(W))),
               "absorb_o")


def test_projections_prefill4k_full_size_sampled_rows():
    """All 4096 rows of the 4K prefill through each projection with 128 heads;
    sampled rows against the oracle (rows are independent)."""
    wl = synth.workload("prefill4k")
    say("projections prefill4k full size")
    g = synth.rng(901)
    W = make_w(g, wl.Hq)
    lat = synth.to_bf16_bits(g.standard_normal((1, wl.Lmax, 512), dtype=np.float32))
    qn = synth.to_bf16_bits(g.standard_normal((1, wl.S, wl.Hq, 128), dtype=np.float32))
    x = synth.to_bf16_bits(g.standard_normal((1, wl.S, wl.Hq, 512), dtype=np.float32))
    dW = dev_bf16(W)
    kv = dsa.mla_kv_up(dev_bf16(lat), dW)
    qa = dsa.mla_absorb_q(dev_bf16(qn), dW)
    oo = dsa.mla_absorb_o(dev_bf16(x), dW)
    rows = sample_rows(wl.S, 24, 902)
    check_proj(host_bf16_as_f32(kv[:, rows]), oracle.kv_up(bf(lat[:, rows]), bf(W)),
               oracle.kv_up(np.abs(bf(lat[:, rows])), np.abs(bf(W))), "kv_up")
    check_proj(host_bf16_as_f32(qa[:, rows]), oracle.absorb_q(bf(qn[:, rows]), bf(W)),
               oracle.absorb_q(np.abs(bf(qn[:, rows])), np.abs(bf(W))), "absorb_q")
    check_proj(host_bf16_as_f32(oo[:, rows]), oracle.absorb_o(bf(x[:, rows]), bf(W)),
               oracle.absorb_o(np.abs(bf(x[:, rows])), np.abs(bf(W))), "absorb_o")


# ------------------------------------------------------------- multi-head form --

def oracle_rows(q, kv, pe, idx, pos, rows):
    """Oracle on a subset of query rows of one batch row, the keys compacted to
    the positions those rows select (ranks keep the causal comparison)."""
    B = q.shape[0]
    Lmax = kv.shape[1]
    outs = []
    for b in range(B):
        sel = idx[b, rows]
        ok = (sel >= 0) & (sel < Lmax)
        union = np.unique(sel[ok])
        remap = np.full(Lmax, -1, np.int64)
        remap[union] = np.arange(union.size)
        ib = np.where(ok, remap[np.where(ok, sel, 0)], -1).astype(np.int32)
        pb = None
        if pos is not None:
            pb = (np.searchsorted(union, pos[b, rows], side="right") - 1).astype(np.int32)[None]
        kvu = bf(kv[b, union])[None] if union.size else np.zeros((1, 1) + kv.shape[2:])
        peu = bf(pe[b, union])[None] if union.size else np.zeros((1, 1, 64))
        outs.append(oracle.sparse_mha(bf(q[b, rows])[None], kvu, peu, ib[None], SCALE, pos=pb)[0])
    return np.stack(outs)


def mha_inputs(B, S, Hq, L, K, seed, fill=1.0, causal=True):
    g = synth.rng(seed)
    q = synth.to_bf16_bits(g.standard_normal((B, S, Hq, 192), dtype=np.float32))
    kv = synth.to_bf16_bits(g.standard_normal((B, L, Hq, 256), dtype=np.float32))
    pe = synth.to_bf16_bits(g.standard_normal((B, L, 64), dtype=np.float32))
    # prefill: the S rows are the last S positions of the L cached ones
    pos = np.broadcast_to(np.arange(L - S, L, dtype=np.int32), (B, S)).copy()
    nv = (pos + 1).reshape(-1) if causal else np.full(B * S, L)
    idx = synth.random_selection(seed + 1, B * S, K, nv, fill).reshape(B, S, K)
    return q, kv, pe, idx, (pos if causal else None)


def run_mha(q, kv, pe, idx, pos):
    import torch
    out = dsa.sparse_mha(dev_bf16(q), dev_bf16(kv), dev_bf16(pe), dev(idx), SCALE,
                         pos=None if pos is None else dev(pos))
    torch.cuda.synchronize()
    return host_bf16_as_f32(out)


MHA_CASES = [
    # name, B, S, Hq, L, K, fill, causal
    ("tiny", 1, 5, 2, 64, 32, 1.0, True),
    ("ragged-heads20", 2, 300, 20, 300, 128, 1.0, True),
    ("dense-causal", 1, 200, 8, 200, 256, 1.0, True),
    ("sparse-half", 1, 140, 16, 700, 512, 0.5, True),
    ("long", 1, 256, 128, 3000, 2048, 1.0, True),
    ("no-positions", 2, 70, 8, 900, 300, 1.0, False),
]


@pytest.mark.parametrize("name,B,S,Hq,L,K,fill,causal", MHA_CASES, ids=[c[0] for c in MHA_CASES])
def test_mha_parity(name, B, S, Hq, L, K, fill, causal):
    say(f"mha case {name}: B={B} S={S} Hq={Hq} L={L} K={K}")
    q, kv, pe, idx, pos = mha_inputs(B, S, Hq, L, K, 1000 + S + Hq, fill, causal)
    g = run_mha(q, kv, pe, idx, pos)
    o = oracle_rows(q, kv, pe, idx, pos, np.arange(S))
    err = np.abs(g - o).max()
    say(f"  max abs err {err:.3e}")
    assert err <= MLA_ATOL


def test_mha_masks_repeats_and_empty_rows():
    """Entries past the row's position are masked, repeats count once, -1 and
    out-of-range entries are skipped, rows with nothing (or pos < 0) give 0."""
    B, S, Hq, L, K = 1, 130, 8, 500, 64
    q, kv, pe, idx, pos = mha_inputs(B, S, Hq, L, K, 1111, 0.5)
    idx[0, 0] = -1                                 # empty row
    idx[0, 1, :6] = [5, 5, 5, 9, 1000, -7]         # repeats and out-of-range entries
    idx[0, 2, :3] = [pos[0, 2], pos[0, 2] + 1, L - 1]   # one kept, two past the position
    pos[0, 3] = -1                                 # a row with no position: empty
    idx[0, 129, :] = -1
    idx[0, 129, 7] = 0                             # a single selected position
    g = run_mha(q, kv, pe, idx, pos)
    o = oracle_rows(q, kv, pe, idx, pos, np.arange(S))
    assert np.all(g[0, 0] == 0) and np.all(g[0, 3] == 0)
    assert np.abs(g - o).max() <= MLA_ATOL
    assert np.allclose(g[0, 129], bf(kv[0, 0, :, 128:]), atol=1e-2)


def test_mha_prefill4k_full_size_sampled_rows():
    """The 4K prefill (4096 rows, 128 heads, top-2048 of the causal prefix) in
    the launch configuration the benchmark uses; sampled rows checked."""
    wl = synth.workload("prefill4k")
    say("mha prefill4k full size")
    q, kv, pe, idx, pos = mha_inputs(1, wl.S, wl.Hq, wl.Lmax, wl.K, 1234)
    g = run_mha(q, kv, pe, idx, pos)
    rows = sample_rows(wl.S, 40, 1235)
    o = oracle_rows(q, kv, pe, idx, pos, rows)
    err = np.abs(g[:, rows] - o).max()
    say(f"  max abs err {err:.3e} over {rows.size} rows")
    assert err <= MLA_ATOL
    assert np.isfinite(g).all()


def test_mha_is_deterministic():
    q, kv, pe, idx, pos = mha_inputs(1, 300, 16, 2000, 1024, 77, 0.7)
    assert np.array_equal(run_mha(q, kv, pe, idx, pos), run_mha(q, kv, pe, idx, pos))


def test_prefill_both_forms_against_the_oracle():
    """From the same latent cache and wkv_b: the multi-head path (kv_up, then
    sparse_mha) and the absorbed path (absorb_q, sparse_mla, absorb_o), both
    on the GPU, against the oracle's non-absorbed definition."""
    import torch
    B, S, Hq, L, K = 1, 130, 8, 600, 256
    g = synth.rng(1300)
    W = make_w(g, Hq)
    lat = synth.to_bf16_bits(g.standard_normal((B, L, 512), dtype=np.float32))
    pe = synth.to_bf16_bits(g.standard_normal((B, L, 64), dtype=np.float32))
    qn = synth.to_bf16_bits(g.standard_normal((B, S, Hq, 128), dtype=np.float32))
    qp = synth.to_bf16_bits(g.standard_normal((B, S, Hq, 64), dtype=np.float32))
    pos = np.broadcast_to(np.arange(L - S, L, dtype=np.int32), (B, S)).copy()
    idx = synth.random_selection(1301, B * S, K, (pos + 1).reshape(-1), 0.6).reshape(B, S, K)
    dW, dlat, dpe = dev_bf16(W), dev_bf16(lat), dev_bf16(pe)
    # multi-head form
    kv = dsa.mla_kv_up(dlat, dW)
    q192 = dev_bf16(np.concatenate([qn, qp], -1))
    mha = dsa.sparse_mha(q192, kv, dpe, dev(idx), SCALE, pos=dev(pos))
    # absorbed form
    q576 = torch.empty((B, S, Hq, 576), dtype=torch.bfloat16, device="cuda")
    q576[..., 512:] = dev_bf16(qp)
    dsa.mla_absorb_q(dev_bf16(qn), dW, out=q576[..., :512])
    x = dsa.sparse_mla(q576, dlat, dpe, dev(idx), SCALE)
    absorbed = dsa.mla_absorb_o(x, dW)
    torch.cuda.synchronize()
    ref = oracle.mla_mha(bf(qn), bf(qp), bf(W), bf(lat), bf(pe), idx, SCALE)
    e1 = np.abs(host_bf16_as_f32(mha) - ref).max()
    e2 = np.abs(host_bf16_as_f32(absorbed) - ref).max()
    say(f"  multi-head form err {e1:.3e}, absorbed form err {e2:.3e}")
    assert e1 <= MLA_ATOL and e2 <= MLA_ATOL


def test_kv_up_and_mha_read_a_fused_cache():
    """Latent and rotary rows read from one fused 576-wide cache (row stride
    576 elements) by the up-projection and the multi-head attention."""
    import torch
    B, S, Hq, L, K = 2, 70, 8, 300, 128
    g = synth.rng(1400)
    W = make_w(g, Hq)
    cache = synth.to_bf16_bits(g.standard_normal((B, L, 576), dtype=np.float32))
    dcache = dev_bf16(cache)
    kv = dsa.mla_kv_up(dcache[..., :512], dev_bf16(W))
    torch.cuda.synchronize()
    check_proj(host_bf16_as_f32(kv), oracle.kv_up(bf(cache[..., :512]), bf(W)),
               oracle.kv_up(np.abs(bf(cache[..., :512])), np.abs(bf(W))), "kv_up fused")
    q = synth.to_bf16_bits(g.standard_normal((B, S, Hq, 192), dtype=np.float32))
    pos = np.broadcast_to(np.arange(L - S, L, dtype=np.int32), (B, S)).copy()
    idx = synth.random_selection(1401, B * S, K, (pos + 1).reshape(-1), 0.5).reshape(B, S, K)
    out = dsa.sparse_mha(dev_bf16(q), kv, dcache[..., 512:], dev(idx), SCALE, pos=dev(pos))
    torch.cuda.synchronize()
    # the oracle attends over its own up-projection, rounded to bf16 as the
    # cached keys and values are
    okv = synth.to_bf16_bits(oracle.kv_up(bf(cache[..., :512]), bf(W)).astype(np.float32))
    o = oracle_rows(q, okv, cache[..., 512:], idx, pos, np.arange(S))
    assert np.abs(host_bf16_as_f32(out) - o).max() <= MLA_ATOL
