"""Pins of the oracle's sparse latent attention in absorbed (MQA) form
(page "Similarities", MLA decode excerpt; page "Sparse latent attention",
softmax and O = AV; page "RoPE coefficients", MLA prefill excerpt for the
non-absorbed form).
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def rand(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def test_dense_recovery_matches_torch_sdpa():
    # Every position selected: the sparse attention is the plain softmax
    # attention over the whole prefix, which PyTorch computes independently.
    B, S, Hq, L, Dl, Dr = 2, 2, 8, 300, 512, 64
    q, lat, pe = rand(1, B, S, Hq, Dl + Dr), rand(2, B, L, Dl), rand(3, B, L, Dr)
    scale = 192 ** -0.5
    idx = np.broadcast_to(np.arange(L, dtype=np.int32), (B, S, L)).copy()
    out, lse = oracle.sparse_mla(q, lat, pe, idx, scale)
    kt = torch.from_numpy(np.concatenate([lat, pe], -1))[:, None]           # [B,1,L,576]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)                            # [B,Hq,S,576]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.expand(B, Hq, L, Dl + Dr), torch.from_numpy(lat)[:, None].expand(B, Hq, L, Dl),
        scale=scale).permute(0, 2, 1, 3).numpy()
    assert np.allclose(out, ref, rtol=1e-10, atol=1e-12)
    logits = torch.einsum("bhsd,bld->bhsl", qt, kt[:, 0]) * scale
    ref_lse = torch.logsumexp(logits, -1).permute(0, 2, 1).numpy()
    assert np.allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_absorbed_equals_non_absorbed():
    # q_abs = q_nope W_UK (per head), out_mha = (sum p c) W_UV^T.
    B, S, Hq, L, Dn, Dv, Dl, Dr, K = 1, 2, 4, 200, 128, 128, 512, 64, 64
    q_nope, q_pe = rand(4, B, S, Hq, Dn), rand(5, B, S, Hq, Dr)
    W = rand(6, Hq, Dn + Dv, Dl) * Dl ** -0.5
    lat, pe = rand(7, B, L, Dl), rand(8, B, L, Dr)
    idx = synth.random_selection(9, B * S, K, [200, 150], fill=0.3).reshape(B, S, K)
    scale = 192 ** -0.5
    mha = oracle.mla_mha(q_nope, q_pe, W, lat, pe, idx, scale)
    q_abs = oracle.absorb_q(q_nope, W)
    x, _ = oracle.sparse_mla(np.concatenate([q_abs, q_pe], -1), lat, pe, idx, scale)
    absorbed = oracle.absorb_o(x, W)
    assert np.allclose(absorbed, mha, rtol=1e-10, atol=1e-12)
    # the same through einsum, so that a wrong slice or transpose inside the
    # absorption helpers fails here even where the two forms would agree
    assert np.allclose(q_abs, np.einsum("bshd,hdc->bshc", q_nope, W[:, :Dn]), rtol=1e-12)
    assert np.allclose(absorbed, np.einsum("bshc,hdc->bshd", x, W[:, Dn:]), rtol=1e-12)
    # the multi-head form on the up-projected keys and values is the same
    # attention (selection distinct and inside the causal range)
    kv = oracle.kv_up(lat, W)
    pos = np.array([[199, 149]], np.int32)
    mha2 = oracle.sparse_mha(np.concatenate([q_nope, q_pe], -1), kv, pe, idx, scale, pos=pos)
    assert np.allclose(mha2, mha, rtol=1e-10, atol=1e-12)


def test_kv_up_is_the_linear_layer_split_per_head():
    # The pages apply wkv_b as a linear layer and view its output as
    # [.., heads, k_nope + v]; PyTorch's linear computes the same product.
    B, L, Hq, Dl = 2, 7, 3, 512
    lat, W = rand(40, B, L, Dl), rand(41, Hq, 256, Dl)
    ref = torch.nn.functional.linear(torch.from_numpy(lat),
                                     torch.from_numpy(W.reshape(Hq * 256, Dl)))
    kv = oracle.kv_up(lat, W)
    assert np.allclose(kv, ref.view(B, L, Hq, 256).numpy(), rtol=1e-12, atol=1e-12)
    # head 1, position 4: k_nope is W_UK[1] c, v is W_UV[1] c
    assert np.allclose(kv[1, 4, 1, :128], W[1, :128] @ lat[1, 4], rtol=1e-12)
    assert np.allclose(kv[1, 4, 1, 128:], W[1, 128:] @ lat[1, 4], rtol=1e-12)


def test_mha_equals_dense_masked_softmax():
    # The MLA prefill excerpt's own formulation: scores over every position,
    # an index mask scattered from the top-k list (repeats collapse), plus the
    # causal mask, softmax, product with v. Written with PyTorch in float64.
    B, S, Hq, L, K = 2, 5, 3, 40, 12
    q, kv, pe = rand(42, B, S, Hq, 192), rand(43, B, L, Hq, 256), rand(44, B, L, 64)
    g = np.random.Generator(np.random.PCG64(45))
    idx = g.integers(-1, L, size=(B, S, K)).astype(np.int32)
    idx[0, 1, :4] = 7                                 # a repeated position
    idx[0, 0, 0], idx[1, 2, 0] = 3, 5                 # positions equal to pos (kept)
    idx[0, 0, 1], idx[1, 2, 1] = 4, 6                 # one past pos (masked)
    pos = np.array([[3, 10, 39, 25, 0], [39, 17, 5, 30, 12]], np.int32)
    scale = 0.09
    out = oracle.sparse_mha(q, kv, pe, idx, scale, pos=pos)
    qt, kvt, pet = map(torch.from_numpy, (q, kv, pe))
    k = torch.cat([kvt[..., :128], pet[:, :, None].expand(B, L, Hq, 64)], -1)
    scores = torch.einsum("bshd,bthd->bsht", qt, k) * scale
    idx_t = torch.from_numpy(idx.astype(np.int64))
    index_mask = torch.full((B, S, L + 1), float("-inf"), dtype=torch.float64)
    index_mask.scatter_(-1, torch.where(idx_t < 0, L, idx_t), 0.0)   # -1 -> spare column
    index_mask = index_mask[..., :L]
    causal = torch.where(torch.arange(L)[None, None] <= torch.from_numpy(pos)[..., None], 0.0,
                         float("-inf")).to(torch.float64)
    scores = scores + (index_mask + causal)[:, :, None]
    ref = torch.einsum("bsht,bthd->bshd", scores.softmax(-1), kvt[..., 128:]).numpy()
    live = np.isfinite(scores.numpy()).any(-1)                     # [B,S,Hq]
    assert np.allclose(out[live], ref[live], rtol=1e-12, atol=1e-12)
    assert np.all(out[~live] == 0)
    assert (~live).any() and live.any()
    # without positions the causal mask is off
    out_nc = oracle.sparse_mha(q, kv, pe, idx, scale)
    assert not np.allclose(out_nc, out)


def test_equal_logits_give_mean_and_single_row_gives_row():
    B, S, Hq, L = 1, 1, 3, 50
    lat, pe = rand(10, B, L, 512), rand(11, B, L, 64)
    q = np.zeros((B, S, Hq, 576))
    sel = np.array([3, 17, 4, 40, 22], np.int32)
    idx = np.full((B, S, 16), -1, np.int32)
    idx[0, 0, [0, 5, 6, 9, 15]] = sel
    out, lse = oracle.sparse_mla(q, lat, pe, idx, 0.1)
    assert np.allclose(out[0, 0], lat[0, sel].mean(0)[None], rtol=1e-13, atol=1e-13)
    assert np.allclose(lse, np.log(5.0))
    one = np.full((B, S, 8), -1, np.int32)
    one[0, 0, 3] = 29
    out1, lse1 = oracle.sparse_mla(rand(12, B, S, Hq, 576), lat, pe, one, 0.3)
    assert np.allclose(out1[0, 0], lat[0, 29][None], rtol=1e-14, atol=1e-14)


def test_index_order_and_padding_do_not_matter():
    B, S, Hq, L, K = 2, 1, 16, 400, 128
    q, lat, pe = rand(13, B, S, Hq, 576), rand(14, B, L, 512), rand(15, B, L, 64)
    idx = synth.random_selection(16, B * S, K, [400, 300], fill=0.25).reshape(B, S, K)
    out, lse = oracle.sparse_mla(q, lat, pe, idx, 192 ** -0.5)
    g = np.random.Generator(np.random.PCG64(17))
    idx2 = idx[..., g.permutation(K)]
    out2, lse2 = oracle.sparse_mla(q, lat, pe, idx2, 192 ** -0.5)
    assert np.allclose(out2, out, rtol=1e-12, atol=1e-13) and np.allclose(lse2, lse)
    compact = np.full((B, S, K + 7), -1, np.int32)
    for b in range(B):
        v = idx[b, 0][idx[b, 0] >= 0]
        compact[b, 0, :v.size] = v
    out3, _ = oracle.sparse_mla(q, lat, pe, compact, 192 ** -0.5)
    assert np.allclose(out3, out, rtol=1e-12, atol=1e-13)


def test_empty_selection_is_zero_with_minus_inf_lse():
    q, lat, pe = rand(18, 1, 1, 2, 576), rand(19, 1, 10, 512), rand(20, 1, 10, 64)
    out, lse = oracle.sparse_mla(q, lat, pe, np.full((1, 1, 4), -1, np.int32), 0.1)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_batches_use_their_own_cache():
    B, S, Hq, L = 3, 2, 2, 20
    q, lat, pe = rand(21, B, S, Hq, 576), rand(22, B, L, 512), rand(23, B, L, 64)
    idx = synth.random_selection(24, B * S, 8, 20).reshape(B, S, 8)
    out, _ = oracle.sparse_mla(q, lat, pe, idx, 0.07)
    for b in range(B):
        o1, _ = oracle.sparse_mla(q[b:b + 1], lat[b:b + 1], pe[b:b + 1], idx[b:b + 1], 0.07)
        assert np.array_equal(o1[0], out[b])
