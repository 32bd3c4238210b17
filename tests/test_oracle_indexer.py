"""Pins of the oracle's lightning-indexer score
I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . k[s])  (aipricedb page, indexer
formula; page "Sparse latent attention", equation S^I).

Each test fixes a structure whose answer has a closed form that a plausible
mistake (dropped ReLU, transposed q, wrong head/weight pairing, off-by-one in
the causal bound) would break.
"""
import numpy as np
import pytest

import oracle
import synth


def rand(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def test_one_hot_weight_selects_one_head():
    B, S, H, D, L = 1, 2, 6, 128, 40
    q = rand(1, B, S, H, D)
    k = rand(2, B, L, D)
    nv = np.array([[40, 17]], np.int32)
    for h in range(H):
        w = np.zeros((B, S, H))
        w[..., h] = 1.0
        I = oracle.indexer_scores(q, w, k, nv)
        for t in range(S):
            n = nv[0, t]
            want = np.maximum(k[0, :n] @ q[0, t, h], 0.0)
            assert np.allclose(I[0, t, :n], want, rtol=1e-13, atol=1e-13)
            assert np.all(np.isnan(I[0, t, n:]))      # causal: beyond n_valid untouched


def test_all_positive_dots_reduce_to_matrix_vector_product():
    # q, k >= 0 elementwise -> every dot is >= 0 and the ReLU is inactive,
    # so I[t, :] = K (sum_h w_h q_h)
    B, S, H, D, L = 2, 3, 8, 128, 50
    q = np.abs(rand(3, B, S, H, D))
    k = np.abs(rand(4, B, L, D))
    w = rand(5, B, S, H)
    nv = np.full((B, S), L, np.int32)
    I = oracle.indexer_scores(q, w, k, nv)
    for b in range(B):
        for t in range(S):
            v = np.einsum("h,hd->d", w[b, t], q[b, t])
            assert np.allclose(I[b, t], k[b] @ v, rtol=1e-12, atol=1e-12)


def test_all_negative_dots_give_zero():
    B, S, H, D, L = 1, 1, 16, 128, 30
    q = -np.abs(rand(6, B, S, H, D))
    k = np.abs(rand(7, B, L, D))
    w = rand(8, B, S, H)
    I = oracle.indexer_scores(q, w, k, np.array([[L]], np.int32))
    assert np.all(I == 0.0)


def test_head_and_feature_permutations_leave_scores_unchanged():
    B, S, H, D, L = 1, 2, 12, 128, 64
    q, k, w = rand(9, B, S, H, D), rand(10, B, L, D), rand(11, B, S, H)
    nv = np.array([[64, 33]], np.int32)
    base = oracle.indexer_scores(q, w, k, nv)
    g = np.random.Generator(np.random.PCG64(12))
    ph, pd = g.permutation(H), g.permutation(D)
    I2 = oracle.indexer_scores(q[:, :, ph][..., pd], w[:, :, ph], k[..., pd], nv)
    assert np.allclose(I2, base, rtol=1e-12, atol=1e-12, equal_nan=True)


def test_relu_is_per_head_not_on_the_sum():
    # one key, two heads with dots +2 and -3, weights 1 and 1:
    # per-head ReLU gives 2; a ReLU after the head sum would give 0.
    q = np.zeros((1, 1, 2, 128))
    k = np.zeros((1, 1, 128))
    k[0, 0, 0] = 1.0
    q[0, 0, 0, 0] = 2.0
    q[0, 0, 1, 0] = -3.0
    w = np.ones((1, 1, 2))
    assert oracle.indexer_scores(q, w, k, np.array([[1]], np.int32))[0, 0, 0] == 2.0


def test_scale_factoring_on_quantised_values():
    # The pages fold q's block scale into the weights and leave k's scale to
    # the kernel; because scales are positive both factor out of the ReLU:
    # I = ks[s] * sum_h (w_h qs_h) ReLU(q8_h . k8_s) on the raw codes.
    wl = synth.workload("tiny")
    g = np.random.Generator(np.random.PCG64(13))
    x = g.standard_normal((1, 1, 4, 128)).astype(np.float32)
    kx = g.standard_normal((1, 96, 128)).astype(np.float32)
    w = g.standard_normal((1, 1, 4))
    q8, qs = oracle.quantize(x)
    k8, ks = oracle.quantize(kx)
    I = oracle.indexer_scores(oracle.dequantize(q8, qs), w, oracle.dequantize(k8, ks),
                              np.array([[96]], np.int32))
    qc = oracle.e4m3_decode(q8)[0, 0]          # [4,128] code values
    kc = oracle.e4m3_decode(k8)[0]             # [96,128]
    folded = ks[0].astype(np.float64) * (np.maximum(kc @ qc.T, 0) @ (w[0, 0] * qs[0, 0]))
    assert np.allclose(I[0, 0], folded, rtol=1e-12, atol=1e-12)
    assert wl.H == 4


def test_tiny_workload_brute_force_end_to_end():
    # Whole tiny decode through the oracle (fp32 indexer, no FP8): the
    # selected set must hold exactly the top-32 scores of the causal prefix.
    wl = synth.workload("tiny")
    x = synth.make_inputs(wl)
    cos, sin = oracle.rope_table(wl.Lmax)
    lat = synth.bf16_bits_to_f32(x["latent"])
    kpe = synth.bf16_bits_to_f32(x["kpe"])
    qm = synth.bf16_bits_to_f32(x["q_mla"])
    res = oracle.decode_path(x["q_raw"], x["k_raw"], x["pos"], x["w"], cos, sin, qm, lat, kpe,
                             wl.K, wl.softmax_scale, bf16_input=False, quantized=False)
    sc = res["scores"][0, 0]
    idx = res["idx"][0, 0]
    assert idx.shape == (32,) and np.all(np.diff(idx) > 0)
    kth = np.sort(sc)[::-1][31]
    assert np.all(sc[idx] >= kth)
    assert np.sum(sc > kth) <= 31
    assert res["out"].shape == (1, 1, 8, 512)
