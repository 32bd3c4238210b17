"""GPU parity of call 1 (RoPE table, prepare, lightning-indexer score)
against the oracle, through the C ABI.

The quantised codes and scales must be bit-identical to the oracle's (both
sides take every rounding decision in float32 with one IEEE rounding per
operation); with the optional Hadamard rotation they are held to the
rounding allowance of gpu_util.check_rotated_codes instead. Scores must lie within 1e-3 of the oracle's fp64 score on the
dequantised values, relative to max(|score|, 1% of the row's largest
|score|)."""
import numpy as np
import pytest

import oracle
import sparse_attention_index_amd as dsa
import synth
from gpu_util import (check_rotated_codes, check_scores, dev, dev_act, host, say)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("P,yarn", [(5, False), (16384, False), (131072, True)])
def test_rope_table_matches_oracle(P, yarn):
    say(f"rope_table P={P} yarn={yarn}")
    c, s = dsa.rope_table(P, yarn=yarn)
    oc, os_ = oracle.rope_table(P, yarn=yarn)
    for g, o in ((host(c), oc), (host(s), os_)):
        ulps = np.abs(g.view(np.int32).astype(np.int64) - o.view(np.int32).astype(np.int64))
        # opposite-sign zeros aside, at most one unit in the last place
        same = (g == o)
        assert np.all(same | (ulps <= 1))
        assert np.mean(~same) < 1e-4


def run_indexer(B, S, H, Lmax, pos, act_bf16, seed, yarn=False, w_scale=None, had=False,
                pow2=False):
    """Fill the whole cache with the append-only call, then score with the
    call's own key rows appended again (identical values)."""
    import torch
    g = synth.rng(seed)
    q_raw = g.standard_normal((B, S, H, 128), dtype=np.float32)
    k_all = g.standard_normal((B, Lmax, 128), dtype=np.float32)
    w = g.standard_normal((B, S, H), dtype=np.float32) * np.float32(
        w_scale if w_scale is not None else (H ** -0.5) * 128 ** -0.5)
    if act_bf16:
        q_raw = synth.bf16_bits_to_f32(synth.to_bf16_bits(q_raw))
        k_all = synth.bf16_bits_to_f32(synth.to_bf16_bits(k_all))
    pos = np.asarray(pos, np.int32).reshape(B, S)
    cos, sin = oracle.rope_table(Lmax, yarn=yarn)
    dcos, dsin = dev(cos), dev(sin)
    kc = torch.zeros((B, Lmax, 128), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((B, Lmax), dtype=torch.float32, device="cuda")
    all_pos = np.broadcast_to(np.arange(Lmax, dtype=np.int32), (B, Lmax)).copy()
    dsa.indexer_append(dev_act(k_all, act_bf16), dev(all_pos), dcos, dsin, kc, ks,
                       hadamard=had, pow2_scale=pow2)
    k_call = np.stack([k_all[b, pos[b]] for b in range(B)])          # [B,S,128]
    scores = torch.full((B, S, Lmax), float("nan"), dtype=torch.float32, device="cuda")
    q8 = torch.empty((B, S, H, 128), dtype=torch.uint8, device="cuda")
    qs = torch.empty((B, S, H), dtype=torch.float32, device="cuda")
    dsa.indexer(dev_act(q_raw, act_bf16), dev(w), dev(pos), dcos, dsin, kc, ks, scores,
                k_raw=dev_act(k_call, act_bf16), q_fp8=q8, q_scale=qs, hadamard=had,
                pow2_scale=pow2)
    torch.cuda.synchronize()
    return dict(q_raw=q_raw, k_all=k_all, w=w, pos=pos, cos=cos, sin=sin, kc=host(kc),
                ks=host(ks), q8=host(q8), qs=host(qs), scores=host(scores))


def oracle_indexer(r, act_bf16, had=False, pow2=False):
    B, Lmax = r["k_all"].shape[:2]
    kpos = np.broadcast_to(np.arange(Lmax, dtype=np.int32), (B, Lmax))
    k8, ks, _ = oracle.indexer_prepare(r["k_all"], kpos, r["cos"], r["sin"], act_bf16,
                                       hadamard_rot=had, pow2=pow2)
    q8, qs, _ = oracle.indexer_prepare(r["q_raw"], r["pos"][..., None], r["cos"], r["sin"],
                                       act_bf16, hadamard_rot=had, pow2=pow2)
    sc = oracle.indexer_scores(oracle.dequantize(q8, qs), r["w"], oracle.dequantize(k8, ks),
                               r["pos"] + 1)
    return dict(k8=k8, ks=ks, q8=q8, qs=qs, scores=sc)


CASES = [
    # B, S, H, Lmax, positions, bf16 activations, seed
    ("tiny-shape", 1, 1, 4, 256, [[255]], False, 0),
    ("ragged", 3, 2, 20, 1000, [[999, 5], [0, 640], [63, 64]], True, 101),
    ("one-key", 1, 1, 64, 17, [[0]], True, 102),
    ("tail", 2, 1, 64, 4133, [[4132], [2000]], True, 103),
    ("f32", 1, 3, 64, 700, [[699, 100, 1]], False, 104),
    # more than eight queries per batch row: the 64-query x 128-key tile path
    ("tiles", 2, 70, 64, 400, [list(range(330, 400)), list(range(0, 140, 2))], True, 105),
    # more than 512 key chunks of 256 in the call: blocks loop over chunks; the
    # new keys of rows 0 / 1 fall in a block's second chunk
    ("loop", 6, 1, 64, 30000, [[29999], [12345], [0], [20000], [1792], [255]], True, 106),
    ("loop-f32", 3, 1, 64, 50000, [[49999], [30001], [70]], False, 107),
]


@pytest.mark.parametrize("name,B,S,H,Lmax,pos,bf16,seed", CASES, ids=[c[0] for c in CASES])
def test_indexer_parity(name, B, S, H, Lmax, pos, bf16, seed):
    say(f"indexer case {name}: B={B} S={S} H={H} Lmax={Lmax}")
    r = run_indexer(B, S, H, Lmax, pos, bf16, seed)
    o = oracle_indexer(r, bf16)
    assert np.array_equal(r["q8"], o["q8"]) and np.array_equal(r["qs"], o["qs"])
    assert np.array_equal(r["kc"], o["k8"]) and np.array_equal(r["ks"], o["ks"])
    n_valid = r["pos"] + 1
    gs = r["scores"].reshape(B * S, Lmax)
    worst = check_scores(gs, o["scores"].reshape(B * S, Lmax), n_valid, name)
    say(f"  worst normalised score error {worst:.2e}")
    for row, n in enumerate(n_valid.reshape(-1)):
        assert np.all(np.isnan(gs[row, n:])), "entries past the causal end were written"


def test_indexer_decode16k_full_size():
    wl = synth.workload("decode16k")
    say("indexer decode16k full size")
    r = run_indexer(wl.B, wl.S, wl.H, wl.Lmax, synth.positions(wl), True, wl.seed,
                    w_scale=wl.w_scale)
    o = oracle_indexer(r, True)
    assert np.array_equal(r["kc"], o["k8"]) and np.array_equal(r["ks"], o["ks"])
    assert np.array_equal(r["q8"], o["q8"]) and np.array_equal(r["qs"], o["qs"])
    worst = check_scores(r["scores"][:, 0], o["scores"][:, 0], r["pos"][:, 0] + 1, "decode16k")
    say(f"  worst normalised score error {worst:.2e}")


def test_indexer_zero_and_extreme_rows():
    """All-zero rows quantise to scale 1 and zero codes; rows mixing huge and
    tiny magnitudes exercise saturation-free scaling and E4M3 subnormals."""
    import torch
    B, S, H, Lmax = 1, 1, 16, 64
    g = synth.rng(7)
    q_raw = g.standard_normal((B, S, H, 128)).astype(np.float32)
    q_raw[0, 0, 0] = 0.0
    q_raw[0, 0, 1] *= np.float32(1e-6)
    q_raw[0, 0, 2, :3] = np.float32(3e4)
    q_raw[0, 0, 3] = np.exp2(g.integers(-30, 10, size=128)).astype(np.float32)
    k_all = g.standard_normal((B, Lmax, 128)).astype(np.float32)
    k_all[0, 5] = 0.0
    k_all[0, 6] = np.exp2(g.integers(-30, 10, size=128)).astype(np.float32)
    w = g.standard_normal((B, S, H)).astype(np.float32)
    pos = np.array([[Lmax - 1]], np.int32)
    cos, sin = oracle.rope_table(Lmax)
    kc = torch.zeros((B, Lmax, 128), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((B, Lmax), dtype=torch.float32, device="cuda")
    dsa.indexer_append(dev(k_all), dev(np.arange(Lmax, dtype=np.int32)[None]), dev(cos),
                       dev(sin), kc, ks)
    q8 = torch.empty((B, S, H, 128), dtype=torch.uint8, device="cuda")
    qs = torch.empty((B, S, H), dtype=torch.float32, device="cuda")
    sc = dsa.indexer(dev(q_raw), dev(w), dev(pos), dev(cos), dev(sin), kc, ks, q_fp8=q8,
                     q_scale=qs)
    ok8, oks, _ = oracle.indexer_prepare(k_all, np.arange(Lmax, dtype=np.int32)[None], cos,
                                         sin, False)
    oq8, oqs, _ = oracle.indexer_prepare(q_raw, pos[..., None], cos, sin, False)
    assert np.array_equal(host(kc), ok8) and np.array_equal(host(ks), oks)
    assert np.array_equal(host(q8), oq8) and np.array_equal(host(qs), oqs)
    assert host(qs)[0, 0, 0] == 1.0 and np.all(host(q8)[0, 0, 0] & 0x7F == 0)
    o = oracle.indexer_scores(oracle.dequantize(oq8, oqs), w, oracle.dequantize(ok8, oks),
                              pos + 1)
    check_scores(host(sc)[:, 0], o[:, 0], pos[:, 0] + 1, "extreme")


def e4m3_boundary_rows(block_scale=1.0):
    """float32 rows [n, 128] whose quotients x / scale run through every
    finite E4M3 value, every midpoint between neighbouring values (ties to
    even), and the float32 neighbours either side, zeros and tiny values,
    both signs. Feature 0 is fl32(448 * block_scale), which sets the row's
    amax, so the scale is fl32(feature0 / 448). With block_scale = 1 the
    scale is exactly 1 and each code is the E4M3 rounding of the value
    itself. With other block scales (not powers of two) the features are
    fl32(target * scale) and their float32 neighbours, so the quantiser's
    quotient lands on or next to each target: this is where a division by a
    reciprocal, without a correctly rounded correction, would differ."""
    vals = oracle.e4m3_decode(np.arange(128, dtype=np.uint8)).astype(np.float32)
    vals = np.unique(vals[np.isfinite(vals)])                      # 0 .. 448
    mids = ((vals[:-1].astype(np.float64) + vals[1:]) / 2).astype(np.float32)
    amax = np.float32(448.0 * block_scale)
    scale = np.float32(amax / np.float32(448.0))
    if block_scale == 1.0:
        near = np.concatenate([np.nextafter(mids, np.float32(0)),
                               np.nextafter(mids, np.float32(1e9))])
        extra = np.array([1e-40, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -9, 447.99997], np.float32)
        pos_vals = np.concatenate([vals, mids, near, extra]).astype(np.float32)
    else:
        x = (np.concatenate([vals, mids]).astype(np.float64) * np.float64(scale)).astype(np.float32)
        pos_vals = np.concatenate([x, np.nextafter(x, np.float32(0)),
                                   np.nextafter(x, np.float32(1e9)),
                                   np.array([1e-40, 1e-30], np.float32)])
    pos_vals = pos_vals[pos_vals <= amax]
    allv = np.concatenate([pos_vals, -pos_vals, np.array([-0.0], np.float32)])
    n = (allv.size + 126) // 127
    rows = np.zeros((n, 128), np.float32)
    rows[:, 0] = amax
    flat = rows[:, 1:].reshape(-1)
    flat[:allv.size] = allv
    rows[:, 1:] = flat.reshape(n, 127)
    return rows


@pytest.mark.parametrize("block_scale", [1.0, 0.37, 3.0 / 7.0, 1.9])
@pytest.mark.parametrize("S", [1, 2])
def test_fp8_codes_at_rounding_boundaries(S, block_scale):
    """The E4M3 encoder of the key append (every S) and of the query
    preparation (fused decode kernel at S = 1, row preparation at S = 2)
    against the oracle's codec, at position 0 where RoPE is the identity,
    with block scales 1 and three scales that are not powers of two."""
    import torch
    say(f"fp8 boundary codes S={S} block scale {block_scale}")
    rows = e4m3_boundary_rows(block_scale)
    n = rows.shape[0]
    cos, sin = oracle.rope_table(4)
    # keys: n batch rows appended at position 0
    kc = torch.zeros((n, 4, 128), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((n, 4), dtype=torch.float32, device="cuda")
    dsa.indexer_append(dev(rows[:, None]), dev(np.zeros((n, 1), np.int32)), dev(cos), dev(sin),
                       kc, ks)
    ok8, oks, _ = oracle.indexer_prepare(rows, np.zeros(n, np.int32), cos, sin, False)
    if block_scale == 1.0:
        assert np.all(oks == 1.0)
    assert np.array_equal(host(kc)[:, 0], ok8) and np.array_equal(host(ks)[:, 0], oks)
    # queries: the rows as heads of S query rows at position 0
    H = 64
    reps = (S * H + n - 1) // n
    q_rows = np.tile(rows, (reps, 1))[:S * H].reshape(1, S, H, 128)
    w = np.ones((1, S, H), np.float32)
    q8 = torch.empty((1, S, H, 128), dtype=torch.uint8, device="cuda")
    qs = torch.empty((1, S, H), dtype=torch.float32, device="cuda")
    dsa.indexer(dev(q_rows), dev(w), dev(np.zeros((1, S), np.int32)), dev(cos), dev(sin),
                kc[:1], ks[:1], q_fp8=q8, q_scale=qs)
    torch.cuda.synchronize()
    oq8, oqs, _ = oracle.indexer_prepare(q_rows, np.zeros((1, S, H), np.int32), cos, sin, False)
    assert np.array_equal(host(q8), oq8) and np.array_equal(host(qs), oqs)


def test_positions_out_of_range_are_skipped():
    import torch
    B, S, H, Lmax = 2, 1, 8, 128
    g = synth.rng(9)
    cos, sin = oracle.rope_table(Lmax)
    kc = torch.zeros((B, Lmax, 128), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((B, Lmax), dtype=torch.float32, device="cuda")
    scores = torch.full((B, S, Lmax), 7.0, dtype=torch.float32, device="cuda")
    pos = np.array([[-1], [Lmax]], np.int32)
    dsa.indexer(dev(g.standard_normal((B, S, H, 128)).astype(np.float32)),
                dev(np.ones((B, S, H), np.float32)), dev(pos), dev(cos), dev(sin), kc, ks,
                scores, k_raw=dev(g.standard_normal((B, S, 128)).astype(np.float32)))
    torch.cuda.synchronize()
    assert np.all(host(scores) == 7.0)
    assert np.all(host(kc) == 0) and np.all(host(ks) == 0)


FLAG_CASES = [
    # name, B, S, H, Lmax, positions, bf16, seed, hadamard, pow2 scales
    ("had-ragged-bf16", 3, 2, 20, 1000, [[999, 5], [0, 640], [63, 64]], True, 111, True, False),
    ("had-f32", 1, 3, 64, 700, [[699, 100, 1]], False, 112, True, False),
    ("pow2-ragged", 2, 2, 64, 300, [[299, 10], [150, 0]], True, 113, False, True),
    ("had-pow2-tail", 2, 1, 64, 4133, [[4132], [2000]], True, 114, True, True),
    ("had-decode", 1, 1, 64, 2048, [[2047]], True, 115, True, False),
    ("had-pow2-tiles", 1, 20, 64, 300, [list(range(280, 300))], True, 116, True, True),
    # one query row per batch row: the fused decode kernel with the options
    # (looping grid for many key chunks; float32 activations; fewer heads)
    ("had-pow2-loop", 6, 1, 64, 30000, [[29999], [12345], [0], [20000], [1792], [255]], True,
     117, True, True),
    ("had-f32-decode", 1, 1, 64, 700, [[699]], False, 118, True, False),
    ("pow2-decode-h20", 2, 1, 20, 1000, [[999], [5]], True, 119, False, True),
    ("had-decode-h20", 2, 1, 20, 1000, [[999], [5]], True, 120, True, False),
]


@pytest.mark.parametrize("name,B,S,H,Lmax,pos,bf16,seed,had,pow2", FLAG_CASES,
                         ids=[c[0] for c in FLAG_CASES])
def test_indexer_hadamard_pow2_parity(name, B, S, H, Lmax, pos, bf16, seed, had, pow2):
    """The optional Hadamard rotation and power-of-two scales. Without the
    rotation, codes and scales are bit-identical to the oracle's. With it,
    the oracle rotates by the definition (float64 product, one rounding) and
    the GPU by a float32 fast transform, so codes and scales are held to the
    rounding allowance of check_rotated_codes. Scores are within the
    tolerance of the oracle run on the GPU's own codes and scales."""
    say(f"indexer flags case {name}: B={B} S={S} H={H} Lmax={Lmax} had={had} pow2={pow2}")
    r = run_indexer(B, S, H, Lmax, pos, bf16, seed, had=had, pow2=pow2)
    if had:
        kpos = np.broadcast_to(np.arange(Lmax, dtype=np.int32), (B, Lmax))
        k_pre = oracle.rope(r["k_all"], kpos, r["cos"], r["sin"], out_bf16=bf16)
        q_pre = oracle.rope(r["q_raw"], r["pos"][..., None], r["cos"], r["sin"], out_bf16=bf16)
        fk = check_rotated_codes(k_pre, r["kc"], r["ks"], bf16, pow2, name + " keys")
        fq = check_rotated_codes(q_pre, r["q8"], r["qs"], bf16, pow2, name + " queries")
        say(f"  codes equal to the oracle's: keys {fk[0]:.5f}, queries {fq[0]:.5f}; "
            f"scales equal: keys {fk[1]:.4f}, queries {fq[1]:.4f}")
    else:
        o = oracle_indexer(r, bf16, had=had, pow2=pow2)
        assert np.array_equal(r["q8"], o["q8"]) and np.array_equal(r["qs"], o["qs"])
        assert np.array_equal(r["kc"], o["k8"]) and np.array_equal(r["ks"], o["ks"])
    if pow2:
        m, _ = np.frexp(r["qs"].astype(np.float64))
        assert np.all(m == 0.5)
    n_valid = r["pos"] + 1
    osc = oracle.indexer_scores(oracle.dequantize(r["q8"], r["qs"]), r["w"],
                                oracle.dequantize(r["kc"], r["ks"]), n_valid)
    gs = r["scores"].reshape(B * S, Lmax)
    worst = check_scores(gs, osc.reshape(B * S, Lmax), n_valid, name)
    say(f"  worst normalised score error {worst:.2e}")
    for row, n in enumerate(n_valid.reshape(-1)):
        assert np.all(np.isnan(gs[row, n:])), "entries past the causal end were written"


def test_pow2_scales_of_tiny_rows():
    """Rows so small that amax/448 is a float32 subnormal: the power-of-two
    scale is still the oracle's (and zero rows keep scale 1)."""
    import torch
    B, S, H, Lmax = 1, 1, 8, 16
    g = synth.rng(17)
    q_raw = g.standard_normal((B, S, H, 128)).astype(np.float32)
    q_raw[0, 0, 0] *= np.float32(1e-37)
    q_raw[0, 0, 1] *= np.float32(3e-39)
    q_raw[0, 0, 2] = 0.0
    q_raw[0, 0, 3] *= np.float32(1e-30)
    cos, sin = oracle.rope_table(Lmax)
    pos = np.array([[Lmax - 1]], np.int32)
    kc = torch.zeros((B, Lmax, 128), dtype=torch.uint8, device="cuda")
    ks = torch.zeros((B, Lmax), dtype=torch.float32, device="cuda")
    dsa.indexer_append(dev(g.standard_normal((B, Lmax, 128)).astype(np.float32)),
                       dev(np.arange(Lmax, dtype=np.int32)[None]), dev(cos), dev(sin), kc, ks,
                       pow2_scale=True)
    q8 = torch.empty((B, S, H, 128), dtype=torch.uint8, device="cuda")
    qs = torch.empty((B, S, H), dtype=torch.float32, device="cuda")
    dsa.indexer(dev(q_raw), dev(np.ones((B, S, H), np.float32)), dev(pos), dev(cos), dev(sin),
                kc, ks, q_fp8=q8, q_scale=qs, pow2_scale=True)
    oq8, oqs, _ = oracle.indexer_prepare(q_raw, pos[..., None], cos, sin, False, pow2=True)
    assert np.array_equal(host(qs), oqs) and np.array_equal(host(q8), oq8)
    assert host(qs)[0, 0, 2] == 1.0
