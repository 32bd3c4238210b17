"""GPU parity of the MLA-side cache append (dsa_mla_append) against the
oracle's interleaved RoPE (page "RoPE coefficients", MLA prefill excerpt;
aipricedb update note: MLA pairs features 2j and 2j+1). Everything is
bit-exact: the latent copy, and the rotated bf16 rotary keys and query
rope parts (both sides: float32 products, one rounding per operation, then
bf16)."""
import numpy as np
import pytest

import oracle
import sparse_attention_index_amd as dsa
import synth
from gpu_util import dev, dev_bf16, host, say

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1          # a bf16 NaN pattern the call never writes


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_append(B, S, Hq, Lmax, pos, seed, yarn=False, fused=False, with_q=True):
    import torch
    g = synth.rng(seed)
    lat_new = synth.to_bf16_bits(g.standard_normal((B, S, 512), dtype=np.float32))
    kpe_new = synth.to_bf16_bits(g.standard_normal((B, S, 64), dtype=np.float32) * 3)
    q = synth.to_bf16_bits(g.standard_normal((B, S, Hq, 576), dtype=np.float32))
    pos = np.asarray(pos, np.int32).reshape(B, S)
    cos, sin = oracle.rope_table(Lmax, yarn=yarn)
    if fused:
        cache = dev_bf16(np.full((B, Lmax, 576), SENTINEL, np.uint16))
        latent, rope = cache[..., :512], cache[..., 512:]
    else:
        latent = dev_bf16(np.full((B, Lmax, 512), SENTINEL, np.uint16))
        rope = dev_bf16(np.full((B, Lmax, 64), SENTINEL, np.uint16))
    dq = dev_bf16(q) if with_q else None
    dsa.mla_append(dev_bf16(lat_new), dev_bf16(kpe_new), dev(pos), dev(cos), dev(sin), latent,
                   rope, q=dq)
    torch.cuda.synchronize()
    return dict(lat_new=lat_new, kpe_new=kpe_new, q=q, pos=pos, cos=cos, sin=sin,
                latent=_bits(latent), rope=_bits(rope), q_out=_bits(dq) if with_q else None)


def check(r, Lmax):
    B, S = r["pos"].shape
    valid = (r["pos"] >= 0) & (r["pos"] < Lmax)
    f = synth.bf16_bits_to_f32
    safe = np.where(valid, r["pos"], 0)
    kpe_rot = synth.to_bf16_bits(oracle.rope(f(r["kpe_new"]), safe, r["cos"], r["sin"],
                                             rope_dim=64, interleaved=True, out_bf16=True))
    q_rope = synth.to_bf16_bits(oracle.rope(f(r["q"][..., 512:]), safe[..., None], r["cos"],
                                            r["sin"], rope_dim=64, interleaved=True,
                                            out_bf16=True))
    written = np.zeros((B, Lmax), bool)
    for b in range(B):
        for s in range(S):
            if not valid[b, s]:
                continue
            p = r["pos"][b, s]
            written[b, p] = True
            assert np.array_equal(r["latent"][b, p], r["lat_new"][b, s])
            assert np.array_equal(r["rope"][b, p], kpe_rot[b, s])
    assert np.all(r["latent"][~written] == SENTINEL)
    assert np.all(r["rope"][~written] == SENTINEL)
    if r["q_out"] is not None:
        assert np.array_equal(r["q_out"][..., :512], r["q"][..., :512])
        exp = np.where(valid[..., None, None], q_rope, r["q"][..., 512:])
        assert np.array_equal(r["q_out"][..., 512:], exp)


CASES = [
    # name, B, S, Hq, Lmax, positions, yarn, fused cache
    ("decode", 1, 1, 128, 16384, [[16383]], False, False),
    ("ragged-invalid", 3, 2, 20, 300, [[299, 0], [-1, 17], [300, 150]], False, False),
    ("prefill", 1, 64, 128, 64, [list(range(64))], False, True),
    ("yarn", 2, 1, 1, 131072, [[131071], [65536]], True, False),
]


@pytest.mark.parametrize("name,B,S,Hq,Lmax,pos,yarn,fused", CASES, ids=[c[0] for c in CASES])
def test_mla_append_parity(name, B, S, Hq, Lmax, pos, yarn, fused):
    say(f"mla_append case {name}: B={B} S={S} Hq={Hq} Lmax={Lmax}")
    r = run_append(B, S, Hq, Lmax, pos, seed=300 + len(name), yarn=yarn, fused=fused)
    check(r, Lmax)


def test_mla_append_without_q():
    say("mla_append without q")
    r = run_append(2, 3, 8, 64, [[1, 2, 3], [63, 0, 5]], seed=311, with_q=False)
    check(r, 64)


def test_rotation_preserves_pair_norms_and_attention_scores_shift():
    """The rotated rope cache and rotated query rope parts give the relative-
    position score structure: q_pe(p) . k_pe(p') depends on p - p' only."""
    import torch
    g = synth.rng(320)
    L = 64
    cos, sin = oracle.rope_table(L)
    kpe = synth.to_bf16_bits(np.tile(g.standard_normal((1, 1, 64), dtype=np.float32), (1, L, 1)))
    latent = dev_bf16(np.zeros((1, L, 512), np.uint16))
    rope = dev_bf16(np.zeros((1, L, 64), np.uint16))
    dsa.mla_append(dev_bf16(np.zeros((1, L, 512), np.uint16)), dev_bf16(kpe),
                   dev(np.arange(L, dtype=np.int32)[None]), dev(cos), dev(sin), latent, rope)
    torch.cuda.synchronize()
    k = synth.bf16_bits_to_f32(_bits(rope))[0].astype(np.float64)      # [L, 64]
    n0 = np.linalg.norm(synth.bf16_bits_to_f32(kpe)[0, 0].reshape(32, 2), axis=1)
    nk = np.linalg.norm(k.reshape(L, 32, 2), axis=2)
    assert np.allclose(nk, n0[None], rtol=1e-2)
    d1 = k[10] @ k[7]
    d2 = k[40] @ k[37]
    assert abs(d1 - d2) <= 2e-2 * np.linalg.norm(k[10]) * np.linalg.norm(k[7])
