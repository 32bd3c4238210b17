"""GPU parity of call 3 (sparse latent attention, absorbed form) against the
oracle: max-abs error <= 2e-2 on the bf16 output (fp32 accumulation on the
GPU, fp64 in the oracle, same bf16 inputs and the same selection)."""
import numpy as np
import pytest

import oracle
import sparse_attention_index_amd as dsa
import synth
from gpu_util import MLA_ATOL, dev, dev_bf16, host, host_bf16_as_f32, say

pytestmark = pytest.mark.gpu


def oracle_on_selection(q_bits, lat_bits, kpe_bits, idx, scale):
    """Oracle output on the selected rows only (the unselected rows do not
    enter the computation); compacting keeps the fp64 input arrays small."""
    B, S, K = idx.shape
    outs, lses = [], []
    for b in range(B):
        rows = np.unique(idx[b][idx[b] >= 0])
        remap = np.full(lat_bits.shape[1] + 1, -1, np.int64)
        remap[rows] = np.arange(rows.size)
        ib = np.where(idx[b] >= 0, remap[np.where(idx[b] >= 0, idx[b], -1)], -1).astype(np.int32)
        lat = synth.bf16_bits_to_f32(lat_bits[b, rows])[None] if rows.size else np.zeros((1, 1, 512))
        pe = synth.bf16_bits_to_f32(kpe_bits[b, rows])[None] if rows.size else np.zeros((1, 1, 64))
        o, l = oracle.sparse_mla(synth.bf16_bits_to_f32(q_bits[b])[None], lat, pe, ib[None], scale)
        outs.append(o[0])
        lses.append(l[0])
    return np.stack(outs), np.stack(lses)


def report(label, g, gl, o, ol):
    """Worst observed errors of a case (stated beside the bar): max-abs on the
    output, its ratio to the largest |output|, max-abs on the finite lse."""
    err = float(np.abs(g - o).max())
    fin = np.isfinite(ol)
    lerr = float(np.abs(gl[fin] - ol[fin]).max(initial=0.0))
    say(f"  {label}: max abs err {err:.3e} (largest |out| {np.abs(o).max():.3f}), "
        f"lse max abs err {lerr:.3e}")
    return err


def run_case(B, S, Hq, L, K, n_valid, seed, fill=1.0, fused=False, scale=192 ** -0.5):
    import torch
    g = synth.rng(seed)
    q = synth.to_bf16_bits(g.standard_normal((B, S, Hq, 576), dtype=np.float32))
    lat = synth.to_bf16_bits(g.standard_normal((B, L, 512), dtype=np.float32))
    kpe = synth.to_bf16_bits(g.standard_normal((B, L, 64), dtype=np.float32))
    idx = synth.random_selection(seed + 1, B * S, K, np.broadcast_to(n_valid, (B * S,)),
                                 fill).reshape(B, S, K)
    if fused:
        cache = dev_bf16(np.concatenate([lat, kpe], -1))          # [B, L, 576]
        dlat, dpe = cache[..., :512], cache[..., 512:]
    else:
        dlat, dpe = dev_bf16(lat), dev_bf16(kpe)
    out, lse = dsa.sparse_mla(dev_bf16(q), dlat, dpe, dev(idx), scale, return_lse=True)
    torch.cuda.synchronize()
    o, ol = oracle_on_selection(q, lat, kpe, idx, scale)
    return host_bf16_as_f32(out), host(lse), o, ol, idx


CASES = [
    # name, B, S, Hq, L, K, n_valid, fill
    ("tiny", 1, 1, 8, 256, 32, 256, 0.125),
    ("decode16k", 1, 1, 128, 16384, 2048, 16384, 0.125),
    ("batch4-partial", 4, 1, 128, 3000, 2048, 3000, 0.5),
    ("short-rows", 2, 3, 128, 100, 2048, 100, 1.0),
    ("heads20", 1, 2, 20, 900, 256, 900, 0.2),
    ("heads1", 1, 1, 1, 500, 64, 500, 0.1),
    ("prefill-rows", 1, 300, 128, 600, 256, 600, 0.4),
    # long selections over more blocks than CUs (whole rows; a partial head
    # group; two splits per row with merge)
    ("long-rows", 1, 300, 128, 1200, 1024, 1200, 0.6),
    ("long-heads80", 1, 272, 80, 700, 512, 700, 0.5),
    ("long-split", 1, 130, 128, 2500, 2048, 2500, 0.9),
    # few rows (32-head blocks, one-wave merge): 16 splits; 25 splits (a
    # partial chunk of the merge); two short rows with empty splits
    ("few-split16", 1, 1, 128, 3000, 1024, 3000, 0.7),
    ("few-split25", 1, 1, 64, 4000, 1600, 4000, 0.5),
    ("few-short-rows", 1, 2, 128, 300, 2048, 300, 1.0),
    # the split merges of the batched plans: 13 splits (register merge for up
    # to 16, three masked), 7 splits (register merge for up to 8, one
    # masked) and 22 splits (the LDS-weight merge)
    ("merge-regs16", 1, 20, 128, 2500, 2048, 2500, 0.9),
    ("merge-regs8-masked", 1, 40, 128, 2500, 2048, 2500, 0.9),
    ("merge-lds", 1, 10, 128, 2500, 2048, 2500, 0.9),
]


@pytest.mark.parametrize("name,B,S,Hq,L,K,n_valid,fill", CASES, ids=[c[0] for c in CASES])
def test_mla_parity(name, B, S, Hq, L, K, n_valid, fill):
    say(f"mla case {name}: B={B} S={S} Hq={Hq} L={L} K={K}")
    g, gl, o, ol, idx = run_case(B, S, Hq, L, K, n_valid, 500 + B * S + Hq, fill)
    err = report(name, g, gl, o, ol)
    assert err <= MLA_ATOL
    assert np.allclose(gl, ol, atol=1e-3, rtol=1e-4)


def test_mla_fused_cache_row():
    say("mla fused 576-wide cache rows")
    g, gl, o, ol, _ = run_case(2, 1, 128, 2000, 512, 2000, 77, 0.25, fused=True)
    assert report("fused", g, gl, o, ol) <= MLA_ATOL
    assert np.allclose(gl, ol, atol=1e-3, rtol=1e-4)


def test_mla_empty_selection_and_out_of_range_indices():
    import torch
    g = synth.rng(88)
    B, S, Hq, L, K = 1, 3, 32, 64, 64
    q = synth.to_bf16_bits(g.standard_normal((B, S, Hq, 576), dtype=np.float32))
    lat = synth.to_bf16_bits(g.standard_normal((B, L, 512), dtype=np.float32))
    kpe = synth.to_bf16_bits(g.standard_normal((B, L, 64), dtype=np.float32))
    idx = np.full((B, S, K), -1, np.int32)
    idx[0, 1, :5] = [3, 9, 64, 1000, -7]           # 64 and 1000 are out of range -> skipped
    idx[0, 2, 10] = 63
    out, lse = dsa.sparse_mla(dev_bf16(q), dev_bf16(lat), dev_bf16(kpe), dev(idx), 0.1,
                              return_lse=True)
    torch.cuda.synchronize()
    out, lse = host_bf16_as_f32(out), host(lse)
    assert np.all(out[0, 0] == 0) and np.all(np.isneginf(lse[0, 0]))
    ref_idx = idx.copy()
    ref_idx[(ref_idx >= L) | (ref_idx < 0)] = -1
    o, ol = oracle_on_selection(q, lat, kpe, ref_idx, 0.1)
    assert np.abs(out[0, 1:] - o[0, 1:]).max() <= MLA_ATOL
    assert np.allclose(out[0, 2], synth.bf16_bits_to_f32(lat[0, 63])[None], atol=1e-2)


def test_mla_batched_empty_splits_and_rows():
    """The batched path (128-head ring blocks, 7 key splits, register merge)
    with a sparse selection, so that many splits hold no key at all, and two
    rows with none: those rows give zeros and lse = -inf."""
    import torch
    B, S, Hq, L, K = 1, 40, 128, 3000, 2048
    g = synth.rng(71)
    q = synth.to_bf16_bits(g.standard_normal((B, S, Hq, 576), dtype=np.float32))
    lat = synth.to_bf16_bits(g.standard_normal((B, L, 512), dtype=np.float32))
    kpe = synth.to_bf16_bits(g.standard_normal((B, L, 64), dtype=np.float32))
    idx = synth.random_selection(72, B * S, K, np.full(B * S, L), 0.005).reshape(B, S, K)
    idx[0, 3] = -1
    idx[0, 17] = -1
    say("mla batched path, empty splits and rows")
    out, lse = dsa.sparse_mla(dev_bf16(q), dev_bf16(lat), dev_bf16(kpe), dev(idx), 0.07,
                              return_lse=True)
    torch.cuda.synchronize()
    g_out, g_lse = host_bf16_as_f32(out), host(lse)
    assert np.all(g_out[0, 3] == 0) and np.all(g_out[0, 17] == 0)
    assert np.all(np.isneginf(g_lse[0, 3])) and np.all(np.isneginf(g_lse[0, 17]))
    o, ol = oracle_on_selection(q, lat, kpe, idx, 0.07)
    assert report("empty splits", g_out, g_lse, o, ol) <= MLA_ATOL
    assert np.allclose(g_lse, ol, atol=1e-3, rtol=1e-4)


def test_mla_decode128k_full_size():
    """Full long-context size (B=4, L=131072, K=2048, YaRN softmax scale) on a
    synthetic selection, in the launch configuration the benchmark uses."""
    wl = synth.workload("decode128k")
    say("mla decode128k full size")
    g, gl, o, ol, _ = run_case(wl.B, 1, 128, wl.Lmax, 2048, wl.Lmax, 4242, 2048 / wl.Lmax,
                               scale=wl.softmax_scale)
    assert report("decode128k", g, gl, o, ol) <= MLA_ATOL
    assert np.allclose(gl, ol, atol=1e-3, rtol=1e-4)


def test_mla_is_deterministic():
    a = run_case(2, 1, 128, 4000, 2048, 4000, 99, 0.5)
    b = run_case(2, 1, 128, 4000, 2048, 4000, 99, 0.5)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
