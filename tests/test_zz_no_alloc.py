"""dsa_sparse_mla_noalloc (the call for callers that cannot allocate) against
dsa_sparse_mla: two calls in a row through the C ABI, the second with a
smaller input, each bit-identical to the workspace call on the same inputs
and within the attention bar of the oracle (max-abs 2e-2 on the bf16 output,
lse within 1e-3). The static scratch keeps the first call's contents when
the second one runs; nothing in it has to start at any value."""
import numpy as np
import pytest

import sparse_attention_index_amd as dsa
import synth
from gpu_util import MLA_ATOL, dev, dev_bf16, host, host_bf16_as_f32, say
from test_gpu_mla import oracle_on_selection

pytestmark = pytest.mark.gpu


def inputs(seed, B, S, Hq, L, K, fill):
    g = synth.rng(seed)
    q = synth.to_bf16_bits(g.standard_normal((B, S, Hq, 576), dtype=np.float32))
    lat = synth.to_bf16_bits(g.standard_normal((B, L, 512), dtype=np.float32))
    kpe = synth.to_bf16_bits(g.standard_normal((B, L, 64), dtype=np.float32))
    idx = synth.random_selection(seed + 1, B * S, K, np.full(B * S, L), fill).reshape(B, S, K)
    return q, lat, kpe, idx


def test_noalloc_matches_workspace_call_twice():
    import torch
    scale = 192 ** -0.5
    # first call: 4 decode rows of 2048 selected keys (32 key splits per row,
    # 16 MiB of partials); second: one row, 64 heads, 1000 keys (smaller)
    for case, (B, S, Hq, L, K, fill) in enumerate([(4, 1, 128, 8192, 2048, 0.25),
                                                   (1, 1, 64, 3000, 1000, 0.33)]):
        say(f"noalloc call {case}: B={B} S={S} Hq={Hq} L={L} K={K}")
        q, lat, kpe, idx = inputs(900 + case, B, S, Hq, L, K, fill)
        dq, dlat, dkpe, didx = dev_bf16(q), dev_bf16(lat), dev_bf16(kpe), dev(idx)
        out = torch.full((B, S, Hq, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, S, Hq), float("nan"), dtype=torch.float32, device="cuda")
        a = dsa.mla_args(dq, dlat, dkpe, didx, scale, out, lse)
        assert dsa.sparse_mla_workspace_bytes(a) > 0          # the split path runs
        dsa.sparse_mla_noalloc(dq, dlat, dkpe, didx, scale, out, lse)
        ref_out, ref_lse = dsa.sparse_mla(dq, dlat, dkpe, didx, scale, return_lse=True)
        torch.cuda.synchronize()
        assert np.array_equal(host(out.view(torch.int16)), host(ref_out.view(torch.int16)))
        assert np.array_equal(host(lse), host(ref_lse))
        o, ol = oracle_on_selection(q, lat, kpe, idx, scale)
        err = float(np.abs(host_bf16_as_f32(out) - o).max())
        say(f"  bit-identical to dsa_sparse_mla; max abs err vs oracle {err:.3e}")
        assert err <= MLA_ATOL
        assert np.allclose(host(lse), ol, rtol=0, atol=1e-3)


def test_noalloc_batched_merges():
    """The batched plans' split merges on the static scratch: 40 rows of 2048
    keys (7 splits, the register merge for up to 8), then 20 rows (13 splits,
    the register merge for up to 16), each bit-identical to the workspace
    call and within the attention bar of the oracle."""
    import torch
    scale = 192 ** -0.5
    for case, (S, L) in enumerate([(40, 2500), (20, 2200)]):
        say(f"noalloc batched call {case}: S={S} Hq=128 L={L} K=2048")
        q, lat, kpe, idx = inputs(960 + case, 1, S, 128, L, 2048, 0.9)
        dq, dlat, dkpe, didx = dev_bf16(q), dev_bf16(lat), dev_bf16(kpe), dev(idx)
        out = torch.full((1, S, 128, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((1, S, 128), float("nan"), dtype=torch.float32, device="cuda")
        dsa.sparse_mla_noalloc(dq, dlat, dkpe, didx, scale, out, lse)
        ref_out, ref_lse = dsa.sparse_mla(dq, dlat, dkpe, didx, scale, return_lse=True)
        torch.cuda.synchronize()
        assert np.array_equal(host(out.view(torch.int16)), host(ref_out.view(torch.int16)))
        assert np.array_equal(host(lse), host(ref_lse))
        o, ol = oracle_on_selection(q, lat, kpe, idx, scale)
        err = float(np.abs(host_bf16_as_f32(out) - o).max())
        say(f"  bit-identical to dsa_sparse_mla; max abs err vs oracle {err:.3e}")
        assert err <= MLA_ATOL
        assert np.allclose(host(lse), ol, rtol=0, atol=1e-3)


def test_noalloc_rejects_more_than_its_scratch():
    import torch
    B, Hq, L, K = 230, 128, 256, 2048                        # 230 rows: ~58 MiB of partials
    q, lat, kpe, idx = inputs(950, B, 1, Hq, L, K, 1.0)
    out = torch.zeros((B, 1, Hq, 512), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsa.DSAError) as e:
        dsa.sparse_mla_noalloc(dev_bf16(q), dev_bf16(lat), dev_bf16(kpe), dev(idx), 0.1, out)
    assert e.value.code == dsa.DSA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert not host(out.view(torch.int16)).any()             # nothing was launched
