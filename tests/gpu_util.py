"""Helpers shared by the GPU parity tests: device transfers, the indexer
tolerance rule and the end-to-end top-k comparison rule."""
from __future__ import annotations

import sys

import numpy as np

INDEXER_RTOL = 1e-3          # relative, with a row floor (see check_scores)
ROW_FLOOR = 0.01             # fraction of the row's largest |score|
MLA_ATOL = 2e-2              # max-abs on the bf16 attention output


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def dev_bf16(bits):
    """uint16 bit patterns -> a bfloat16 device tensor with those bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to("cuda")


def dev_act(values_f32, bf16: bool):
    """Activation values (already bf16-representable when bf16) -> device."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16) if bf16 else t


def host(t):
    return t.detach().cpu().numpy()


def host_bf16_as_f32(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def score_errors(g, o):
    """Normalised error of GPU scores g against oracle scores o over one row:
    |g - o| / max(|o|, ROW_FLOOR * max|o|)."""
    o = np.asarray(o, np.float64)
    g = np.asarray(g, np.float64)
    floor = ROW_FLOOR * np.max(np.abs(o)) if o.size else 0.0
    den = np.maximum(np.abs(o), floor)
    den = np.where(den > 0, den, 1.0)
    return np.abs(g - o) / den


def check_scores(g_rows, o_rows, n_valid, label=""):
    worst = 0.0
    for r, n in enumerate(np.asarray(n_valid).reshape(-1)):
        if n <= 0:
            continue
        e = score_errors(g_rows[r, :n], o_rows[r, :n])
        worst = max(worst, float(e.max()))
        assert np.all(np.isfinite(g_rows[r, :n])), (label, r)
        assert e.max() <= INDEXER_RTOL, (label, r, float(e.max()), int(e.argmax()))
    return worst


def check_topk_membership(g_idx, o_idx, o_scores, n_valid, K, label=""):
    """End-to-end top-k rule: GPU and oracle selections may differ only in
    positions whose oracle score lies within the indexer tolerance of the
    oracle's k-th score; both must be ascending, unique, causal, -1 padded."""
    mismatched_rows = 0
    for r, n in enumerate(np.asarray(n_valid).reshape(-1)):
        keff = min(K, int(n))
        gi, oi = g_idx[r], o_idx[r]
        assert np.all(gi[keff:] == -1) and np.all(oi[keff:] == -1), (label, r)
        gs = gi[:keff]
        assert np.all(np.diff(gs) > 0) and gs.min(initial=0) >= 0 and gs.max(initial=-1) < n
        if np.array_equal(gs, oi[:keff]):
            continue
        mismatched_rows += 1
        sc = np.asarray(o_scores[r, :n], np.float64)
        kth = np.sort(sc)[::-1][keff - 1]
        tol = INDEXER_RTOL * max(abs(kth), ROW_FLOOR * np.max(np.abs(sc)))
        diff = np.setxor1d(gs, oi[:keff])
        assert np.all(np.abs(sc[diff] - kth) <= tol), (label, r, diff[:8], sc[diff][:8], kth)
    return mismatched_rows


def check_topk_properties(scores, idx, n_valid, K, label=""):
    """Top-k properties on the GPU's own scores (any size): k_eff entries,
    ascending, unique, causal; every selected score >= every unselected one;
    among scores equal to the threshold the lowest positions are taken."""
    for r, n in enumerate(np.asarray(n_valid).reshape(-1)):
        n = int(n)
        keff = min(K, n)
        sel = idx[r, :keff]
        assert np.all(idx[r, keff:] == -1), (label, r)
        assert np.all(np.diff(sel) > 0) and sel.min(initial=0) >= 0 and sel.max(initial=-1) < n
        s = np.asarray(scores[r, :n], np.float64)
        s = np.where(s == 0.0, 0.0, s)
        mask = np.zeros(n, bool)
        mask[sel] = True
        if keff == n:
            continue
        thr = s[mask].min()
        assert thr >= s[~mask].max(), (label, r)
        ties_out = np.nonzero((~mask) & (s == thr))[0]
        ties_in = np.nonzero(mask & (s == thr))[0]
        if ties_out.size:
            assert ties_in.max() < ties_out.min(), (label, r)


def check_rotated_codes(x_pre, g_codes, g_scales, act_bf16, pow2, label=""):
    """Codes and scales of Hadamard-rotated rows, judged against the oracle's
    rotation (the definition H x / sqrt(128): a float64 sum rounded once) with
    an allowance for the GPU's float32 fast transform.

    x_pre: float32 [N, 128], the rows fed to the rotation. The GPU adds
    a +- b in float32 at 7 levels and multiplies by fl32(128^-0.5): its value
    lies within delta = 10 u sum|x| / sqrt(128) of the exact product (7
    additions, the constant's and the product's rounding, u = 2^-24; the
    oracle's own rounding adds u |y|). A GPU value is therefore any float32
    in [y - delta, y + delta], cast to bfloat16 when the activations are
    bf16. The scale must come from an amax inside the range those values
    allow, and each code must be the E4M3 encoding of the quotient of one of
    them by the GPU's own scale. Returns (fraction of codes equal to the
    oracle's, fraction of scales equal)."""
    import oracle
    u = 2.0 ** -24
    x = np.asarray(x_pre, np.float32).reshape(-1, 128)
    codes = np.asarray(g_codes, np.uint8).reshape(-1, 128)
    scales = np.asarray(g_scales, np.float32).reshape(-1)
    y = oracle.hadamard(x).astype(np.float64)
    delta = 10 * u * np.abs(x.astype(np.float64)).sum(axis=1, keepdims=True) / np.sqrt(128.0) \
        + u * np.abs(y)
    lo = np.nextafter((y - delta).astype(np.float32), np.float32(-np.inf))
    hi = np.nextafter((y + delta).astype(np.float32), np.float32(np.inf))
    if act_bf16:
        lo, hi = oracle.round_bf16(lo), oracle.round_bf16(hi)
    lo64, hi64 = lo.astype(np.float64), hi.astype(np.float64)
    straddle = (lo64 <= 0) & (hi64 >= 0)
    amin = np.where(straddle, 0.0, np.minimum(np.abs(lo64), np.abs(hi64)))
    amax_lo = amin.max(axis=1)
    amax_hi = np.maximum(np.abs(lo64), np.abs(hi64)).max(axis=1)
    s_lo = (amax_lo.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    s_hi = (amax_hi.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    if pow2:
        p2 = lambda s: np.where(s > 0, 2.0 ** np.ceil(np.log2(np.maximum(s, 1e-45))), 1.0)
        s_lo, s_hi = p2(s_lo.astype(np.float64)), p2(s_hi.astype(np.float64))
    bad_s = np.nonzero((scales < s_lo) | (scales > s_hi))[0]
    assert bad_s.size == 0, (label, "scale outside the allowance", bad_s[:4],
                             scales[bad_s[:4]], s_lo[bad_s[:4]], s_hi[bad_s[:4]])
    sc = scales[:, None]
    q_lo = oracle.e4m3_decode(oracle.e4m3_encode(lo / sc))
    q_hi = oracle.e4m3_decode(oracle.e4m3_encode(hi / sc))
    got = oracle.e4m3_decode(codes)
    bad = np.argwhere((got < q_lo) | (got > q_hi))
    assert bad.size == 0, (label, "code outside the allowance", bad[:4])
    o_codes, o_scales = oracle.quantize(oracle.hadamard(x, out_bf16=act_bf16), pow2=pow2)
    return float(np.mean(codes == o_codes)), float(np.mean(scales == o_scales))
