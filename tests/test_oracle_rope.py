"""Pins of the oracle's rotary table and rotary embedding.

Pairing (page "Rotate first features", its description and the
apply_rotary_emb excerpt; the 2025.11.17 update note on the aipricedb page):
the indexer pairs feature j with j+32 (non-interleaved), MLA pairs 2j with
2j+1 (interleaved). The worked example below is derived by hand from that
rule for x = (1, 2, ..., 64) at position 3 with theta_j = 10000^(-j/32):
  non-interleaved: y[0]  = cos 3 - 33 sin 3,  y[32] = sin 3 + 33 cos 3
  interleaved:     y[0]  = cos 3 - 2 sin 3,   y[1]  = sin 3 + 2 cos 3
"""
import math

import numpy as np
import pytest

import oracle


def closed_form_row(pos, npairs=32, base=10000.0):
    """cos/sin of pos*theta_i evaluated in double from the definition."""
    th = [base ** (-2.0 * i / (2 * npairs)) for i in range(npairs)]
    c = np.array([[math.cos(pos * t) for t in th]], np.float32)
    s = np.array([[math.sin(pos * t) for t in th]], np.float32)
    return c, s, th


def test_worked_example_pairings():
    x = np.arange(1, 65, dtype=np.float32)[None, :]
    c, s, th = closed_form_row(3)
    # place the single row at table row 0 and rotate with pos 0 -> uses that row
    ni = oracle.rope(x, np.array([0]), c, s, rope_dim=64, interleaved=False)[0]
    il = oracle.rope(x, np.array([0]), c, s, rope_dim=64, interleaved=True)[0]
    assert ni[0] == pytest.approx(math.cos(3) - 33 * math.sin(3), rel=1e-6)
    assert ni[0] == pytest.approx(-5.64695, abs=1e-5)
    assert ni[32] == pytest.approx(math.sin(3) + 33 * math.cos(3), rel=1e-6)
    assert ni[32] == pytest.approx(-32.52863, abs=1e-5)
    t31 = 3 * th[31]
    assert ni[63] == pytest.approx(32 * math.sin(t31) + 64 * math.cos(t31), rel=1e-6)
    assert ni[63] == pytest.approx(64.01280, abs=1e-5)
    assert il[0] == pytest.approx(math.cos(3) - 2 * math.sin(3), rel=1e-6)
    assert il[0] == pytest.approx(-1.27223, abs=1e-5)
    assert il[1] == pytest.approx(math.sin(3) + 2 * math.cos(3), rel=1e-6)
    assert il[1] == pytest.approx(-1.83886, abs=1e-5)


def test_pairings_are_a_permutation_of_each_other():
    g = np.random.Generator(np.random.PCG64(21))
    x = g.standard_normal((64, 128)).astype(np.float32)
    pos = g.integers(0, 4096, size=64).astype(np.int32)
    cos, sin = oracle.rope_table(4096)
    perm = np.empty(64, np.int64)          # (Px)[2j] = x[j], (Px)[2j+1] = x[j+32]
    perm[0::2] = np.arange(32)
    perm[1::2] = np.arange(32) + 32
    xp = x.copy()
    xp[:, :64] = x[:, perm]
    il = oracle.rope(xp, pos, cos, sin, rope_dim=64, interleaved=True)
    back = il.copy()
    back[:, perm] = il[:, :64]
    ni = oracle.rope(x, pos, cos, sin, rope_dim=64, interleaved=False)
    assert np.array_equal(ni, back)
    assert np.array_equal(ni[:, 64:], x[:, 64:])     # features 64..127 pass through


def test_identity_at_position_zero_and_norm_preserved():
    g = np.random.Generator(np.random.PCG64(22))
    x = g.standard_normal((32, 128)).astype(np.float32)
    cos, sin = oracle.rope_table(1000)
    y0 = oracle.rope(x, np.zeros(32, np.int32), cos, sin)
    assert np.array_equal(y0, x)
    pos = g.integers(0, 1000, size=32).astype(np.int32)
    y = oracle.rope(x, pos, cos, sin).astype(np.float64)
    xd = x.astype(np.float64)
    n_in = xd[:, :32] ** 2 + xd[:, 32:64] ** 2
    n_out = y[:, :32] ** 2 + y[:, 32:64] ** 2
    assert np.allclose(n_out, n_in, rtol=1e-5, atol=1e-6)


def test_dot_products_depend_on_relative_position():
    g = np.random.Generator(np.random.PCG64(23))
    q = g.standard_normal((1, 128)).astype(np.float32)
    k = g.standard_normal((1, 128)).astype(np.float32)
    cos, sin = oracle.rope_table(2048)
    dots = []
    for m, n in [(10, 3), (110, 103), (1007, 1000)]:
        qm = oracle.rope(q, np.array([m]), cos, sin).astype(np.float64)
        kn = oracle.rope(k, np.array([n]), cos, sin).astype(np.float64)
        dots.append(float((qm * kn).sum()))
    assert dots[1] == pytest.approx(dots[0], rel=1e-4, abs=1e-4)
    assert dots[2] == pytest.approx(dots[0], rel=1e-4, abs=1e-4)


def test_plain_table_matches_definition():
    P = 16384
    cos, sin = oracle.rope_table(P)
    th = np.array([10000.0 ** (-2.0 * i / 64) for i in range(32)])
    p = np.arange(P, dtype=np.float64)[:, None]
    ang = p * th[None, :]
    # the table is built from float32 angles: allow the float32 rounding of
    # theta and of the product (|d ang| <= ang * 2^-23) plus float32 output rounding
    tol = ang * 2.0 ** -23 + 2.0 ** -24 * 2
    assert np.all(np.abs(cos - np.cos(ang)) <= tol)
    assert np.all(np.abs(sin - np.sin(ang)) <= tol)
    assert np.all(cos[0] == 1.0) and np.all(sin[0] == 0.0)


def test_bf16_cast_back():
    g = np.random.Generator(np.random.PCG64(24))
    x = g.standard_normal((8, 128)).astype(np.float32)
    cos, sin = oracle.rope_table(100)
    pos = np.arange(8, dtype=np.int32) * 7
    y32 = oracle.rope(x, pos, cos, sin)
    y16 = oracle.rope(x, pos, cos, sin, out_bf16=True)
    assert np.array_equal(y16, oracle.round_bf16(y32))


def test_yarn_frequency_invariants():
    plain = oracle.rope_freqs(64).astype(np.float64)
    yarn = oracle.rope_freqs(64, yarn=True, orig_len=4096, factor=40.0,
                             beta_fast=32.0, beta_slow=1.0).astype(np.float64)
    ratio = yarn / plain
    assert ratio[0] == 1.0
    assert ratio[31] == pytest.approx(1 / 40, rel=1e-6)
    assert np.all(np.diff(ratio) <= 1e-7)
    assert np.all((ratio >= 1 / 40 - 1e-7) & (ratio <= 1 + 1e-7))
    # low-frequency pairs are fully interpolated, high-frequency ones untouched
    assert np.sum(ratio == 1.0) >= 8 and np.sum(np.isclose(ratio, 1 / 40)) >= 8
    # plain frequencies are the float32 values of 10000^(-2i/64)
    ref = np.array([10000.0 ** (-2.0 * i / 64) for i in range(32)])
    assert np.all(np.abs(plain - ref) <= ref * 2.0 ** -24)


@pytest.mark.parametrize("orig,factor,bf,bs", [(4096, 40.0, 32.0, 1.0), (4096, 40.0, 16.0, 2.0),
                                                 (8192, 8.0, 32.0, 1.0)])
def test_yarn_ramp_follows_rotation_counts(orig, factor, bf, bs):
    """The YaRN ramp's end points, pinned by the YaRN paper's rule stated in
    wavelengths (Peng et al. 2023): a pair that turns more than beta_fast
    times over the original context keeps its frequency, one that turns less
    than beta_slow times is fully interpolated (divided by the factor), and
    the pairs in between are blended; the page's excerpt makes the blend
    linear in the pair index (linear_ramp_factor(low, high, dim // 2)).
    Rotation counts come from the wavelength 2 pi / theta_i here, not from
    the oracle's correction-dimension formula, so a low rounded up or a
    high rounded down (or swapped betas) fails."""
    plain = oracle.rope_freqs(64).astype(np.float64)
    yarn = oracle.rope_freqs(64, yarn=True, orig_len=orig, factor=factor, beta_fast=bf,
                             beta_slow=bs).astype(np.float64)
    ratio = yarn / plain
    theta = np.array([10000.0 ** (-2.0 * i / 64) for i in range(32)])
    turns = orig / (2 * np.pi / theta)                    # rotations over the original context
    keep = turns > bf
    full = turns < bs
    assert keep.any() and full.any()
    assert np.all(ratio[keep] == 1.0)
    assert np.allclose(ratio[full], 1 / factor, rtol=1e-6)
    mid = ~keep & ~full
    assert np.all((ratio[mid] > 1 / factor * (1 + 1e-6)) & (ratio[mid] < 1.0))
    # linear in the index between the last kept pair (smooth 1) and the first
    # fully interpolated pair (smooth 0)
    low, high = np.nonzero(keep)[0].max(), np.nonzero(full)[0].min()
    smooth = (ratio - 1 / factor) / (1 - 1 / factor)
    i = np.arange(low, high + 1)
    assert np.allclose(smooth[i], 1 - (i - low) / (high - low), atol=1e-6)


def test_yarn_table_is_plain_table_with_yarn_frequencies():
    cos_y, sin_y = oracle.rope_table(5000, yarn=True)
    f = oracle.rope_freqs(64, yarn=True).astype(np.float64)
    p = np.arange(5000, dtype=np.float64)[:, None]
    ang = p * f[None, :]
    tol = ang * 2.0 ** -23 + 2.0 ** -23
    assert np.all(np.abs(cos_y - np.cos(ang)) <= tol)
    assert np.all(np.abs(sin_y - np.sin(ang)) <= tol)
