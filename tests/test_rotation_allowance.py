"""The allowance the GPU tests grant Hadamard-rotated codes (gpu_util.
check_rotated_codes), exercised on the CPU: it accepts the codes of a
float32 fast Walsh-Hadamard transform (any butterfly order computes the
same signed sums with different float32 roundings) and rejects a code or
scale moved by one step. The rotation is the indexer's H_128 / sqrt(128)
(page "Sparse latent attention", the rotated q and k)."""
import numpy as np
import pytest

import oracle
from gpu_util import check_rotated_codes


def fwht_f32(x, strides):
    """float32 butterflies (a + b, a - b) in the given stride order, then one
    float32 multiplication by fl32(128^-0.5)."""
    v = np.array(x, np.float32)
    for s in strides:
        idx = np.arange(128)
        lo = idx[(idx & s) == 0]
        a, b = v[:, lo].copy(), v[:, lo + s].copy()
        v[:, lo] = a + b
        v[:, lo + s] = a - b
    return v * np.float32(128 ** -0.5)


def rows(seed, n, bf16):
    x = np.random.default_rng(seed).standard_normal((n, 128)).astype(np.float32)
    x[0, :5] *= 40.0                      # a dominant block sets amax
    return oracle.round_bf16(x) if bf16 else x


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("strides", [[1, 2, 4, 8, 16, 32, 64], [64, 32, 16, 8, 4, 2, 1]])
def test_fast_transform_codes_are_accepted(bf16, pow2, strides):
    x = rows(1, 2000, bf16)
    y = fwht_f32(x, strides)
    if bf16:
        y = oracle.round_bf16(y)
    codes, scales = oracle.quantize(y, pow2=pow2)
    same_codes, same_scales = check_rotated_codes(x, codes, scales, bf16, pow2, "fwht")
    # float32 rows: the amax element's last bit often differs, so the scale
    # does too; bf16 rows rarely change
    assert same_codes > 0.99 and same_scales > (0.95 if bf16 else 0.2)


def test_moved_code_or_scale_is_rejected():
    x = rows(2, 200, True)
    y = oracle.round_bf16(fwht_f32(x, [1, 2, 4, 8, 16, 32, 64]))
    codes, scales = oracle.quantize(y)
    bad = codes.copy()
    # move one mid-range code by one step (sign bit kept; 0x30 is 1.0)
    r, c = np.argwhere((codes & 0x7F) == 0x30)[0]
    bad[r, c] += 1
    with pytest.raises(AssertionError):
        check_rotated_codes(x, bad, scales, True, False, "planted code")
    bad_s = scales.copy()
    bad_s[3] = np.nextafter(bad_s[3] * np.float32(1.01), np.float32(np.inf))
    with pytest.raises(AssertionError):
        check_rotated_codes(x, codes, bad_s, True, False, "planted scale")
    # an unrotated row is far outside the allowance
    plain, plain_s = oracle.quantize(x)
    with pytest.raises(AssertionError):
        check_rotated_codes(x, plain, plain_s, True, False, "no rotation")
