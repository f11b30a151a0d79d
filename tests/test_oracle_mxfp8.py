"""Pins of the oracle's MXFP8 activation quantiser: the scale exponent against an
exhaustive search, codes against torch's CPU E4M3 cast, and the whole round
trip against the brute-force nearest-value search."""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import moe
from oracle.brute import mxfp8_roundtrip_brute


def _search_exponent(amax):
    e = -127
    for cand in range(-127, 128):
        if 448.0 * 2.0 ** cand <= amax:
            e = cand
    return e if amax > 0 else -127


def test_scale_exponent_boundaries():
    for j in range(-140, 120, 7):
        b = 448.0 * 2.0 ** j
        for a in (b, np.nextafter(b, 0), np.nextafter(b, np.inf), 1.3 * b, 0.9 * b):
            assert moe.mxfp8_scale_exponent(a) == _search_exponent(a), a
    assert moe.mxfp8_scale_exponent(0.0) == -127
    assert moe.mxfp8_scale_exponent(448.0) == 0
    assert moe.mxfp8_scale_exponent(447.9) == -1
    assert moe.mxfp8_scale_exponent(2.0 ** -140) == -127      # clamped below
    with pytest.raises(ValueError):
        moe.mxfp8_scale_exponent(np.inf)


def test_scale_exponent_random():
    rng = np.random.default_rng(4)
    for a in np.ldexp(rng.random(3000) + 0.5, rng.integers(-130, 130, 3000)):
        assert moe.mxfp8_scale_exponent(a) == _search_exponent(a)


def test_codes_match_torch_cast_after_scaling():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)) * 3)).astype(np.float32)
    codes, scales = moe.mxfp8_quantize(x.astype(np.float64))
    e = scales.astype(np.int64) - 127
    scaled = np.ldexp(x.astype(np.float64).reshape(64, 8, 32), -e[:, :, None]).reshape(64, 256)
    t = torch.from_numpy(np.clip(scaled, -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(codes, t.view(torch.uint8).numpy())


def test_block_max_saturates_under_the_literal_rule():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((32, 64))
    codes, scales = moe.mxfp8_quantize(x)
    vals = np.abs(F.e4m3_value(codes)).reshape(32, 2, 32)
    np.testing.assert_array_equal(vals.max(axis=2), 448.0)


def test_zero_block():
    codes, scales = moe.mxfp8_quantize(np.zeros((1, 32)))
    assert (codes == 0).all() and (scales == 0).all()
    np.testing.assert_array_equal(moe.mxfp8_dequantize(codes, scales), 0.0)


def test_roundtrip_matches_exhaustive_search():
    rng = np.random.default_rng(7)
    blocks = [rng.standard_normal(32) * s for s in (1.0, 1e-3, 37.0, 1e-30)]
    blocks.append(np.concatenate([[0.0, -0.0], rng.standard_normal(30)]))
    for b in blocks:
        got = moe.mxfp8_roundtrip(b[None, :])[0]
        want, byte = mxfp8_roundtrip_brute(list(b))
        np.testing.assert_array_equal(got, np.array(want))
        assert moe.mxfp8_quantize(b[None, :])[1][0, 0] == byte


def test_roundtrip_error_bound_below_block_max():
    # elements that do not saturate are within half an E4M3 step (2^-4 relative
    # for normals, 2^-10 * 2^e absolute for subnormals) of their input
    rng = np.random.default_rng(8)
    x = rng.standard_normal((16, 32))
    codes, scales = moe.mxfp8_quantize(x)
    dq = moe.mxfp8_dequantize(codes, scales)
    e = (scales.astype(np.int64) - 127)[:, 0:1]
    scaled = np.abs(np.ldexp(x, -e))
    ok = scaled <= 448
    err = np.abs(dq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, np.ldexp(2.0 ** -10, e))
    assert (err[ok] <= bound[ok]).all()
