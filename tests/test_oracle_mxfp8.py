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


# ---------------------------------------------------------------- round-trip spread
def test_spread_zero_without_uncertainty_and_far_from_decisions():
    rng = np.random.default_rng(11)
    v = rng.normal(size=(6, 64))
    rt, sp = moe.mxfp8_roundtrip_spread(v, 0.0)
    np.testing.assert_array_equal(rt, moe.mxfp8_roundtrip(v))
    assert not sp.any()
    # grid points of E4M3 under scale 2^0 with the block maximum at 500 (e = 0):
    # every element sits on a code, a hair of uncertainty changes nothing
    grid = np.array([F.e4m3_value(c) for c in range(1, 120)])
    v = np.concatenate([grid[:31], [500.0]])[None, :]
    rt, sp = moe.mxfp8_roundtrip_spread(v, 1e-12)
    assert not sp[0, :31].any()


def test_spread_at_a_rounding_midpoint_is_one_code_step():
    # block maximum 600 -> e = 0; 1.0625 is halfway between the codes 1.0 and
    # 1.125: round-to-nearest-even gives 1.0, an upward nudge gives 1.125
    v = np.array([[1.0625] + [0.5] * 30 + [600.0]])
    rt, sp = moe.mxfp8_roundtrip_spread(v, 1e-9)
    assert rt[0, 0] == 1.0 and sp[0, 0] == 0.125
    assert sp[0, 1] == 0.0


def test_spread_at_a_scale_boundary_covers_the_halved_block_max():
    # block maximum exactly 448 -> e = 0 and it is exact; just below, e = -1 and
    # the literal rule saturates it to 448 * 2^-1 = 224
    v = np.array([[448.0] + [3.0] * 31])
    rt, sp = moe.mxfp8_roundtrip_spread(v, 1e-9)
    assert rt[0, 0] == 448.0 and sp[0, 0] == 224.0
    below = moe.mxfp8_roundtrip(np.array([[np.nextafter(448.0, 0)] + [3.0] * 31]))
    assert below[0, 0] == 224.0
    assert sp[0, 1] == 0.0          # 3.0 is a code at both exponents


def test_spread_bounds_every_perturbation_brute_force():
    rng = np.random.default_rng(12)
    for trial in range(40):
        v = rng.normal(size=(2, 64)) * np.ldexp(1.0, int(rng.integers(-8, 8)))
        # push some elements onto decision points: midpoints and scale boundaries
        v[0, 3] = 1.0625 * np.ldexp(1.0, moe.mxfp8_scale_exponent(np.abs(v[0, :32]).max()))
        v[1, 40] = 448.0 * np.ldexp(1.0, int(rng.integers(-6, 3)))
        dv = np.abs(v) * 10.0 ** rng.uniform(-9, -3)
        rt, sp = moe.mxfp8_roundtrip_spread(v, dv)
        for _ in range(30):
            vp = v + dv * rng.uniform(-1, 1, size=v.shape)
            assert (np.abs(moe.mxfp8_roundtrip(vp) - rt) <= sp).all()
        for sign in (-1.0, 1.0):     # the interval's ends
            assert (np.abs(moe.mxfp8_roundtrip(v + sign * dv) - rt) <= sp).all()


def test_forward_spread_zero_for_bf16_and_acc_unchanged():
    import workloads as W
    for act in ("bf16", "mxfp8"):
        case = W.make_case("sp", W.LayerShape(6, 256, 128, 3, 3, 2), 13, act=act)
        args = (case.hidden_bits, case.topk_ids, case.topk_weights, case.experts(), 3)
        acc = moe.forward(*args, act=act)
        acc2, bound = moe.forward(*args, act=act, with_spread=True)
        np.testing.assert_array_equal(acc, acc2)
        assert (bound >= 0).all()
        if act == "bf16":
            assert not bound.any()


def test_fp32_dot_bound_covers_fp32_evaluation():
    # a float32 evaluation of random dot products in 128-element blocks stays
    # inside the bound the spread uses for h's producers
    rng = np.random.default_rng(14)
    for k in (128, 512, 2048):
        x = rng.normal(size=(64, k)).astype(np.float32)
        w = rng.normal(size=(k, 8)).astype(np.float32)
        exact = x.astype(np.float64) @ w.astype(np.float64)
        acc = np.zeros((64, 8), np.float32)
        for b in range(0, k, 128):
            acc = (acc + x[:, b:b + 128] @ w[b:b + 128]).astype(np.float32)
        absum = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64))
        assert (np.abs(acc - exact) <= moe.fp32_dot_bound(k) * absum).all()
