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


# ---------------------------------------------------------------- admissible requantisations
def _codes_of(values_blocks, e):
    """E4M3 codes of [n, 32*nb] values at block exponents e [n, nb]."""
    n, k = values_blocks.shape
    b = values_blocks.reshape(n, k // 32, 32)
    return F.e4m3_encode(np.ldexp(b, -e[:, :, None])).reshape(n, k)


def test_requant_check_without_uncertainty_takes_only_the_quantisation_of_v():
    rng = np.random.default_rng(11)
    v = rng.normal(size=(6, 64))
    c, s = moe.mxfp8_quantize(v)
    r = moe.mxfp8_requant_check(v, 0.0, c, s)
    assert r["n_bad"] == 0 and r["n_differ"] == 0 and r["n_ambiguous"] == 0 and r["n"] == v.size
    np.testing.assert_array_equal(r["values"], moe.mxfp8_roundtrip(v))
    c2 = c.copy()
    c2[2, 7] = c2[2, 7] + 1 if (c2[2, 7] & 0x7F) < 0x7E else c2[2, 7] - 1   # one code step off
    r = moe.mxfp8_requant_check(v, 0.0, c2, s)
    assert r["n_bad"] == 1 and not r["admissible"][2, 7]
    s2 = s.copy()
    s2[4, 1] += 1                                     # another block exponent: all 32 elements wrong
    assert moe.mxfp8_requant_check(v, 0.0, c, s2)["n_bad"] == 32


def test_requant_check_at_a_rounding_midpoint_takes_either_neighbour():
    # block maximum 600 -> e = 0; 1.0625 is halfway between the codes 1.0 and
    # 1.125: an interval around it admits both, and nothing further
    v = np.array([[1.0625] + [0.5] * 30 + [600.0]])
    c, s = moe.mxfp8_quantize(v)
    assert F.e4m3_value(c[0, 0]) == 1.0
    r = moe.mxfp8_requant_check(v, 1e-9, c, s)
    assert r["n_bad"] == 0 and r["n_ambiguous"] == 1 and r["ambiguous"][0, 0] and r["n_differ"] == 0
    up = c.copy()
    up[0, 0] += 1                                     # 1.125
    r = moe.mxfp8_requant_check(v, 1e-9, up, s)
    assert r["n_bad"] == 0 and r["n_differ"] == 1 and r["values"][0, 0] == 1.125
    up[0, 0] += 1                                     # 1.25: two steps, not a correct rounding
    assert moe.mxfp8_requant_check(v, 1e-9, up, s)["n_bad"] == 1
    up = c.copy()
    up[0, 1] += 1                                     # 0.5 sits on a code: no neighbour is correct
    assert moe.mxfp8_requant_check(v, 1e-9, up, s)["n_bad"] == 1


def test_requant_check_at_a_scale_boundary_takes_either_exponent():
    # block maximum exactly 448 -> e = 0; just below it e = -1, where the
    # literal rule saturates it to 448 * 2^-1 = 224 and 3.0 is still a code
    v = np.array([[448.0] + [3.0] * 31])
    c, s = moe.mxfp8_quantize(v)
    assert s[0, 0] == 127
    r = moe.mxfp8_requant_check(v, 1e-9, c, s)
    assert r["n_bad"] == 0 and r["n_ambiguous"] == 32
    e_low = np.array([[-1]])
    c_low = _codes_of(np.nextafter(v, 0), e_low)
    r = moe.mxfp8_requant_check(v, 1e-9, c_low, np.array([[126]], np.uint8))
    assert r["n_bad"] == 0 and r["values"][0, 0] == 224.0 and r["values"][0, 1] == 3.0
    assert r["n_differ"] == 1
    # a third exponent is not reachable
    c_2 = _codes_of(v, np.array([[-2]]))
    assert moe.mxfp8_requant_check(v, 1e-9, c_2, np.array([[125]], np.uint8))["n_bad"] == 32


def test_requant_check_admits_every_quantisation_inside_the_interval_brute_force():
    """Quantise random points v' of [v - dv, v + dv] (and its ends) with the
    oracle's own quantiser: each one is admissible; a code moved by two steps
    where the element is not ambiguous is not."""
    rng = np.random.default_rng(12)
    for trial in range(40):
        v = rng.normal(size=(2, 64)) * np.ldexp(1.0, int(rng.integers(-8, 8)))
        # push some elements onto decision points: midpoints and scale boundaries
        v[0, 3] = 1.0625 * np.ldexp(1.0, moe.mxfp8_scale_exponent(np.abs(v[0, :32]).max()))
        v[1, 40] = 448.0 * np.ldexp(1.0, int(rng.integers(-6, 3)))
        dv = np.abs(v) * 10.0 ** rng.uniform(-9, -3)
        for j in range(32):
            vp = v + dv * (rng.uniform(-1, 1, size=v.shape) if j > 1 else (2 * j - 1))
            c, s = moe.mxfp8_quantize(vp)
            r = moe.mxfp8_requant_check(v, dv, c, s)
            assert r["n_bad"] == 0, (trial, j)
            assert (r["ambiguous"] | (r["values"] == r["rt"])).all()
        c, s = moe.mxfp8_quantize(v)
        r = moe.mxfp8_requant_check(v, dv, c, s)
        plain = np.argwhere(~r["ambiguous"] & (np.abs(F.e4m3_value(c)) > 1) & (np.abs(F.e4m3_value(c)) < 200))
        i, k = plain[0]
        c2 = c.copy()
        c2[i, k] += 2
        assert moe.mxfp8_requant_check(v, dv, c2, s)["n_bad"] == 1


def test_forward_with_its_own_requantisation_is_the_forward():
    import workloads as W
    case = W.make_case("hq", W.LayerShape(6, 256, 128, 3, 3, 2), 13, act="mxfp8")
    args = (case.hidden_bits, case.topk_ids, case.topk_weights, case.experts(), 3)
    acc = moe.forward(*args, act="mxfp8")
    seen = []

    def own(e, routes, h, dh):
        seen.extend(routes)
        assert (dh >= 0).all() and dh.shape == h.shape
        c, s = moe.mxfp8_quantize(h)
        r = moe.mxfp8_requant_check(h, dh, c, s)
        assert r["n_bad"] == 0 and r["n_differ"] == 0
        return r["values"]

    np.testing.assert_array_equal(moe.forward(*args, act="mxfp8", h_requant=own), acc)
    ids = case.topk_ids
    assert sorted(seen) == sorted((t, s) for t in range(6) for s in range(2) if 0 <= ids[t, s] < 3)


def _silu_f32_hw(z32):
    """silu in float32 the way a GPU evaluates it on its exponential unit:
    exp(-z) as 2^(-z * log2 e) with the argument rounded to float32, then
    1 + e, the reciprocal and the product, each rounded to float32."""
    arg = (-z32 * np.float32(np.log2(np.e))).astype(np.float32)
    with np.errstate(over="ignore"):
        e = np.exp2(arg.astype(np.float64)).astype(np.float32)
        r = (np.float32(1) / (np.float32(1) + e)).astype(np.float32)
    return (z32 * r).astype(np.float32)


@pytest.mark.parametrize("H,I,seed", [(256, 128, 1), (384, 256, 2), (7168, 256, 3), (2048, 512, 4)])
def test_h_uncertainty_covers_an_fp32_evaluation(H, I, seed):
    """g and u as float32 dot products summed in 128-element blocks (two K
    halves added at the end), silu on an emulated hardware exponential, the
    product in float32: h stays within h_uncertainty of the exact h.  MXFP4
    weights with scales 2^-7..2^3 make |g| reach the hundreds, so silu's
    exponential is exercised far into both tails."""
    import workloads as W
    rng = np.random.default_rng(seed)
    w13c, w13s, _, _ = W.gen_expert(seed, 0, H, I, 120, 130)
    w13 = F.dequant_mxfp4(w13c, w13s)
    x = moe.mxfp8_roundtrip(rng.standard_normal((24, H)))
    gu = x @ w13.T
    g, u = gu[:, :I], gu[:, I:]
    h = moe.silu(g) * u
    dh = moe.h_uncertainty(x, w13, g, u, h)
    assert np.abs(g).max() > 80
    x32, w32 = x.astype(np.float32), w13.astype(np.float32)
    half = (H // 128 + 1) // 2 * 128
    parts = []
    for lo, hi in ((0, half), (half, H)):
        acc = np.zeros((24, 2 * I), np.float32)
        for b in range(lo, hi, 128):
            acc = (acc + (x32[:, b:b + 128].astype(np.float64) @ w32[:, b:b + 128].T.astype(np.float64))
                   .astype(np.float32)).astype(np.float32)
        parts.append(acc)
    gu32 = (parts[0] + parts[1]).astype(np.float32)
    h32 = (_silu_f32_hw(gu32[:, :I]) * gu32[:, I:]).astype(np.float32)
    err = np.abs(h32.astype(np.float64) - h)
    assert (err <= dh).all(), float((err / np.maximum(dh, 1e-300)).max())
    # the bound is tight enough to leave most requantisation decisions unique
    c, sc = moe.mxfp8_quantize(h)
    assert moe.mxfp8_requant_check(h, dh, c, sc)["n_ambiguous"] < 0.05 * h.size


def test_silu_prime_and_its_critical_points():
    """silu' against a central difference of silu; its extrema sit at
    +-SILU_PRIME_CRIT (a dense grid finds no larger |silu'| anywhere else)."""
    z = np.linspace(-60, 60, 240001)
    dz = 1e-6
    np.testing.assert_allclose(moe.silu_prime(z), (moe.silu(z + dz) - moe.silu(z - dz)) / (2 * dz), atol=1e-8)
    c = moe.SILU_PRIME_CRIT
    assert abs(c - 2.3994) < 1e-4
    d = moe.silu_prime(z)
    inner = np.argmax(d)
    assert abs(z[inner] - c) < 1e-3 and abs(z[np.argmin(d)] + c) < 1e-3
    assert d.max() <= moe.silu_prime(c) + 1e-15 and d.min() >= moe.silu_prime(-c) - 1e-15


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


def test_quantum_is_the_e4m3_grid_spacing():
    """mxfp8_quantum against the distance between neighbouring E4M3 values of
    every code at exponent 0 (block maximum 448 fixes e = 0)."""
    vals = np.array([F.e4m3_value(c) for c in range(0, 0x7F)])
    for c in range(0, 0x7E):
        v = np.zeros((1, 32))
        v[0, 0] = 448.0
        v[0, 1] = vals[c]
        assert moe.mxfp8_quantum(v)[0, 1] == vals[c + 1] - vals[c], c
    # a value one quantum away from a code always quantises to that code or a neighbour
    rng = np.random.default_rng(16)
    v = rng.normal(size=(8, 64)) * 3
    c, s = moe.mxfp8_quantize(v)
    r = moe.mxfp8_requant_check(v, moe.mxfp8_quantum(v), c, s)
    assert r["n_bad"] == 0 and r["n_ambiguous"] > 0.9 * v.size
