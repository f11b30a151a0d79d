"""Pins of the acceptance rule: constructed outputs with known ULP and relative
L2 errors land on the right side of both bounds."""
import numpy as np

from oracle import check_rows, ulp_bf16, rel_l2


def test_exact_and_half_ulp_pass():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((4, 64))
    assert check_rows(ref, ref)["pass"]
    assert check_rows(ref + 0.5 * ulp_bf16(ref), ref)["pass"]


def test_three_ulp_passes_four_ulp_alone_fails():
    ref = np.full((1, 1000), 1.0)
    out = ref.copy()
    out[0, 0] += 3 * 2.0 ** -7
    assert check_rows(out, ref)["pass"]
    # 4 ULP on one element: fails the ULP bound but the row L2 is tiny -> pass
    out[0, 0] = 1.0 + 4 * 2.0 ** -7
    r = check_rows(out, ref)
    assert r["pass"] and r["max_ulp"] == 4.0
    # 4 ULP on every element: rel L2 = 4 * 2^-7 = 0.03 > 4e-3 -> fail
    out = ref + 4 * 2.0 ** -7
    assert not check_rows(out, ref)["pass"]


def test_rel_l2_bound():
    rng = np.random.default_rng(1)
    ref = rng.standard_normal((2, 4096))
    noise = rng.standard_normal((2, 4096))
    noise /= np.linalg.norm(noise, axis=1, keepdims=True)
    ok = ref + 3.9e-3 * np.linalg.norm(ref, axis=1, keepdims=True) * noise
    bad = ref + 4.1e-3 * np.linalg.norm(ref, axis=1, keepdims=True) * noise
    assert check_rows(ok, ref)["pass"]
    assert not check_rows(bad, ref)["pass"]
    assert abs(rel_l2(ok[0], ref[0]) - 3.9e-3) < 1e-12


def test_nonfinite_fails_and_zero_rows_exact():
    ref = np.ones((2, 8))
    out = ref.copy()
    out[1, 3] = np.nan
    r = check_rows(out, ref)
    assert not r["pass"] and r["failing_rows"] == [1]
    ref = np.zeros((1, 8))
    assert check_rows(np.zeros((1, 8)), ref)["pass"]
    assert not check_rows(np.full((1, 8), 1e-30), ref)["pass"]
