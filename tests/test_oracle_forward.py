"""Pins of the oracle forward: brute force on the tiny configuration, the
dense SwiGLU special case against torch float64, and exact invariants."""
import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from oracle.brute import forward_brute
import workloads as W


@pytest.fixture(scope="module")
def tiny():
    case = W.config_case(0)
    return case, case.experts()


def test_tiny_vs_brute_force(tiny):
    case, ew = tiny
    ref = oracle.forward(case.hidden_bits, case.topk_ids, case.topk_weights, ew, case.shape.experts)
    brute = np.array(forward_brute(case.hidden_bits, case.topk_ids, case.topk_weights, *ew,
                                   experts=case.shape.experts))
    np.testing.assert_allclose(ref, brute, rtol=1e-12, atol=1e-12 * np.abs(brute).max())


def test_tiny_mxfp8_vs_brute_force():
    shape = W.LayerShape(3, 64, 64, 4, 4, 2)
    case = W.make_case("mx", shape, 77, routing="softmax_topk", act="mxfp8")
    ew = case.experts()
    ref = oracle.forward(case.hidden_bits, case.topk_ids, case.topk_weights, ew, 4, act="mxfp8")
    brute = np.array(forward_brute(case.hidden_bits, case.topk_ids, case.topk_weights, *ew,
                                   experts=4, act="mxfp8"))
    # an h element next to an E4M3 rounding boundary could round differently
    # if the two summation orders straddle it; none does on this seed
    np.testing.assert_allclose(ref, brute, rtol=1e-9, atol=1e-9 * np.abs(brute).max())


def test_dense_swiglu_special_case():
    shape = W.LayerShape(5, 128, 64, 1, 1, 1)
    case = W.make_case("dense", shape, 11)
    ids = np.zeros((5, 1), np.int32)
    w = np.ones((5, 1), np.float32)
    w13c, w13s, w2c, w2s = case.expert(0)
    got = oracle.forward(case.hidden_bits, ids, w, (w13c[None], w13s[None], w2c[None], w2s[None]), 1)
    x = torch.from_numpy(case.hidden_bits.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    w13 = torch.from_numpy(F.dequant_mxfp4(w13c, w13s))
    w2 = torch.from_numpy(F.dequant_mxfp4(w2c, w2s))
    gate, up = w13[:64], w13[64:]
    want = torch.nn.functional.linear(torch.nn.functional.silu(x @ gate.T) * (x @ up.T), w2)
    np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12 * float(want.abs().max()))


def _fwd(case, ids=None, w=None, ew=None, **kw):
    return oracle.forward(case.hidden_bits, case.topk_ids if ids is None else ids,
                          case.topk_weights if w is None else w, ew, case.shape.experts, **kw)


@pytest.fixture(scope="module")
def mid():
    shape = W.LayerShape(24, 256, 128, 6, 9, 3)
    case = W.make_case("mid", shape, 21, routing="uniform")
    return case, case.experts()


def test_zero_weight_route_changes_nothing(mid):
    case, ew = mid
    ids = case.topk_ids.copy()
    w = case.topk_weights.copy()
    t, s = np.argwhere(ids < 6)[3]
    w0 = w.copy(); w0[t, s] = 0.0
    ids_inv = ids.copy(); ids_inv[t, s] = -1
    np.testing.assert_array_equal(_fwd(case, ids, w0, ew), _fwd(case, ids_inv, w, ew))


def test_invalid_route_weight_is_ignored(mid):
    case, ew = mid
    ids = case.topk_ids.copy()
    ids[0, 0] = -1
    ids[1, 1] = 6              # not resident
    w1 = case.topk_weights.copy(); w1[0, 0] = np.nan; w1[1, 1] = np.inf
    w2 = case.topk_weights.copy(); w2[0, 0] = 0.25; w2[1, 1] = -3.0
    a = _fwd(case, ids, w1, ew)
    assert np.isfinite(a).all()
    np.testing.assert_array_equal(a, _fwd(case, ids, w2, ew))


def test_expert_relabelling_changes_nothing(mid):
    case, ew = mid
    E = case.shape.experts
    p = np.random.default_rng(0).permutation(E)          # new storage slot of expert e is p[e]
    inv = np.argsort(p)
    ew2 = tuple(a[inv] for a in ew)                       # slot p[e] holds old expert e
    ids2 = case.topk_ids.copy()
    m = (ids2 >= 0) & (ids2 < E)
    ids2[m] = p[ids2[m]]
    np.testing.assert_allclose(_fwd(case, ids2, None, ew2), _fwd(case, None, None, ew), rtol=1e-12, atol=0)


def test_token_permutation_permutes_rows(mid):
    case, ew = mid
    p = np.random.default_rng(1).permutation(case.shape.tokens)
    ref = _fwd(case, None, None, ew)
    perm_case = W.Case("p", case.shape, case.seed, case.hidden_bits[p], case.topk_ids[p],
                       case.topk_weights[p], case.scale_lo, case.scale_hi)
    np.testing.assert_allclose(_fwd(perm_case, None, None, ew), ref[p], rtol=1e-12, atol=1e-300)


def test_token_subset_matches_full(mid):
    case, ew = mid
    full = _fwd(case, None, None, ew)
    sub = [7, 0, 23, 7]
    np.testing.assert_allclose(_fwd(case, None, None, ew, tokens=sub), full[sub], rtol=1e-12, atol=1e-300)


def test_weights_times_two_doubles_exactly(mid):
    case, ew = mid
    np.testing.assert_array_equal(_fwd(case, None, case.topk_weights * 2, ew), 2 * _fwd(case, None, None, ew))


def test_w2_scale_plus_one_doubles_exactly(mid):
    case, ew = mid
    w13c, w13s, w2c, w2s = ew
    np.testing.assert_array_equal(_fwd(case, None, None, (w13c, w13s, w2c, w2s + 1)),
                                  2 * _fwd(case, None, None, ew))


def test_up_scale_plus_one_doubles_but_gate_does_not(mid):
    case, ew = mid
    w13c, w13s, w2c, w2s = ew
    inter = case.shape.inter
    up = w13s.copy(); up[:, inter:] += 1
    gate = w13s.copy(); gate[:, :inter] += 1
    ref = _fwd(case, None, None, ew)
    np.testing.assert_array_equal(_fwd(case, None, None, (w13c, up, w2c, w2s)), 2 * ref)
    assert not np.array_equal(_fwd(case, None, None, (w13c, gate, w2c, w2s)), 2 * ref)


def test_tokens_without_valid_route_are_positive_zero(mid):
    case, ew = mid
    ids = case.topk_ids.copy()
    ids[4, :] = -1
    out = _fwd(case, ids, None, ew)
    assert (out[4] == 0).all() and not np.signbit(out[4]).any()


def test_negative_control_swapped_nibbles(tiny):
    case, ew = tiny
    w13c, w13s, w2c, w2s = ew
    swap = lambda c: ((c >> 4) | (c << 4)).astype(np.uint8)
    ref = oracle.forward(case.hidden_bits, case.topk_ids, case.topk_weights, ew, 8)
    bad = oracle.forward(case.hidden_bits, case.topk_ids, case.topk_weights,
                         (swap(w13c), w13s, swap(w2c), w2s), 8)
    assert oracle.rel_l2(bad, ref) > 0.5
    assert not oracle.check_rows(bad, ref)["pass"]


def test_single_flipped_code_is_detected(tiny):
    case, ew = tiny
    w13c, w13s, w2c, w2s = (a.copy() for a in ew)
    e = int(case.topk_ids[0, 0])
    ref = oracle.forward(case.hidden_bits, case.topk_ids, case.topk_weights, ew, 8)
    w2c[e, 5, 3] ^= 0x04
    bad = oracle.forward(case.hidden_bits, case.topk_ids, case.topk_weights, (w13c, w13s, w2c, w2s), 8)
    assert not np.array_equal(bad, ref)
