"""Pins of the oracle's router top-k: a hand-worked example with ties, the two
formulations against each other, closed forms and invariances of the weights."""
import math

import numpy as np

from oracle.router import router_topk, router_topk_np


def test_hand_example_with_ties_and_nan():
    lg = np.array([[0.5, 2.0, -1.0, 2.0, np.nan, 0.5, 3.0, -np.inf]], np.float32)
    ids, w = router_topk(lg, 5)
    # 3.0 (id 6), then the tie 2.0 at ids 1 and 3 (lower id first), then 0.5 at ids 0 and 5
    assert ids.tolist() == [[6, 1, 3, 0, 5]]
    e = [1.0, math.exp(-1.0), math.exp(-1.0), math.exp(-2.5), math.exp(-2.5)]
    s = sum(e)
    np.testing.assert_allclose(w[0], [v / s for v in e], rtol=0, atol=1e-15)
    # NaN and -inf both count as -inf: the lower id (4) first, and both weigh 0;
    # the six finite logits (the five above and -1.0 at id 2) share the weight
    ids8, w8 = router_topk(lg, 8)
    assert ids8[0].tolist() == [6, 1, 3, 0, 5, 2, 4, 7]
    assert w8[0, 6] == 0.0 and w8[0, 7] == 0.0
    e6 = e + [math.exp(-4.0)]
    np.testing.assert_allclose(w8[0, :6], [v / sum(e6) for v in e6], rtol=0, atol=1e-15)
    np.testing.assert_allclose(router_topk_np(lg, 8)[1], w8, rtol=1e-13, atol=0)


def test_two_formulations_agree():
    rng = np.random.default_rng(21)
    for e_all, k in ((224, 8), (896, 16), (33, 33), (5, 1)):
        lg = rng.standard_normal((7, e_all)).astype(np.float32)
        lg[:, ::7] = np.round(lg[:, ::7] * 4) / 4        # plenty of exact ties
        a_ids, a_w = router_topk(lg, k)
        b_ids, b_w = router_topk_np(lg, k)
        np.testing.assert_array_equal(a_ids, b_ids)
        np.testing.assert_allclose(a_w, b_w, rtol=1e-13, atol=0)


def test_weights_closed_forms_and_invariances():
    rng = np.random.default_rng(22)
    lg = rng.standard_normal((5, 64)).astype(np.float32)
    ids, w = router_topk(lg, 6)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert (np.diff(w, axis=1) <= 0).all()               # descending logits give descending weights
    # two selected logits differing by d have weights in the ratio exp(d)
    sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(w[:, 0] / w[:, 1], np.exp(sel[:, 0] - sel[:, 1]), rtol=1e-13)
    # shifting every logit by 4 changes neither ids nor weights (logits on a 2^-10
    # grid below 8 in magnitude, so the shift is exact in fp32)
    lq = (np.round(lg * 1024) / 1024).astype(np.float32)
    idq, wq = router_topk(lq, 6)
    ids2, w2 = router_topk(lq + np.float32(4.0), 6)
    np.testing.assert_array_equal(idq, ids2)
    np.testing.assert_allclose(wq, w2, rtol=1e-12)
    # k = 1: the argmax with weight exactly 1
    ids1, w1 = router_topk(lg, 1)
    np.testing.assert_array_equal(ids1[:, 0], np.argmax(lg, axis=1))
    assert (w1 == 1.0).all()
