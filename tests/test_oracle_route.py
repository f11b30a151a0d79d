"""Pins of the oracle's route metadata: two independent formulations agree,
a worked example by hand, and the invariants of a stable per-expert sort."""
import numpy as np
import pytest

from oracle.route import route_sort, route_sort_by_key
import workloads as W


def _check_invariants(ids, experts, counts, offsets, perm, rowpos):
    flat = ids.reshape(-1)
    valid = [f for f in range(flat.size) if 0 <= flat[f] < experts]
    assert counts.sum() == len(valid) == offsets[-1] == perm.size
    assert offsets[0] == 0 and (np.diff(offsets) == counts).all()
    assert sorted(perm.tolist()) == valid
    for e in range(experts):
        seg = perm[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all()
        assert (np.diff(seg) > 0).all()
    for pos, f in enumerate(perm):
        assert rowpos[f] == pos
    inval = [f for f in range(flat.size) if not (0 <= flat[f] < experts)]
    assert (rowpos[inval] == -1).all()


def test_worked_example():
    ids = np.array([[2, 0], [0, -1], [5, 2]], np.int32)
    counts, offsets, perm, rowpos = route_sort(ids, 3)
    np.testing.assert_array_equal(counts, [2, 0, 2])
    np.testing.assert_array_equal(offsets, [0, 2, 2, 4])
    np.testing.assert_array_equal(perm, [1, 2, 0, 5])
    np.testing.assert_array_equal(rowpos, [2, 0, 1, -1, -1, 3])


@pytest.mark.parametrize("seed,tokens,k,experts,eglob,bad", [
    (0, 16, 2, 8, 8, 0.0), (1, 37, 8, 16, 24, 0.05), (2, 128, 8, 224, 384, 0.0),
    (3, 1, 8, 224, 384, 0.0), (4, 300, 4, 7, 7, 0.2), (5, 0, 8, 8, 8, 0.0)])
def test_two_formulations_agree(seed, tokens, k, experts, eglob, bad):
    ids, _ = W.gen_routes(seed, tokens, k, experts, eglob, "uniform", invalid_frac=bad)
    a = route_sort(ids, experts)
    b = route_sort_by_key(ids, experts)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    _check_invariants(ids, experts, *a)


def test_duplicates_and_all_invalid():
    ids = np.array([[1, 1, 1], [1, 0, 1]], np.int32)
    c, o, p, r = route_sort(ids, 2)
    np.testing.assert_array_equal(p, [4, 0, 1, 2, 3, 5])
    _check_invariants(ids, 2, c, o, p, r)
    ids = np.full((3, 2), -1, np.int32)
    c, o, p, r = route_sort(ids, 4)
    assert p.size == 0 and (r == -1).all() and (o == 0).all()


def test_zipf_routing_is_skewed_and_distinct():
    ids, w = W.gen_routes(3000, 4096, 8, 224, 384, "zipf", invalid_frac=0.01)
    valid = ids[(ids >= 0) & (ids < 224)]
    share = np.bincount(valid, minlength=224) / valid.size
    assert share.max() > 0.10                     # a hot expert above 10 % of rows
    for row in ids:
        v = row[(row >= 0) & (row < 224)]
        assert len(set(v.tolist())) == v.size     # distinct within a token
    assert abs((ids.size - valid.size) / ids.size - 0.01) < 1e-3
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-6)
    counts, offsets, perm, rowpos = route_sort(ids, 224)
    _check_invariants(ids, 224, counts, offsets, perm, rowpos)
