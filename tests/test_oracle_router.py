"""Pins of oracle.router (the router front-end) against a hand-worked
example, a selection invariant checked by brute force, and softmax identities
computed by scipy."""

import itertools
import os

import numpy as np
import pytest
from scipy.special import softmax

from oracle import router as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "router_worked_example.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        case, what, *vals = line.split()
        out[(case, what)] = [float(v) for v in vals]
    return out


def test_worked_example():
    g = _golden()
    s = np.array([[1, 3, 2, 3]], dtype=np.float32)
    ids, w = R.topk_route(s, 2)
    assert ids[0].tolist() == g[("case1", "ids")]
    assert np.allclose(w[0], g[("case1", "weights")], rtol=0, atol=1e-15)
    ids, w = R.topk_route(s, 2, bias=np.array([0, 0, 2, -1], dtype=np.float32))
    assert ids[0].tolist() == g[("case2", "ids")]
    assert np.allclose(w[0], g[("case2", "weights")], rtol=0, atol=1e-15)
    ids, w = R.topk_route(np.zeros((1, 3), dtype=np.float32), 3)
    assert ids[0].tolist() == g[("case3", "ids")]
    assert np.allclose(w[0], g[("case3", "weights")], rtol=0, atol=1e-15)


def _is_topk(key, sel):
    """Every selected key beats every unselected one (equal keys: the lower
    index wins), and the list is in that order."""
    rest = [j for j in range(len(key)) if j not in sel]
    better = lambda a, b: key[a] > key[b] or (key[a] == key[b] and a < b)
    return (all(better(a, b) for a in sel for b in rest)
            and all(better(sel[i], sel[i + 1]) for i in range(len(sel) - 1)))


def test_selection_brute_force_small():
    """Over every k-subset (in every order) exactly one satisfies the top-k
    rule, and the oracle returns it -- on keys with many ties."""
    rng = np.random.default_rng(0)
    for trial in range(60):
        e = int(rng.integers(1, 7))
        k = int(rng.integers(1, e + 1))
        key = rng.integers(-2, 3, size=e).astype(np.float32)   # small ints: ties
        ids, _ = R.topk_route(key[None, :], k)
        winners = [p for p in itertools.permutations(range(e), k) if _is_topk(key, list(p))]
        assert winners == [tuple(ids[0].tolist())], (key, k, winners, ids)


def test_bias_steers_selection_only():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((50, 64)).astype(np.float32)
    b = rng.normal(0, np.sqrt(0.5), 64).astype(np.float32)
    ids, w = R.topk_route(s, 8, bias=b)
    key = s + b
    for i in range(50):
        assert _is_topk(key[i], ids[i].tolist())
    # the weights are the softmax of the selected raw scores (not of the keys)
    sel = np.take_along_axis(s.astype(np.float64), ids.astype(np.int64), axis=1)
    assert np.allclose(w, softmax(sel, axis=1), rtol=1e-14, atol=0)


def test_renormalised_full_softmax_identity():
    """Without bias the weights equal the renormalised top-k entries of a
    softmax over all experts (scipy), and the ids are the k most probable."""
    rng = np.random.default_rng(2)
    s = rng.standard_normal((40, 128)).astype(np.float32)
    ids, w = R.topk_route(s, 8)
    p = softmax(s.astype(np.float64), axis=1)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13, atol=0)
    assert np.all(np.min(sel, axis=1) >= np.sort(p, axis=1)[:, -8])


@pytest.mark.parametrize("shift", [-7.5, 0.25, 100.0])
def test_weights_closed_forms(shift):
    rng = np.random.default_rng(3)
    s = rng.standard_normal((20, 32)).astype(np.float32)
    ids, w = R.topk_route(s, 4)
    # ratio of two weights is exp of the score difference
    sel = np.take_along_axis(s.astype(np.float64), ids.astype(np.int64), axis=1)
    assert np.allclose(w[:, 0] / w[:, 1], np.exp(sel[:, 0] - sel[:, 1]), rtol=1e-13)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    # adding a constant to every score changes nothing when it is exact in float32
    ids2, w2 = R.topk_route(s + np.float32(shift), 4)
    if np.all((s + np.float32(shift)) - np.float32(shift) == s):
        assert np.array_equal(ids, ids2)
        assert np.allclose(w, w2, rtol=1e-12)
    # k = E: every expert, weights = the full softmax
    idsa, wa = R.topk_route(s, 32)
    full = softmax(s.astype(np.float64), axis=1)
    assert np.allclose(wa, np.take_along_axis(full, idsa.astype(np.int64), axis=1), rtol=1e-13)


def test_check_routing_hand_worked_and_brute_force():
    # hand-worked: E = 4; entries 2 (id 4) and 3 (id -1) are out of range
    assert R.check_routing(np.array([[0, 3], [4, -1]], dtype=np.int32), 4) == (2, 2)
    assert R.check_routing(np.zeros((0, 8), dtype=np.int32), 4) == (0, -1)
    # brute force over small random cases: a plain loop over the entries
    rng = np.random.default_rng(3)
    for _ in range(50):
        t, k, e = int(rng.integers(0, 6)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
        ids = rng.integers(-3, e + 3, size=(t, k)).astype(np.int32)
        cnt, first = 0, -1
        for i, v in enumerate(ids.reshape(-1).tolist()):
            if not 0 <= v < e:
                cnt += 1
                first = i if first < 0 else first
        assert R.check_routing(ids, e) == (cnt, first)
