"""Pins for the oracle's top-k selection and gate weights.

Each test checks the oracle against something other than itself: brute-force
enumeration, numpy/scipy library routines, closed forms and hand-worked cases.
Sources: ai-from-scratch "19. All-to-all" (intro: a list of expert ids per
token; "Why the router can ruin your day": selection-only bias), aicassindra
"gpu_moe_all_to_all" ("Two collectives per layer": gate weights at combine).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _rank_tuple(v, e):
    # larger is better: numbers above every NaN, then value, then lower id
    if math.isnan(v):
        return (0, 0.0, -e)
    return (1, v, -e)


def _brute_force_topk(s, k):
    """Enumerate every ordered k-tuple of distinct experts and keep the
    lexicographically best sequence of ranks; that tuple takes the best
    expert first, then the best of the rest, and so on."""
    E = len(s)
    best = None
    best_key = None
    for tup in itertools.permutations(range(E), k):
        key = tuple(_rank_tuple(float(s[e]), e) for e in tup)
        if best_key is None or key > best_key:
            best, best_key = tup, key
    return list(best)


VALUES = np.array([0.0, -0.0, 1.0, -1.0, 0.5, np.inf, -np.inf, np.nan, 2.0, 1.0], np.float32)


@pytest.mark.parametrize("seed", range(40))
def test_selection_brute_force(orc, seed):
    r = np.random.default_rng(seed)
    T = int(r.integers(1, 6))
    E = int(r.integers(1, 7))
    k = int(r.integers(1, min(E, 3) + 1))
    # values drawn from a small set so that ties, signed zeros, infinities
    # and NaNs all occur
    logits = r.choice(VALUES, size=(T, E)).astype(np.float32)
    bias = r.choice(np.array([0.0, 0.5, -0.5, 1.0], np.float32), size=E) if seed % 2 else None
    idx, _ = orc.route_topk(logits, bias, k)
    for t in range(T):
        s = logits[t] if bias is None else (logits[t] + bias).astype(np.float32)
        assert list(idx[t]) == _brute_force_topk(s, k), (logits[t], bias, k)


@pytest.mark.parametrize("T,E,k", [(64, 16, 2), (33, 256, 8), (17, 384, 8), (9, 512, 10), (5, 64, 64)])
def test_selection_matches_stable_argsort(orc, T, E, k):
    r = np.random.default_rng(T * 1000 + E)
    logits = r.standard_normal((T, E), dtype=np.float32)
    # plant exact ties and a NaN
    logits[:, E // 2] = logits[:, 0]
    logits[0, 1] = np.nan
    bias = r.uniform(-0.1, 0.1, E).astype(np.float32)
    idx, _ = orc.route_topk(logits, bias, k)
    s = logits + bias                       # float32 add, as the selection rule states
    ref = np.argsort(-s, axis=1, kind="stable")[:, :k]   # NaN sorts last
    np.testing.assert_array_equal(idx, ref)


def test_selection_closed_forms(orc):
    T, E, k = 7, 12, 4
    idx, w = orc.route_topk(np.zeros((T, E), np.float32), None, k)
    np.testing.assert_array_equal(idx, np.tile(np.arange(k), (T, 1)))
    assert np.all(w == 1.0 / k)          # exp(0) = 1 and the sum is k, exactly
    # a large bias on a set S forces the selection to S
    S = [9, 2, 5, 11]
    bias = np.zeros(E, np.float32)
    bias[S] = 1e4
    logits = np.random.default_rng(1).standard_normal((T, E), dtype=np.float32)
    idx, _ = orc.route_topk(logits, bias, k)
    for t in range(T):
        assert sorted(idx[t]) == sorted(S)
    # k = E gives a full ordering of all experts
    idx, w = orc.route_topk(logits, None, E)
    for t in range(T):
        assert sorted(idx[t]) == list(range(E))
        assert np.all(np.diff(logits[t][idx[t]]) <= 0)


@pytest.mark.parametrize("normalize", [True, False])
def test_weights_match_scipy_softmax(orc, normalize):
    r = np.random.default_rng(7)
    T, E, k = 50, 64, 6
    logits = (3 * r.standard_normal((T, E))).astype(np.float32)
    bias = r.uniform(-1, 1, E).astype(np.float32)
    idx, w = orc.route_topk(logits, bias, k, normalize=normalize)
    l64 = logits.astype(np.float64)
    for t in range(T):
        if normalize:
            ref = scipy.special.softmax(l64[t][idx[t]])
        else:
            ref = scipy.special.softmax(l64[t])[idx[t]]
        np.testing.assert_allclose(w[t], ref, rtol=1e-13, atol=0)
    if normalize:
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)


def test_bias_is_selection_only(orc):
    r = np.random.default_rng(3)
    T, E, k = 40, 32, 4
    logits = r.standard_normal((T, E), dtype=np.float32)
    idx0, w0 = orc.route_topk(logits, None, k)
    # a bias that keeps the ranking (tiny, positive on the selected set)
    # must leave the weights bitwise unchanged
    for t in range(T):
        bias = np.zeros(E, np.float32)
        bias[idx0[t]] = np.float32(1e-3)
        idx1, w1 = orc.route_topk(logits[t:t + 1], bias, k)
        s = logits[t] + bias
        if list(np.argsort(-s, kind="stable")[:k]) == list(idx0[t]):
            np.testing.assert_array_equal(idx1[0], idx0[t])
            assert np.array_equal(w1[0], w0[t])
    # a bias that changes the selection: weights follow the unbiased logits
    bias = np.zeros(E, np.float32)
    bias[E - 1] = 100.0
    idx2, w2 = orc.route_topk(logits, bias, k)
    assert np.all(idx2[:, 0] == E - 1)
    for t in range(T):
        ref = scipy.special.softmax(logits[t].astype(np.float64)[idx2[t]])
        np.testing.assert_allclose(w2[t], ref, rtol=1e-13)


def test_golden_route(orc):
    for case in _golden():
        if "logits" not in case:
            continue
        logits = np.array(case["logits"], np.float32)
        bias = None if case["bias"] is None else np.array(case["bias"], np.float32)
        idx, w = orc.route_topk(logits, bias, case["k"])
        np.testing.assert_array_equal(idx, np.array(case["topk_idx"]))
        if "topk_w" in case:
            np.testing.assert_allclose(w, np.array(case["topk_w"]), rtol=1e-15, atol=1e-17)


def test_route_rejects_bad_sizes(orc):
    with pytest.raises(ValueError):
        orc.route_topk(np.zeros((2, 3), np.float32), None, 4)


# ---------------------------------------------------------------------------
# group-limited routing (ai-from-scratch "19. All-to-all", "DeepSeek's
# numbers": at most 4 nodes per token)
# ---------------------------------------------------------------------------

def _sort_key(v, e):
    # ascending sort key of the selection order: numbers before NaN, larger
    # first, then lower id
    return (1, 0.0, e) if math.isnan(v) else (0, -v, e)


def _grouped_by_sorting(s, k, G, M):
    """Reformulation with Python's sort: order groups by their best member,
    keep M, order the allowed experts, keep k."""
    E = len(s)
    gs = E // G
    best = [min(range(g * gs, (g + 1) * gs), key=lambda e: _sort_key(float(s[e]), e)) for g in range(G)]
    groups = sorted(range(G), key=lambda g: _sort_key(float(s[best[g]]), best[g]))[:M]
    allowed = [e for e in range(E) if e // gs in groups]
    return sorted(allowed, key=lambda e: _sort_key(float(s[e]), e))[:k]


@pytest.mark.parametrize("seed", range(30))
def test_grouped_brute_force(orc, seed):
    r = np.random.default_rng(100 + seed)
    E = int(r.choice([4, 6, 8]))
    G = int(r.choice([d for d in (1, 2, 3, 4, 8) if E % d == 0]))
    M = int(r.integers(1, G + 1))
    k = int(r.integers(1, min(M * (E // G), 3) + 1))
    T = 4
    logits = r.choice(VALUES, size=(T, E)).astype(np.float32)
    bias = r.choice(np.array([0.0, 0.5, -0.5], np.float32), size=E) if seed % 2 else None
    idx, _ = orc.route_topk_grouped(logits, bias, k, G, M)
    for t in range(T):
        s = logits[t] if bias is None else (logits[t] + bias).astype(np.float32)
        assert list(idx[t]) == _grouped_by_sorting(s, k, G, M), (logits[t], bias, k, G, M)


@pytest.mark.parametrize("T,E,k,G,M", [(64, 64, 4, 8, 2), (50, 512, 10, 8, 4), (33, 256, 8, 16, 3), (20, 384, 8, 64, 8)])
def test_grouped_matches_numpy(orc, T, E, k, G, M):
    r = np.random.default_rng(E + G)
    logits = r.standard_normal((T, E), dtype=np.float32)
    bias = r.uniform(-0.1, 0.1, E).astype(np.float32)
    idx, w = orc.route_topk_grouped(logits, bias, k, G, M)
    s = (logits + bias).astype(np.float32)                     # distinct finite scores
    gmax = s.reshape(T, G, E // G).max(axis=2)
    top_groups = np.argsort(-gmax, axis=1, kind="stable")[:, :M]
    allowed = np.zeros((T, G), bool)
    np.put_along_axis(allowed, top_groups, True, axis=1)
    masked = np.where(np.repeat(allowed, E // G, axis=1), s, -np.inf)
    ref = np.argsort(-masked, axis=1, kind="stable")[:, :k]
    np.testing.assert_array_equal(idx, ref)
    assert all(len(set(row // (E // G))) <= M for row in idx)
    for t in range(T):
        ref_w = scipy.special.softmax(logits[t].astype(np.float64)[idx[t]])
        np.testing.assert_allclose(w[t], ref_w, rtol=1e-13)


def test_grouped_reduces_to_plain(orc):
    r = np.random.default_rng(8)
    T, E, k = 40, 64, 6
    logits = r.choice(VALUES, size=(T, E)).astype(np.float32)
    bias = r.uniform(-1, 1, E).astype(np.float32)
    plain = orc.route_topk(logits, bias, k)
    for G in (1, 4, 16):                  # every group allowed
        got = orc.route_topk_grouped(logits, bias, k, G, G)
        np.testing.assert_array_equal(got[0], plain[0])
        np.testing.assert_array_equal(got[1], plain[1])
    got = orc.route_topk_grouped(logits, bias, k, E, k)   # one expert per group
    np.testing.assert_array_equal(got[0], plain[0])


def test_grouped_rejects_bad_sizes(orc):
    z = np.zeros((2, 12), np.float32)
    for k, G, M in ((2, 5, 1), (2, 4, 5), (4, 4, 1), (2, 4, 0)):
        with pytest.raises(ValueError):
            orc.route_topk_grouped(z, None, k, G, M)
