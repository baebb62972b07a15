"""Pins for the oracle's dispatch layout: counts, offsets, drops, positions.

Sources: aicassindra "gpu_moe_all_to_all" ("Two collectives per layer":
per-destination counts before the payload; "Bucketing": sort by destination
and build the offset table; "How to tell whether the all-to-all is your
bottleneck": the uniform round-robin router), ai-from-scratch "19.
All-to-all" ("Why the router can ruin your day": over-capacity tokens are
dropped), "MoE All-to-All Dispatch and Ragged Routing" ("Fixed Capacity vs.
Ragged Routing").
"""

import json
import os

import numpy as np
import pytest

import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _random_idx(r, T, E, k, skew=0.0):
    """k distinct experts per token, optionally skewed towards low ids."""
    p = np.exp(-skew * np.log(np.arange(1, E + 1)))
    p /= p.sum()
    return np.stack([r.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)


def _library_layout(idx, E, R, C):
    """Reference built from numpy routines: bincount, cumsum and a stable argsort."""
    T, k = idx.shape
    flat = idx.ravel()
    demand = np.bincount(flat, minlength=E)
    counts = demand if C < 0 else np.minimum(demand, C)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    order = np.argsort(flat, kind="stable")          # assignments grouped by expert, in token order
    sorted_e = flat[order]
    starts = np.concatenate([[0], np.cumsum(demand)])[:-1]
    rank = np.arange(flat.size) - starts[sorted_e]   # rank of each assignment inside its expert
    kept = np.ones_like(rank, bool) if C < 0 else rank < C
    pos = np.full(flat.size, -1, np.int64)
    pos[order[kept]] = offsets[sorted_e[kept]] + rank[kept]
    send_src = (order[kept] // k).astype(np.int32)   # kept assignments, already in send order
    el = E // R
    return dict(expert_demand=demand, expert_counts=counts, expert_offsets=offsets,
                dest_counts=counts.reshape(R, el).sum(axis=1),
                dest_offsets=offsets[::el], pos=pos.reshape(T, k), send_src=send_src)


CASES = [
    (200, 16, 2, 4, -1, 0.0),
    (200, 16, 2, 4, 20, 1.0),
    (333, 64, 8, 8, -1, 0.5),
    (333, 64, 8, 8, 30, 1.0),
    (97, 384, 8, 64, -1, 0.0),
    (500, 512, 10, 64, 12, 0.5),
    (50, 6, 6, 3, 7, 0.0),
    (10, 5, 1, 1, 0, 0.0),
    (1, 8, 3, 8, -1, 0.0),
]


@pytest.mark.parametrize("T,E,k,R,C,skew", CASES)
def test_layout_matches_library_reference(orc, T, E, k, R, C, skew):
    r = np.random.default_rng(T + E + k)
    idx = _random_idx(r, T, E, k, skew)
    got = orc.dispatch_layout(idx, E, R, C)
    ref = _library_layout(idx, E, R, C)
    for name in ("expert_demand", "expert_counts", "expert_offsets", "dest_counts", "dest_offsets", "pos"):
        np.testing.assert_array_equal(got[name], ref[name], err_msg=name)
    N = int(ref["expert_offsets"][-1])
    np.testing.assert_array_equal(got["send_src"][:N], ref["send_src"])
    assert np.all(got["send_src"][N:] == -1)


@pytest.mark.parametrize("T,E,k,R,C,skew", CASES)
def test_layout_invariants(orc, T, E, k, R, C, skew):
    r = np.random.default_rng(1 + T + E + k)
    idx = _random_idx(r, T, E, k, skew)
    L = orc.dispatch_layout(idx, E, R, C)
    demand, counts, pos = L["expert_demand"], L["expert_counts"], L["pos"]
    assert demand.sum() == T * k
    if C < 0:
        assert counts.sum() == T * k and np.all(pos >= 0)
    else:
        assert np.all(counts == np.minimum(demand, C))
        assert (pos < 0).sum() == np.maximum(demand - C, 0).sum()
    N = int(L["expert_offsets"][-1])
    assert L["dest_offsets"][-1] == N
    kept = pos[pos >= 0]
    # every send row below N is written by exactly one replica
    assert np.array_equal(np.sort(kept), np.arange(N))
    # brute force: position = expert start + earlier kept replicas of that expert
    kept_so_far = np.zeros(E, np.int64)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            if pos[t, j] >= 0:
                assert pos[t, j] == L["expert_offsets"][e] + kept_so_far[e]
                assert L["send_src"][pos[t, j]] == t
                kept_so_far[e] += 1
            else:
                # dropped only once the expert's capacity is used up, in token order
                assert C >= 0 and kept_so_far[e] == C
    # destination segments hold exactly their experts' rows
    el = E // R
    for rr in range(R):
        lo, hi = L["dest_offsets"][rr], L["dest_offsets"][rr + 1]
        seg_experts = {int(idx.ravel()[i]) for i in np.flatnonzero((pos.ravel() >= lo) & (pos.ravel() < hi))}
        assert seg_experts <= set(range(rr * el, (rr + 1) * el))


def test_round_robin_closed_form(orc):
    T, E, k, R = 96, 16, 2, 4
    idx = synthetic.round_robin_idx(T, E, k)
    L = orc.dispatch_layout(idx, E, R, -1)
    per = T * k // E
    assert np.all(L["expert_demand"] == per)
    t = np.arange(T)[:, None]
    j = np.arange(k)[None, :]
    e = (t * k + j) % E
    np.testing.assert_array_equal(L["pos"], e * per + (t * k + j) // E)
    np.testing.assert_array_equal(L["dest_counts"], np.full(R, T * k // R))


def test_capacity_closed_forms(orc):
    T, E, k, R = 50, 8, 3, 2
    idx = np.tile(np.arange(k, dtype=np.int32), (T, 1))   # what constant logits select
    for C in (0, 1, 17, 49, 50, 80):
        L = orc.dispatch_layout(idx, E, R, C)
        for t in range(T):
            assert np.all((L["pos"][t] >= 0) == (t < C))
    r = np.random.default_rng(5)
    idx = _random_idx(r, 300, E, k, 1.0)
    free = orc.dispatch_layout(idx, E, R, -1)
    big = orc.dispatch_layout(idx, E, R, int(free["expert_demand"].max()))
    for name in free:
        np.testing.assert_array_equal(free[name], big[name], err_msg=name)
    none = orc.dispatch_layout(idx, E, R, 0)
    assert np.all(none["pos"] == -1) and none["expert_offsets"][-1] == 0


def test_golden_layout(orc):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        if "pos" not in case:
            continue
        idx = np.array(case["topk_idx"], np.int32)
        L = orc.dispatch_layout(idx, case["E"], case["R"], case["capacity"])
        for name in ("expert_demand", "expert_counts", "expert_offsets", "dest_counts", "dest_offsets", "pos"):
            np.testing.assert_array_equal(L[name], np.array(case[name]), err_msg=(case["name"], name))
        N = L["expert_offsets"][-1]
        np.testing.assert_array_equal(L["send_src"][:N], np.array(case["send_src"]))


def test_layout_rejects_bad_input(orc):
    with pytest.raises(ValueError):
        orc.dispatch_layout(np.array([[0, 9]], np.int32), 8, 2, -1)
    with pytest.raises(ValueError):
        orc.dispatch_layout(np.array([[0, 1]], np.int32), 8, 3, -1)
