"""Pins for the oracle's receive-side regroup (source-major segments to
expert-major rows) and its inverse on the return path.

Sources: aicassindra "gpu_moe_all_to_all", "Two collectives per layer"
(per-destination counts precede the payload; outputs return along the
inverse permutation) and "Bucketing" (one contiguous message per peer);
"MoE All-to-All Dispatch and Ragged Routing", "Why MoE Token Dispatch is
All-to-All" (a GPU holds a few of the experts) and "Fixed Capacity vs.
Ragged Routing" (the receiver pools its local experts).
"""

import json
import os

import numpy as np
import pytest

import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _labels(cnt):
    """Local expert of each received row, in source-major order."""
    S, El = cnt.shape
    return np.concatenate([np.repeat(np.arange(El), cnt[s]) for s in range(S)]).astype(np.int64)


def test_golden_regroup(orc):
    case = [c for c in json.load(open(GOLDEN))["cases"] if c["name"].startswith("regroup")][0]
    out = orc.recv_regroup_layout(np.array(case["recv_counts"]))
    for name in ("local_expert_offsets", "source_offsets", "recv_pos"):
        np.testing.assert_array_equal(out[name], np.array(case[name]), err_msg=name)


@pytest.mark.parametrize("S,El,seed", [(3, 2, 0), (64, 8, 1), (8, 6, 2), (1, 5, 3), (7, 1, 4), (16, 16, 5)])
def test_regroup_matches_stable_sort(orc, S, El, seed):
    r = np.random.default_rng(seed)
    cnt = r.integers(0, 9, size=(S, El)).astype(np.int32)
    cnt[r.random((S, El)) < 0.2] = 0                     # empty blocks
    out = orc.recv_regroup_layout(cnt)
    lab = _labels(cnt)
    order = np.argsort(lab, kind="stable")               # expert-major, source order kept
    ref = np.empty_like(order)
    ref[order] = np.arange(order.size)
    np.testing.assert_array_equal(out["recv_pos"], ref)
    np.testing.assert_array_equal(out["local_expert_offsets"], np.concatenate([[0], np.cumsum(cnt.sum(0))]))
    np.testing.assert_array_equal(out["source_offsets"], np.concatenate([[0], np.cumsum(cnt.sum(1))]))
    if S == 1 or El == 1:
        np.testing.assert_array_equal(out["recv_pos"], np.arange(lab.size))
    # round trip through the grouped layout is the identity
    x = r.integers(0, 2 ** 16, size=(lab.size, 24), dtype=np.uint16)
    g = orc.scatter_rows(x, out["recv_pos"], lab.size)
    np.testing.assert_array_equal(orc.gather_rows(g, out["recv_pos"]), x)
    # each expert's block holds exactly its rows
    for l in range(El):
        lo, hi = out["local_expert_offsets"][l], out["local_expert_offsets"][l + 1]
        np.testing.assert_array_equal(g[lo:hi], x[lab == l])


def test_regroup_after_dispatch_from_several_sources(orc):
    """Simulate S source ranks with the oracle's own dispatch, exchange their
    segments for destination r, regroup, and compare each local expert's rows
    with the rows collected directly from the sources' token lists."""
    S, T, H, E, k, R = 4, 300, 16, 32, 4, 4
    El = E // R
    srcs = []
    for s in range(S):
        w = synthetic.Workload("src", T=T, H=H, E=E, k=k, R=R, skew=0.5)
        d = synthetic.make_inputs(w, seed=10 + s)
        idx, _ = orc.route_topk(d["logits"], None, k)
        L = orc.dispatch_layout(idx, E, R, 40)          # capacity: some rows dropped
        N = int(L["expert_offsets"][-1])
        srcs.append((d["x"], idx, L, orc.dispatch_permute(d["x"], L["pos"], N)))
    for r in range(R):
        cnt = np.array([L["expert_counts"][r * El:(r + 1) * El] for (_, _, L, _) in srcs], np.int32)
        recv = np.concatenate([send[L["dest_offsets"][r]:L["dest_offsets"][r + 1]] for (_, _, L, send) in srcs])
        out = orc.recv_regroup_layout(cnt)
        grouped = orc.scatter_rows(recv, out["recv_pos"], recv.shape[0])
        for l in range(El):
            e = r * El + l
            direct = [x[t] for (x, idx, L, _) in srcs for t in range(T)
                      if any(idx[t, j] == e and L["pos"][t, j] >= 0 for j in range(k))]
            lo, hi = out["local_expert_offsets"][l], out["local_expert_offsets"][l + 1]
            assert hi - lo == len(direct)
            if direct:
                np.testing.assert_array_equal(grouped[lo:hi], np.stack(direct))


def test_regroup_rejects_negative_counts(orc):
    with pytest.raises(ValueError):
        orc.recv_regroup_layout(np.array([[1, -1]]))
