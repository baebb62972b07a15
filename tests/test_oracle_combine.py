"""Pins for the oracle's permute, combine and bf16 rounding.

Sources: aicassindra "gpu_moe_all_to_all" ("Two collectives per layer":
outputs return along the inverse permutation and are scaled by the gate
weights), "MoE All-to-All Dispatch and Ragged Routing" ("Returning Tokens
to the Original GPU": residual x + dx at the origin), ai-from-scratch "19.
All-to-all" (a dropped token counts as having skipped that expert; the shared
expert is always active).
"""

import json
import os

import numpy as np
import pytest
import torch

import synthetic
from tolerance import assert_bf16_close

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _bits(vals):
    return synthetic.bf16_bits_from_f32(np.asarray(vals, np.float32))


def _pipeline(orc, w, seed=0, capacity=None, shared=None):
    d = synthetic.make_inputs(w, seed)
    C = w.capacity if capacity is None else capacity
    idx, wt = orc.route_topk(d["logits"], d["bias"], w.k)
    L = orc.dispatch_layout(idx, w.E, w.R, C)
    N = int(L["expert_offsets"][-1])
    send = orc.dispatch_permute(d["x"], L["pos"], max(N, 1))
    return d, idx, wt, L, N, send


SMALL = synthetic.Workload("small", T=300, H=64, E=16, k=4, R=4, bias="uniform")


def test_permute_rows_are_bit_copies(orc):
    d, idx, wt, L, N, send = _pipeline(orc, SMALL)
    canary = 0xBEEF
    send = orc.dispatch_permute(d["x"], L["pos"], N + 7, fill=canary)
    for t in range(SMALL.T):
        for j in range(SMALL.k):
            assert np.array_equal(send[L["pos"][t, j]], d["x"][t])
    assert np.all(send[N:] == canary)
    # send_src is the inverse map: row p holds token send_src[p]
    np.testing.assert_array_equal(send[:N], d["x"][L["send_src"][:N]])


def test_identity_expert_returns_x_plus_residual(orc):
    d, idx, wt, L, N, send = _pipeline(orc, SMALL)
    out = orc.combine_reduce(send, L["pos"], wt, None, d["residual"])
    x = orc.bf16_to_f64(d["x"])
    r = orc.bf16_to_f64(d["residual"])
    np.testing.assert_allclose(out, x + r, rtol=0, atol=1e-14)
    # after the single rounding, within one bf16 step of bf16(x + r)
    # (or within 1e-14 near zero, where the sum of weights' rounding shows)
    assert_bf16_close(orc.bf16_round(out), orc.bf16_round(x + r), atol=1e-14, err_msg="identity")


def test_all_dropped_returns_residual(orc):
    d, idx, wt, L, N, send = _pipeline(orc, SMALL, capacity=0)
    assert N == 0 and np.all(L["pos"] == -1)
    out = orc.combine_reduce(np.zeros((1, SMALL.H), np.uint16), L["pos"], wt, None, d["residual"])
    np.testing.assert_array_equal(orc.bf16_round(out), d["residual"])


def test_k1_weight_is_one(orc):
    w = synthetic.Workload("k1", T=200, H=32, E=8, k=1, R=2)
    d, idx, wt, L, N, send = _pipeline(orc, w)
    assert np.all(wt == 1.0)
    out = orc.combine_reduce(send, L["pos"], wt, None, d["residual"])
    exact = orc.bf16_to_f64(d["x"]) + orc.bf16_to_f64(d["residual"])   # exact in float64
    assert np.array_equal(out, exact)


def test_scaling_by_two_is_exact(orc):
    d, idx, wt, L, N, send = _pipeline(orc, SMALL)
    y = orc.bf16_to_f64(send)
    y2 = _bits(2 * y.astype(np.float32))
    assert np.array_equal(orc.bf16_to_f64(y2), 2 * y)
    o1 = orc.combine_reduce(send, L["pos"], wt, None, None)
    o2 = orc.combine_reduce(y2, L["pos"], wt, None, None)
    assert np.array_equal(o2, 2 * o1)


@pytest.mark.parametrize("capacity", [-1, 40])
def test_combine_matches_einsum(orc, capacity):
    w = synthetic.Workload("sh", T=257, H=48, E=32, k=6, R=8, skew=1.0, shared=True)
    d, idx, wt, L, N, send = _pipeline(orc, w, capacity=capacity)
    r = np.random.default_rng(11)
    # an arbitrary expert output with a wide spread of magnitudes
    y = _bits(r.standard_normal(send.shape) * np.exp2(r.integers(-20, 20, size=send.shape)))
    out = orc.combine_reduce(y, L["pos"], wt, d["shared"], d["residual"])
    pos = L["pos"]
    mask = pos >= 0
    rows = orc.bf16_to_f64(y)[np.where(mask, pos, 0)]             # [T, k, H]
    ref = np.einsum("tj,tjh->th", np.where(mask, wt, 0.0), rows)
    ref += orc.bf16_to_f64(d["shared"]) + orc.bf16_to_f64(d["residual"])
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-9)
    if capacity >= 0:
        assert (~mask).any()
    # the shared expert enters with weight one
    no_sh = orc.combine_reduce(y, L["pos"], wt, None, d["residual"])
    np.testing.assert_allclose(out - no_sh, orc.bf16_to_f64(d["shared"]), rtol=0, atol=1e-9)
    # token subsets give the same rows
    toks = np.array([256, 0, 17, 17], np.int64)
    np.testing.assert_array_equal(orc.combine_reduce(y, L["pos"], wt, d["shared"], d["residual"], tokens=toks), out[toks])


def test_golden_combine(orc):
    with open(GOLDEN) as f:
        case = json.load(f)["cases"][0]
    idx = np.array(case["topk_idx"], np.int32)
    logits = np.array(case["logits"], np.float32)
    _, wt = orc.route_topk(logits, None, case["k"])
    L = orc.dispatch_layout(idx, case["E"], case["R"], case["capacity"])
    x = _bits(case["x"])
    send = orc.dispatch_permute(x, L["pos"], int(L["expert_offsets"][-1]))
    out = orc.combine_reduce(send, L["pos"], wt, None, _bits(case["residual"]))
    np.testing.assert_allclose(out, np.array(case["combine_identity_exact"]), rtol=1e-15)
    np.testing.assert_array_equal(orc.bf16_round(out), _bits(case["combine_identity_bf16"]))


def test_bf16_round_matches_torch_on_float32_values(orc):
    r = np.random.default_rng(2)
    u = r.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[~np.isnan(f)]
    # ties, subnormals, the overflow edge and signed zeros
    extra = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130, 3 * 2 ** -134,
                      2 ** -149, 3.3961776e38, 3.3895314e38, 3.4e38, -0.0, 0.0, np.inf, -np.inf],
                     np.float32)
    f = np.concatenate([f, extra])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.bf16_round(f.astype(np.float64))
    np.testing.assert_array_equal(got, ref)
    nan = orc.bf16_round(np.array([np.nan]))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def test_bf16_round_direct_from_double(orc):
    # halfway between 1 and 1 + 2^-7 plus a hair above: rounds up, although
    # a detour through float32 would first land on the tie and round to even
    v = 1.0 + 2 ** -8 + 2 ** -40
    assert orc.bf16_round(np.array([v]))[0] == 0x3F81
    assert orc.bf16_round(np.array([1.0 + 2 ** -8]))[0] == 0x3F80
