"""Seeded random sweep of whole-path configurations on the GPU against the
oracle: route (plain or group-limited), layout, permute and combine, with
random T, H, E, k, R, capacity, bias and shared expert. The cases come from
one fixed generator, so a failure names a reproducible configuration.

Bars as in test_gpu_parity: ids, counts, offsets, positions, send_src and
send rows bit-exact; weights within the float32 softmax bound; combined
rows within one bf16 step (or 1e-5 absolute) of the oracle evaluated on the
oracle's own weights, widened by the weights' float32 error.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tolerance import assert_bf16_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ATOL = 1e-5


def make_cases(n=64, seed=2024):
    r = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        E = int(r.choice([8, 16, 24, 60, 64, 96, 128, 200, 256, 384, 512, 1000, 1024]))
        R = int(r.choice([d for d in range(1, min(E, 64) + 1) if E % d == 0]))
        k = int(r.integers(1, min(E, 32) + 1))
        T = int(r.integers(1, 3000))
        H = int(r.choice([8, 64, 264, 512, 1032, 2048]))
        capacity = -1 if r.random() < 0.5 else int(r.integers(0, max(1, 2 * T * k // E) + 1))
        bias = bool(r.random() < 0.5)
        shared = bool(r.random() < 0.3)
        groups = None
        if r.random() < 0.3:
            divs = [g for g in range(2, min(E, 64) + 1) if E % g == 0]
            if divs:
                G = int(r.choice(divs))
                M = int(r.integers(1, G + 1))
                if k <= M * (E // G):
                    groups = (G, M)
        cases.append((T, H, E, k, R, capacity, bias, shared, groups, int(r.integers(0, 1 << 30))))
    return cases


CASES = make_cases()


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import combine_route_topk_amd
    return combine_route_topk_amd


def up(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def up_bf16(a):
    return None if a is None else up(a.view(np.int16)).view(torch.bfloat16)


def down_u16(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}-H{c[1]}-E{c[2]}-k{c[3]}-R{c[4]}-C{c[5]}"
                                             f"{'-bias' if c[6] else ''}{'-shared' if c[7] else ''}"
                                             f"{'-g%dm%d' % c[8] if c[8] else ''}" for c in CASES])
def test_random_path(moe, case):
    T, H, E, k, R, capacity, use_bias, use_shared, groups, seed = case
    print("[case]", case, flush=True)
    r = np.random.default_rng(seed)
    logits = r.standard_normal((T, E), dtype=np.float32)
    bias = r.uniform(-0.5, 0.5, E).astype(np.float32) if use_bias else None
    x = synthetic.bf16_bits_from_f32(r.standard_normal((T, H), dtype=np.float32))
    res = synthetic.bf16_bits_from_f32(r.standard_normal((T, H), dtype=np.float32))
    sh = synthetic.bf16_bits_from_f32(r.standard_normal((T, H), dtype=np.float32)) if use_shared else None

    if groups is None:
        o_idx, o_w = oracle.route_topk(logits, bias, k)
        idx, wt = moe.moe_route_topk(up(logits), up(bias), k)
    else:
        o_idx, o_w = oracle.route_topk_grouped(logits, bias, k, *groups)
        idx, wt = moe.moe_route_topk_grouped(up(logits), up(bias), k, *groups)
    L = moe.moe_dispatch_layout(idx, E, R, capacity)
    rows = T * k if capacity < 0 else min(T * k, E * capacity)
    send = moe.moe_dispatch_permute(up_bf16(x), L["pos"], E, capacity, send_rows=max(rows, 1))
    out = moe.moe_combine_reduce(send, L["pos"], wt, up_bf16(sh), up_bf16(res))
    torch.cuda.synchronize()

    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    sel = np.take_along_axis(logits.astype(np.float64), o_idx.astype(np.int64), axis=1)
    wtol = (np.abs(sel - sel.max(axis=1, keepdims=True)) + k + 5) * 2.0 ** -24 * o_w + 2.0 ** -126
    assert np.all(np.abs(wt.cpu().numpy().astype(np.float64) - o_w) <= wtol)

    OL = oracle.dispatch_layout(o_idx, E, R, capacity)
    for name in ("expert_demand", "expert_counts", "expert_offsets", "dest_counts", "dest_offsets", "pos"):
        np.testing.assert_array_equal(L[name].cpu().numpy(), OL[name], err_msg=name)
    N = int(OL["expert_offsets"][-1])
    np.testing.assert_array_equal(L["send_src"][:N].cpu().numpy(), OL["send_src"][:N])
    o_send = oracle.dispatch_permute(x, OL["pos"], max(rows, 1))
    np.testing.assert_array_equal(down_u16(send)[:N], o_send[:N])
    ref = oracle.combine_reduce(o_send, OL["pos"], o_w, sh, res)
    xmax = np.abs(oracle.bf16_to_f64(x)).max() if T else 0.0
    assert_bf16_close(down_u16(out), oracle.bf16_round(ref), ATOL + k * wtol.max() * xmax, err_msg=str(case))
