"""GPU parity of moe_route_dispatch_layout, routing and layout in one call.

Its outputs must equal those of moe_route_topk followed by
moe_dispatch_layout bit for bit (ids, weights, counts, offsets, positions,
send rows), and the oracle's: ids and layout bit-exact, weights within the
float32 softmax bound. Batches of at most 4096 assignments (E <= 512, 16-byte
rows) take the one-launch path, where the last block to finish builds the
layout; the rest take the two kernels. The one-launch path is also checked
with a workspace full of garbage, on repeated calls sharing a workspace, and
replayed from a HIP graph. Every test prints its case first.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
READY = 0x6D6F6574 << 32   # the ticket's ready word (its upper half is the kernel's magic)
LAYOUT = ("expert_demand", "expert_counts", "expert_offsets", "dest_counts", "dest_offsets", "pos")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import combine_route_topk_amd
    return combine_route_topk_amd


def say(*a):
    print("[case]", *a, flush=True)


def up(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def weight_tolerance(logits, idx, w_ref, k, normalize=True):
    """float32 softmax bound: rounding of l - m, 2 ulp of expf, the sum's
    roundings (k terms, or E without renormalisation), the divide, 2 spare."""
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), axis=1)
    if normalize:
        d = np.abs(sel - sel.max(axis=1, keepdims=True))
        n = k
    else:
        d = np.abs(logits.astype(np.float64).max(axis=1, keepdims=True) - sel)
        n = logits.shape[1]
    return (d + n + 5) * 2.0 ** -24 * w_ref + 2.0 ** -126


def check(moe, logits, bias, k, R, capacity, normalize=True, workspace=None):
    """Run the fused call and the two separate calls on the same inputs and
    compare them with each other and with the oracle."""
    T, E = logits.shape
    lg, b = up(logits), up(bias)
    F = moe.moe_route_dispatch_layout(lg, b, k, R, capacity, normalize=normalize, workspace=workspace)
    idx, wt = moe.moe_route_topk(lg, b, k, normalize=normalize)
    L = moe.moe_dispatch_layout(idx, E, R, capacity)
    torch.cuda.synchronize()
    assert torch.equal(F["topk_idx"], idx), "ids differ from moe_route_topk's"
    assert torch.equal(F["topk_w"].view(torch.int32), wt.view(torch.int32)), "weights differ from moe_route_topk's"
    for n in LAYOUT:
        assert torch.equal(F[n], L[n]), f"{n} differs from moe_dispatch_layout's"
    o_idx, o_w = oracle.route_topk(logits, bias, k, normalize=normalize)
    np.testing.assert_array_equal(F["topk_idx"].cpu().numpy(), o_idx)
    fin = np.all(np.isfinite(np.take_along_axis(logits, o_idx.astype(np.int64), axis=1)), axis=1)
    tol = weight_tolerance(logits[fin], o_idx[fin], o_w[fin], k, normalize)
    assert np.all(np.abs(F["topk_w"].cpu().numpy()[fin] - o_w[fin]) <= tol)
    OL = oracle.dispatch_layout(o_idx, E, R, capacity)
    for n in LAYOUT:
        np.testing.assert_array_equal(F[n].cpu().numpy(), OL[n], err_msg=n)
    N = int(OL["expert_offsets"][-1])
    np.testing.assert_array_equal(F["send_src"][:N].cpu().numpy(), OL["send_src"][:N])
    assert torch.equal(F["send_src"][:N], L["send_src"][:N])
    return F


@pytest.mark.parametrize("cfg", sorted(synthetic.WORKLOADS))
def test_workloads(moe, cfg):
    """Tiny and decode take the one-launch path; the others the two kernels."""
    w = synthetic.WORKLOADS[cfg]
    d = synthetic.make_inputs(w, seed=0, with_activations=False)
    say("route+layout", w.describe(),
        "one launch" if w.T * w.k <= 4096 and w.E <= 512 else "two launches")
    check(moe, d["logits"], d["bias"], w.k, w.R, w.capacity)


# T, E, k, R, capacity, bias, normalize: every tokens-per-wave shape of the
# one-launch path (16, 8, 4, 2 and 1 tokens per wave, 4 and 8 slots per
# lane, two and three candidates), ragged last blocks, capacity drops, and
# shapes past its limits (4097 assignments, E = 520 or 1024, E % 4 != 0)
SWEEP = [
    (1, 16, 2, 4, -1, False, True),
    (37, 16, 4, 4, 3, True, True),
    (255, 16, 3, 2, -1, False, False),
    (512, 32, 8, 8, -1, True, True),
    (300, 24, 6, 4, 40, False, True),
    (129, 64, 8, 16, -1, True, True),
    (700, 64, 5, 8, 30, False, False),
    (63, 100, 7, 4, -1, True, True),
    (511, 128, 8, 32, -1, False, True),
    (128, 256, 8, 32, -1, True, True),
    (33, 256, 1, 8, 0, False, True),
    (409, 300, 10, 10, -1, True, True),
    (200, 512, 10, 64, -1, False, True),
    (2048, 512, 2, 64, 5, True, False),
    (4096, 64, 1, 8, -1, False, True),
    (1365, 512, 3, 8, -1, True, True),
    (4097, 64, 1, 8, -1, False, True),       # past 4096 assignments: two launches
    (100, 520, 4, 8, -1, True, True),        # E > 512: two launches
    (100, 1024, 8, 16, -1, False, True),
    (333, 70, 6, 7, -1, True, True),         # E % 4 != 0: 4-byte loads, two launches
]


@pytest.mark.parametrize("case", SWEEP, ids=[str(c) for c in SWEEP])
def test_sweep(moe, case):
    T, E, k, R, C, use_bias, normalize = case
    r = np.random.default_rng(T * 7 + E)
    logits = r.standard_normal((T, E), dtype=np.float32)
    logits[::11, E // 3] = logits[::11, E // 3 + 1]                      # exact ties
    logits[::5] -= (np.log1p(np.arange(E)) * 0.7).astype(np.float32)     # a skew toward low ids
    bias = r.uniform(-0.3, 0.3, E).astype(np.float32) if use_bias else None
    say(f"route+layout T={T} E={E} k={k} R={R} C={C} bias={use_bias} normalize={normalize}")
    check(moe, logits, bias, k, R, C, normalize)


def test_garbage_and_shared_workspace(moe):
    """A workspace of random bytes (the ticket words included) on the first
    call, which takes the stamped slow path, then one workspace shared by
    calls of different sizes in a row, which take the atomic-add path."""
    ws = torch.from_numpy(np.random.default_rng(1).integers(0, 256, 4096, dtype=np.uint8)).to(DEV)
    cases = [(128, 256, 8, 32, -1), (256, 16, 2, 4, -1), (64, 512, 10, 64, 3), (1000, 64, 4, 8, -1),
             (1, 32, 2, 4, -1), (128, 256, 8, 32, -1)]
    for n, (T, E, k, R, C) in enumerate(cases):
        r = np.random.default_rng(100 + n)
        logits = r.standard_normal((T, E), dtype=np.float32)
        say(f"route+layout shared workspace call {n}: T={T} E={E} k={k}")
        assert moe.moe_route_dispatch_layout_workspace_size(T, E, k, R) <= ws.numel()
        check(moe, logits, None, k, R, C, workspace=ws)
        # every one-launch call leaves the ticket ready for the next
        assert int(ws[:8].view(torch.int64).item()) == READY


def test_zero_tokens(moe):
    say("route+layout with zero tokens")
    F = moe.moe_route_dispatch_layout(torch.empty((0, 64), device=DEV), None, 4, 8)
    torch.cuda.synchronize()
    for n in ("expert_demand", "expert_counts", "expert_offsets", "dest_counts", "dest_offsets"):
        assert bool((F[n] == 0).all()), n


@pytest.mark.parametrize("cfg", [1, 2])
def test_graph_replay(moe, cfg):
    """The one-launch path captured in a HIP graph with the permute and the
    combine: each replay (which reuses the call's stamp) reproduces the eager
    step bit for bit, with eager work and synchronisation between replays."""
    w = synthetic.WORKLOADS[cfg]
    d = synthetic.make_inputs(w, seed=0)
    say("route+layout graph replay", w.describe())
    logits, bias = up(d["logits"]), up(d["bias"])
    x = up(d["x"].view(np.int16)).view(torch.bfloat16)
    res = up(d["residual"].view(np.int16)).view(torch.bfloat16)
    ws = torch.zeros(moe.moe_route_dispatch_layout_workspace_size(w.T, w.E, w.k, w.R), dtype=torch.uint8,
                     device=DEV)
    F = moe.moe_route_dispatch_layout(logits, bias, w.k, w.R, w.capacity, workspace=ws)
    send = torch.empty((moe.send_rows_bound(w.T, w.k, w.E, w.capacity), w.H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()

    def step():
        moe.moe_route_dispatch_layout(logits, bias, w.k, w.R, w.capacity, workspace=ws, out=F, stream=s)
        moe.moe_dispatch_permute(x, F["pos"], w.E, w.capacity, send=send, stream=s)
        moe.moe_combine_reduce(send, F["pos"], F["topk_w"], None, res, out=out, stream=s)

    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    N = int(F["expert_offsets"][w.E].item())
    ref = {n: F[n].clone() for n in ("topk_idx", "topk_w") + LAYOUT}
    ref["send"], ref["out"] = send[:N].clone(), out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for n in ("topk_idx",) + LAYOUT:
            F[n].fill_(-9)
        F["topk_w"].fill_(float("nan"))
        send.view(torch.int16).fill_(0x5A5A)
        out.view(torch.int16).fill_(0x1234)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {n: F[n] for n in ("topk_idx", "topk_w") + LAYOUT}
        got["send"], got["out"] = send[:N], out
        for n, t in ref.items():
            a, b = got[n], t
            if a.dtype.is_floating_point:
                a = a.view(torch.int16 if a.element_size() == 2 else torch.int32)
                b = b.view(torch.int16 if b.element_size() == 2 else torch.int32)
            assert torch.equal(a, b), f"replay {rep}: {n} differs from the eager step"
        assert int(ws[:8].view(torch.int64).item()) == READY


@pytest.mark.parametrize("T,E,k,R", [(128, 256, 8, 32), (512, 64, 8, 8), (4096, 128, 1, 16)])
def test_back_to_back_calls_see_new_ids(moe, T, E, k, R):
    """64 calls in a row on one stream and one workspace, each on new logits
    written just before it: the last block of each call must build the
    layout from that call's ids, which the other blocks release through the
    ticket's read-modify-write. Every call is compared with the two
    separate calls on the same logits; a layout built from ids of the call
    before would differ."""
    say(f"back-to-back fused calls T={T} E={E} k={k} R={R}")
    gen = torch.Generator(device=DEV).manual_seed(T + E)
    ws = torch.empty(moe.moe_route_dispatch_layout_workspace_size(T, E, k, R), dtype=torch.uint8, device=DEV)
    outs, refs = [], []
    for i in range(64):
        lg = torch.randn((T, E), device=DEV, generator=gen)
        F = moe.moe_route_dispatch_layout(lg, None, k, R, -1, workspace=ws)
        idx, wt = moe.moe_route_topk(lg, None, k)
        L = moe.moe_dispatch_layout(idx, E, R, -1)
        outs.append(F)
        refs.append((idx, wt, L))
    torch.cuda.synchronize()
    for i, (F, (idx, wt, L)) in enumerate(zip(outs, refs)):
        assert torch.equal(F["topk_idx"], idx), f"call {i}: ids"
        assert torch.equal(F["topk_w"].view(torch.int32), wt.view(torch.int32)), f"call {i}: weights"
        for n in LAYOUT + ("send_src",):
            assert torch.equal(F[n], L[n]), f"call {i}: {n}"
