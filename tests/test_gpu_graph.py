"""The four calls of one step captured in a HIP graph and replayed: every
replay must reproduce the eager step bit for bit.

Between replays the outputs are overwritten by eager work and the device is
synchronised, so a replay that skipped or misordered a node (or read stale
memory) would show. The library issues no memset or copy, only kernel
launches, so the whole step is capturable. Every test prints its case first.
"""

import numpy as np
import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


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


def up_bf16(a):
    return None if a is None else up(a.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_graph_replay_matches_eager(moe, cfg):
    w = synthetic.WORKLOADS[cfg]
    d = synthetic.make_inputs(w, seed=0)
    say("graph replay", w.describe())
    logits, bias = up(d["logits"]), up(d["bias"])
    x, sh, res = up_bf16(d["x"]), up_bf16(d["shared"]), up_bf16(d["residual"])
    rows = w.T * w.k if w.capacity < 0 else min(w.T * w.k, w.E * w.capacity)
    i32 = dict(dtype=torch.int32, device=DEV)
    idx = torch.empty((w.T, w.k), **i32)
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device=DEV)
    L = {"expert_demand": torch.empty(w.E, **i32), "expert_counts": torch.empty(w.E, **i32),
         "expert_offsets": torch.empty(w.E + 1, **i32), "dest_counts": torch.empty(w.R, **i32),
         "dest_offsets": torch.empty(w.R + 1, **i32), "pos": torch.empty((w.T, w.k), **i32),
         "send_src": torch.empty(w.T * w.k, **i32)}
    ws = torch.empty(max(moe.moe_layout_workspace_size(w.T, w.E, w.k, w.R), 16), dtype=torch.uint8, device=DEV)
    send = torch.empty((rows, w.H), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()

    def step():
        moe.moe_route_topk(logits, bias, w.k, topk_idx=idx, topk_w=wt, stream=s)
        moe.moe_dispatch_layout(idx, w.E, w.R, w.capacity, workspace=ws, out=L, stream=s)
        moe.moe_dispatch_permute(x, L["pos"], w.E, w.capacity, send=send, stream=s)
        moe.moe_combine_reduce(send, L["pos"], wt, sh, res, out=out, stream=s)

    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        step()
    torch.cuda.synchronize()
    N = int(L["expert_offsets"][w.E].item())
    ref = {"idx": idx.clone(), "wt": wt.clone(), "send": send[:N].clone(), "out": out.clone(),
           **{k: v.clone() for k, v in L.items() if k != "send_src"}, "send_src": L["send_src"][:N].clone()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work between replays: scribble over every output
        idx.fill_(-7)
        wt.fill_(float("nan"))
        for v in L.values():
            v.fill_(-9)
        send.view(torch.int16).fill_(0x5A5A)
        out.view(torch.int16).fill_(0x1234)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {"idx": idx, "wt": wt, "send": send[:N], "out": out,
               **{k: v for k, v in L.items() if k != "send_src"}, "send_src": L["send_src"][:N]}
        for name, t in ref.items():
            a, b = got[name], t
            if a.dtype.is_floating_point:
                a, b = a.view(torch.int16 if a.element_size() == 2 else torch.int32), \
                    b.view(torch.int16 if b.element_size() == 2 else torch.int32)
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
