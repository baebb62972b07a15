"""GPU parity of the receive-side regroup against the CPU oracle.

The regroup is index and byte work, so the bar is bit-exact: both offset
tables, recv_pos, and every moved row. Rows past N (or past what a map
names) must stay untouched. Cases cover the hand-worked example, random
count matrices at the size limits (S or E_l at 1024, S*E_l at 4096), empty
blocks and sources, negative counts (read as 0), a receive buffer larger
than N, a destination fed by several simulated sources, and the largest
workload's single-GPU share (send buffer viewed as the receive buffer).
Every test prints the case it runs before touching the GPU.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")
FILL = 0x5A5A


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import combine_route_topk_amd
    return combine_route_topk_amd


def say(*a):
    print("[case]", *a, flush=True)


def up(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def up_bf16(a_u16):
    return up(a_u16.view(np.int16)).view(torch.bfloat16)


def down_u16(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def rand_rows(rng, n, H):
    return rng.integers(0, 1 << 16, size=(n, H), dtype=np.uint16)


def check_regroup(moe, cnt, H, max_rows=None, seed=0, recv=None):
    """Run layout, regroup and ungroup on the GPU and compare all of it with
    the oracle bit for bit."""
    cnt = np.asarray(cnt, np.int32)
    S, El = cnt.shape
    ref = oracle.recv_regroup_layout(np.maximum(cnt, 0))
    N = int(ref["source_offsets"][-1])
    rows = N if max_rows is None else max_rows
    say(f"regroup S={S} E_l={El} N={N} max_rows={rows} H={H}")
    L = moe.moe_recv_regroup_layout(up(cnt), rows)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(L["local_expert_offsets"].cpu().numpy(), ref["local_expert_offsets"])
    np.testing.assert_array_equal(L["source_offsets"].cpu().numpy(), ref["source_offsets"])
    np.testing.assert_array_equal(L["recv_pos"][:N].cpu().numpy(), ref["recv_pos"])
    if rows == 0:
        return L
    rng = np.random.default_rng(seed)
    if recv is None:
        recv = rand_rows(rng, rows, H)
    n_rows = L["source_offsets"][S:]
    grouped = torch.full((rows, H), FILL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    moe.moe_recv_regroup(up_bf16(recv), L["recv_pos"], n_rows, grouped=grouped)
    back = torch.full((rows, H), FILL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    moe.moe_recv_ungroup(grouped, L["recv_pos"], n_rows, out=back)
    torch.cuda.synchronize()
    want = oracle.scatter_rows(recv[:N], ref["recv_pos"], rows, fill=FILL)
    np.testing.assert_array_equal(down_u16(grouped), want)
    want_back = oracle.gather_rows(want, ref["recv_pos"])
    got_back = down_u16(back)
    np.testing.assert_array_equal(got_back[:N], want_back)
    np.testing.assert_array_equal(got_back[:N], recv[:N])
    assert np.all(got_back[N:] == FILL), "ungroup wrote rows past N"
    return L


def test_hand_worked(moe):
    case = next(c for c in json.load(open(GOLDEN))["cases"] if "recv_counts" in c)
    L = check_regroup(moe, case["recv_counts"], H=8)
    np.testing.assert_array_equal(L["local_expert_offsets"].cpu().numpy(), case["local_expert_offsets"])
    np.testing.assert_array_equal(L["source_offsets"].cpu().numpy(), case["source_offsets"])
    np.testing.assert_array_equal(L["recv_pos"].cpu().numpy(), case["recv_pos"])


SHAPES = [  # (S, E_l, max count, H)
    (1, 1, 50, 8),
    (1, 8, 40, 64),
    (8, 1, 40, 64),
    (4, 4, 0, 64),          # nothing received
    (64, 8, 30, 2048),      # 64 sources x 8 local experts
    (32, 12, 20, 7168),     # 384 experts on 32 GPUs, wide rows
    (1024, 4, 3, 16),       # S at its limit
    (4, 1024, 3, 16),       # E_l at its limit
    (64, 64, 2, 24),        # S*E_l at its limit, H not a multiple of 64
    (3, 5, 700, 4104),      # ragged slab tail: 4104 = 4096 + 8 columns
    (2, 3, 5, 65536),       # the largest row width: 16 slabs per row
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_random_counts(moe, shape):
    S, El, cmax, H = shape
    rng = np.random.default_rng(S * 7919 + El)
    cnt = rng.integers(0, cmax + 1, size=(S, El)).astype(np.int32)
    if S * El > 4:  # empty blocks, an empty source and an empty expert
        cnt[rng.integers(0, S, size=S * El // 4), rng.integers(0, El, size=S * El // 4)] = 0
        cnt[S // 2, :] = 0
        cnt[:, El // 2] = 0
    check_regroup(moe, cnt, H)


def test_negative_counts_read_as_zero(moe):
    cnt = np.array([[3, -2, 1], [-1, 4, 0], [2, 2, -7]], np.int32)
    check_regroup(moe, cnt, H=64)


@pytest.mark.parametrize("extra", [0, 1, 5000])
def test_buffer_larger_than_n(moe, extra):
    rng = np.random.default_rng(extra)
    cnt = rng.integers(0, 60, size=(16, 8)).astype(np.int32)
    check_regroup(moe, cnt, H=256, max_rows=int(cnt.sum()) + extra)


def test_zero_rows_buffer(moe):
    check_regroup(moe, np.zeros((4, 4), np.int32), H=64, max_rows=0)


def test_simulated_destination(moe):
    """S sources dispatch their own tokens (oracle layout and permute); one
    destination receives segment d of every source's send buffer with the
    matching slice of that source's expert counts, regroups on the GPU, and
    must hold each of its local experts' rows contiguously, in source order
    and, within a source, in that source's send order."""
    w = synthetic.WORKLOADS[1]      # tiny: 256 tokens, 16 experts, top-2, 4 ranks
    El = w.E // w.R
    d_id = 1
    segs, counts = [], []
    for s in range(w.R):
        inp = synthetic.make_inputs(w, seed=100 + s)
        idx, _ = oracle.route_topk(inp["logits"], inp["bias"], w.k)
        L = oracle.dispatch_layout(idx, w.E, w.R, w.capacity)
        N = int(L["expert_offsets"][-1])
        send = oracle.dispatch_permute(inp["x"], L["pos"], max(N, 1))
        a, b = int(L["dest_offsets"][d_id]), int(L["dest_offsets"][d_id + 1])
        segs.append(send[a:b])
        counts.append(L["expert_counts"][d_id * El:(d_id + 1) * El])
    recv = np.concatenate(segs).view(np.uint16)
    cnt = np.stack(counts).astype(np.int32)
    Lg = check_regroup(moe, cnt, H=w.H, recv=recv)
    # expert l's block holds source 0's rows of l, then source 1's, ...
    leo = Lg["local_expert_offsets"].cpu().numpy()
    assert leo[-1] == recv.shape[0]
    np.testing.assert_array_equal(np.diff(leo), cnt.sum(axis=0))


def test_largest_workload_share(moe):
    """The 32768-token, 512-expert, top-10 workload on 64 ranks: this GPU's
    send buffer viewed as a receive buffer (64 sources x 8 local experts,
    counts = the layout's expert counts), regrouped and ungrouped at full
    size. Layout tables are compared whole; all N regrouped rows against the
    oracle's scatter of the same receive buffer, and the ungrouped rows by
    the round trip."""
    w = synthetic.WORKLOADS[5]      # fine_grained
    El = w.E // w.R
    inp = synthetic.make_inputs(w, seed=0)
    idx, _ = oracle.route_topk(inp["logits"], inp["bias"], w.k)
    L = oracle.dispatch_layout(idx, w.E, w.R, w.capacity)
    cnt = L["expert_counts"].reshape(w.R, El).astype(np.int32)
    ref = oracle.recv_regroup_layout(cnt)
    N = int(ref["source_offsets"][-1])
    rows = w.T * w.k
    say(f"regroup full share S={w.R} E_l={El} N={N} rows={rows} H={w.H}")
    G = moe.moe_recv_regroup_layout(up(cnt), rows)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(G["local_expert_offsets"].cpu().numpy(), ref["local_expert_offsets"])
    np.testing.assert_array_equal(G["source_offsets"].cpu().numpy(), ref["source_offsets"])
    np.testing.assert_array_equal(G["recv_pos"][:N].cpu().numpy(), ref["recv_pos"])
    gen = torch.Generator(device=DEV).manual_seed(5)
    recv = torch.randint(-32768, 32768, (rows, w.H), dtype=torch.int16, device=DEV, generator=gen)
    recv = recv.view(torch.bfloat16)
    n_rows = G["source_offsets"][w.R:]
    grouped = moe.moe_recv_regroup(recv, G["recv_pos"], n_rows)
    back = moe.moe_recv_ungroup(grouped, G["recv_pos"], n_rows)
    torch.cuda.synchronize()
    assert torch.equal(back[:N].view(torch.int16), recv[:N].view(torch.int16))
    o_grouped = oracle.scatter_rows(down_u16(recv[:N]), ref["recv_pos"], N)
    assert torch.equal(grouped[:N].view(torch.int16), up(o_grouped.view(np.int16))), \
        "regrouped rows differ from the oracle's"
