"""GPU parity of the tile-signalled return path: the stand-in expert GEMM
(MFMA, fp32 accumulation) against the oracle's float64 linear map, and the
rows the signalled consumer returns against the GEMM's own output.

Bars:
  * y: |y_gpu - v| <= 2^-8 |v| + 2 * H * 2^-24 * sum_h |x_h w_h| for the
    exact value v (one bf16 rounding of an fp32 sum of H exact products);
    and, element by element against the oracle's output y_o (v rounded once
    to bf16), |y_gpu - y_o| <= that bound + half a bf16 step of y_o, since
    y_o itself lies within half a step of v;
  * ret: bit-identical to y on every row below N; rows at or past N
    untouched (canary); the status word reads 0;
  * y from the signalled launch: bit-identical to the plain launch (same
    tiles, same arithmetic), whatever the consumer count, band grouping or
    remote-first rotation.
Every test prints the case it runs before touching the GPU.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CANARY = 0x5A5A


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


def up_bf16(u16):
    return up(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16)


def down_u16(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def canary(rows, cols):
    return torch.full((rows, cols), CANARY, dtype=torch.int16, device=DEV).view(torch.bfloat16)


def labels(cnt):
    S, El = cnt.shape
    return np.concatenate([np.repeat(np.arange(El), cnt[s]) for s in range(S)]).astype(np.int64)


def check_y(y_bits, x_bits, lab, W):
    """Rows y_bits [n, H_out] computed from inputs x_bits [n, H] of local
    experts lab [n], against the exact value and the oracle."""
    ref = np.empty_like(y_bits)
    exact = np.empty(y_bits.shape)
    mag = np.empty(y_bits.shape)
    for l in np.unique(lab):
        m = lab == l
        ref[m] = oracle.expert_linear(x_bits[m], np.array([[int(m.sum())]], np.int32), W[l][None])
        xs, wl = oracle.bf16_to_f64(x_bits[m]), oracle.bf16_to_f64(W[l])
        exact[m] = xs @ wl.T
        mag[m] = np.abs(xs) @ np.abs(wl).T
    got = oracle.bf16_to_f64(y_bits)
    bound = 2.0 ** -8 * np.abs(exact) + 2 * x_bits.shape[1] * 2.0 ** -24 * mag + 2.0 ** -133
    bad = np.abs(got - exact) > bound
    assert not bad.any(), f"{bad.sum()} values outside the bound; worst excess {(np.abs(got - exact) - bound).max()}"
    # the oracle's correctly rounded value obeys the same bound (a check of
    # the bound itself); where cancellation leaves a result near zero the
    # fp32 sum may sit more than one bf16 step from it, so no ulp bar here
    ref_v = oracle.bf16_to_f64(ref)
    assert np.all(np.abs(ref_v - exact) <= bound)
    # the GPU against the oracle, element by element
    bad = np.abs(got - ref_v) > bound + bf16_half_step(ref_v)
    assert not bad.any(), f"{bad.sum()} values differ from the oracle beyond the bound"


def bf16_half_step(v):
    """Half the spacing of bf16 values at |v| (8 significant bits; the
    subnormal spacing 2^-133 below 2^-126)."""
    _, e = np.frexp(np.abs(v))              # |v| = m * 2^e, 0.5 <= m < 1
    return np.ldexp(1.0, np.maximum(e - 9, -134))


CASES = [  # (S, E_l, max count, H, H_out, seed)
    (4, 4, 300, 256, 256, 0),
    (3, 2, 129, 64, 128, 1),       # one row past a tile edge
    (8, 1, 40, 512, 384, 2),
    (2, 8, 1000, 128, 256, 3),     # long blocks, several bands each
    (16, 6, 90, 7168 // 8, 256, 4),
    (4, 2, 200, 256, 640, 5),      # a full 512-column tile, then a 128-column one
    (2, 3, 300, 192, 1024, 6),     # two full column tiles; 6 K-steps
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_expert_linear_small(moe, case):
    S, El, cmax, H, H_out, seed = case
    r = np.random.default_rng(seed)
    cnt = r.integers(0, cmax + 1, size=(S, El)).astype(np.int32)
    cnt[0, 0] = 0
    cnt[-1, -1] = 128
    N = int(cnt.sum())
    rows = N + 7
    recv = synthetic.bf16_bits_from_f32(r.standard_normal((rows, H)).astype(np.float32))
    W = synthetic.bf16_bits_from_f32((r.standard_normal((El, H_out, H)) / np.sqrt(H)).astype(np.float32))
    say(f"expert_linear S={S} E_l={El} N={N} H={H} H_out={H_out}")
    y = canary(rows, H_out)
    moe.moe_expert_linear(up_bf16(recv), up(cnt), up_bf16(W), y=y)
    torch.cuda.synchronize()
    yb = down_u16(y)
    check_y(yb[:N], recv[:N], labels(cnt), W)
    assert np.all(yb[N:] == CANARY), "rows past N written"


RETURN_CASES = [  # (consumers, band_group, self_rank, H_out); 0 consumers = producers return
    (0, 1, 0, 256),
    (0, 3, 2, 256),
    (1, 1, 0, 256),
    (8, 4, 3, 256),
    (64, 2, 1, 256),
    (4, 64, 2, 256),
    (16, 2, 1, 1152),              # three column tiles per band, the last partial
    (0, 2, 3, 1152),
]


@pytest.mark.parametrize("rc", RETURN_CASES, ids=[str(c) for c in RETURN_CASES])
def test_signalled_return_matches_plain(moe, rc):
    consumers, group, self_rank, H_out = rc
    r = np.random.default_rng(10 + consumers)
    S, El, H = 4, 3, 256
    cnt = r.integers(0, 400, size=(S, El)).astype(np.int32)
    cnt[1, :] = 0                               # a source with nothing to return
    N = int(cnt.sum())
    rows = N + 5
    recv = synthetic.bf16_bits_from_f32(r.standard_normal((rows, H)).astype(np.float32))
    W = synthetic.make_expert_weights(El, H_out, H, seed=1)
    say(f"expert_linear_return consumers={consumers} band_group={group} self={self_rank} N={N}")
    y_plain = moe.moe_expert_linear(up_bf16(recv), up(cnt), up_bf16(W))
    y, ret, ws = moe.moe_expert_linear_return(up_bf16(recv), up(cnt), up_bf16(W), self_rank, consumers, group,
                                              y=canary(rows, H_out), ret=canary(rows, H_out))
    torch.cuda.synchronize()
    status = int(ws[:4].view(torch.int32).item())
    assert status == 0, f"status word {status}"
    yb, rb = down_u16(y), down_u16(ret)
    np.testing.assert_array_equal(yb[:N], down_u16(y_plain)[:N])
    np.testing.assert_array_equal(rb[:N], yb[:N])
    assert np.all(rb[N:] == CANARY) and np.all(yb[N:] == CANARY)
    check_y(yb[:N], recv[:N], labels(cnt), W)


def test_repeated_calls_reuse_workspace(moe):
    """Flags are cleared by each call itself: back-to-back calls on one
    workspace, with different counts, all return every row."""
    r = np.random.default_rng(20)
    S, El, H, H_out = 8, 2, 128, 128
    ws = torch.empty(moe.moe_expert_linear_workspace_size(S, El, 4096), dtype=torch.uint8, device=DEV)
    W = up_bf16(synthetic.make_expert_weights(El, H_out, H, seed=2))
    recv = up_bf16(synthetic.bf16_bits_from_f32(r.standard_normal((4096, H)).astype(np.float32)))
    for call in range(4):
        cnt = r.integers(0, 256 if call % 2 else 64, size=(S, El)).astype(np.int32)
        N = int(cnt.sum())
        say(f"repeated expert_linear_return call={call} N={N}")
        y, ret, _ = moe.moe_expert_linear_return(recv, up(cnt), W, call % S, 8 * (call % 2), 3, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 0
        assert torch.equal(ret[:N].view(torch.int16), y[:N].view(torch.int16))


def test_counts_past_buffer_do_nothing(moe):
    say("expert_linear_return with counts totalling more than max_rows")
    S, El, H, H_out, rows = 2, 2, 64, 128, 100
    cnt = np.array([[60, 30], [20, 10]], np.int32)          # 120 > 100 rows
    W = up_bf16(synthetic.make_expert_weights(El, H_out, H))
    recv = up_bf16(np.zeros((rows, H), np.uint16))
    y, ret, ws = moe.moe_expert_linear_return(recv, up(cnt), W, 0, 4, 2, y=canary(rows, H_out),
                                              ret=canary(rows, H_out))
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 2
    assert bool((y.view(torch.int16) == CANARY).all()) and bool((ret.view(torch.int16) == CANARY).all())


def test_largest_workload_share(moe):
    """The 32768-token, 512-expert, top-10 workload on 64 ranks: this GPU's
    send buffer read as 64 source segments x 8 local experts, through the
    stand-in expert (2048 -> 2048). ret must equal y bit for bit; y rows are
    checked against the oracle on a sample, including every block's first
    and last row of one source."""
    w = synthetic.WORKLOADS[5]
    El = w.E // w.R
    d = synthetic.make_inputs(w, seed=0)
    idx, _ = oracle.route_topk(d["logits"], d["bias"], w.k)
    L = oracle.dispatch_layout(idx, w.E, w.R, w.capacity)
    N = int(L["expert_offsets"][-1])
    cnt = L["expert_counts"].reshape(w.R, El).astype(np.int32)
    say(f"expert_linear_return full share S={w.R} E_l={El} N={N} H={w.H}")
    send = moe.moe_dispatch_permute(up_bf16(d["x"]), up(L["pos"]), w.E, w.capacity)
    W = synthetic.make_expert_weights(El, w.H, w.H)
    for consumers in (0, 32):
        y, ret, ws = moe.moe_expert_linear_return(send, up(cnt), up_bf16(W), 0, consumers, 4)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == 0
        assert torch.equal(ret.view(torch.int16), y.view(torch.int16)), f"consumers={consumers}"
    recv = oracle.dispatch_permute(d["x"], L["pos"], N)
    starts = np.concatenate([[0], np.cumsum(cnt.ravel())])[:-1]
    r = np.random.default_rng(3)
    sample = np.unique(np.concatenate([r.integers(0, N, 96), starts[:El], starts[1:El + 1] - 1, [N - 1]]))
    sample = sample[(sample >= 0) & (sample < N)]
    yb = down_u16(y[torch.from_numpy(sample).to(DEV)])
    check_y(yb, recv[sample], labels(cnt)[sample], W)
