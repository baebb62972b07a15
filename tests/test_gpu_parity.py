"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar (from the definitions in include/moe_ep.h):
  * expert ids, counts, offsets, positions, send_src, the drop mask and the
    send rows: bit-exact;
  * gate weights: within the float32 error bound derived in
    `weight_tolerance` (rounding of l - m, expf, the k-term sum, the divide);
  * combined rows: float32 output within 1e-5 absolute of the float64
    oracle; bf16 output within 1 bf16 step of the oracle's correctly rounded
    value, or within 1e-5 absolute near zero.
Every test prints the case it runs before touching the GPU.
"""

import functools

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tolerance import assert_bf16_close, bf16_value

pytestmark = pytest.mark.gpu

ATOL = 1e-5
CONFIGS = sorted(synthetic.WORKLOADS)


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import combine_route_topk_amd
    return combine_route_topk_amd


DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def up(a, bf16=False):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if bf16:
        t = t.view(torch.bfloat16)
    return t.to(DEV)


def down_u16(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


@functools.lru_cache(maxsize=8)
def inputs(cfg, seed=0):
    return synthetic.make_inputs(synthetic.WORKLOADS[cfg], seed)


@functools.lru_cache(maxsize=8)
def oracle_path(cfg, seed=0):
    w = synthetic.WORKLOADS[cfg]
    d = inputs(cfg, seed)
    idx, wt = oracle.route_topk(d["logits"], d["bias"], w.k)
    L = oracle.dispatch_layout(idx, w.E, w.R, w.capacity)
    N = int(L["expert_offsets"][-1])
    send = oracle.dispatch_permute(d["x"], L["pos"], max(N, 1))
    out = oracle.combine_reduce(send, L["pos"], wt, d["shared"], d["residual"])
    return dict(idx=idx, w=wt, L=L, N=N, send=send, out=out)


def weight_tolerance(logits, idx, w_ref, k):
    """Absolute bound on |w_gpu - w_exact| for float32 softmax over the k
    selected logits: |l - m| * 2^-24 for the rounded difference, 2 ulp for
    expf, k - 1 ulp for the running sum, 1 ulp for the divide, 2 ulp spare."""
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), axis=1)
    d = np.abs(sel - sel.max(axis=1, keepdims=True))
    return (d + k + 5) * 2.0 ** -24 * w_ref + 2.0 ** -126


def send_rows_bound(w):
    return w.T * w.k if w.capacity < 0 else min(w.T * w.k, w.E * w.capacity)


def gpu_layout(moe, idx_t, w, capacity=None):
    C = w.capacity if capacity is None else capacity
    return moe.moe_dispatch_layout(idx_t, w.E, w.R, C)


# ---------------------------------------------------------------------------
# per-step parity on the five workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", CONFIGS)
def test_route_topk(moe, cfg):
    w = synthetic.WORKLOADS[cfg]
    d = inputs(cfg)
    ref = oracle_path(cfg)
    say("route_topk", w.describe())
    idx, wt = moe.moe_route_topk(up(d["logits"]), None if d["bias"] is None else up(d["bias"]), w.k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
    err = np.abs(wt.cpu().numpy().astype(np.float64) - ref["w"])
    tol = weight_tolerance(d["logits"], ref["idx"], ref["w"], w.k)
    assert np.all(err <= tol), f"max weight error {err.max()} (worst ratio {(err / tol).max()})"


@pytest.mark.parametrize("cfg", CONFIGS)
def test_dispatch_layout(moe, cfg):
    w = synthetic.WORKLOADS[cfg]
    ref = oracle_path(cfg)
    say("dispatch_layout", w.describe())
    L = gpu_layout(moe, up(ref["idx"]), w)
    torch.cuda.synchronize()
    for name in ("expert_demand", "expert_counts", "expert_offsets", "dest_counts", "dest_offsets", "pos"):
        np.testing.assert_array_equal(L[name].cpu().numpy(), ref["L"][name], err_msg=name)
    N = ref["N"]
    np.testing.assert_array_equal(L["send_src"][:N].cpu().numpy(), ref["L"]["send_src"][:N])


@pytest.mark.parametrize("cfg", CONFIGS)
def test_dispatch_permute(moe, cfg):
    w = synthetic.WORKLOADS[cfg]
    d = inputs(cfg)
    ref = oracle_path(cfg)
    N = ref["N"]
    rows = send_rows_bound(w)
    say("dispatch_permute", w.describe(), f"N={N} send_rows={rows}")
    send = torch.full((rows, w.H), 0x5A5A, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    moe.moe_dispatch_permute(up(d["x"], True), up(ref["L"]["pos"]), w.E, w.capacity, send=send)
    torch.cuda.synchronize()
    got = down_u16(send)
    np.testing.assert_array_equal(got[:N], ref["send"][:N])
    assert np.all(got[N:] == 0x5A5A), "rows past N were written"


@pytest.mark.parametrize("out_fp32", [False, True])
@pytest.mark.parametrize("cfg", CONFIGS)
def test_combine_reduce(moe, cfg, out_fp32):
    w = synthetic.WORKLOADS[cfg]
    d = inputs(cfg)
    ref = oracle_path(cfg)
    say("combine_reduce", w.describe(), "fp32 out" if out_fp32 else "bf16 out")
    out = moe.moe_combine_reduce(
        up(ref["send"], True), up(ref["L"]["pos"]), up(ref["w"].astype(np.float32)),
        None if d["shared"] is None else up(d["shared"], True),
        None if d["residual"] is None else up(d["residual"], True), out_fp32=out_fp32)
    torch.cuda.synchronize()
    if out_fp32:
        err = np.abs(out.cpu().numpy().astype(np.float64) - ref["out"])
        assert err.max() <= ATOL, f"max abs error {err.max()}"
    else:
        ulps, ndiff = assert_bf16_close(down_u16(out), oracle.bf16_round(ref["out"]), ATOL, err_msg=w.name)
        say(f"bf16 out: max step difference {ulps} (|ref| > 1e-3), {ndiff} of {out.numel()} differ")


@pytest.mark.parametrize("cfg", CONFIGS)
def test_end_to_end(moe, cfg):
    """All four calls chained on the GPU, as the benchmark runs them."""
    w = synthetic.WORKLOADS[cfg]
    d = inputs(cfg)
    ref = oracle_path(cfg)
    say("end_to_end", w.describe())
    x = up(d["x"], True)
    idx, wt = moe.moe_route_topk(up(d["logits"]), None if d["bias"] is None else up(d["bias"]), w.k)
    L = gpu_layout(moe, idx, w)
    send = moe.moe_dispatch_permute(x, L["pos"], w.E, w.capacity)
    out = moe.moe_combine_reduce(send, L["pos"], wt,
                                 None if d["shared"] is None else up(d["shared"], True),
                                 up(d["residual"], True))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(idx.cpu().numpy(), ref["idx"])
    np.testing.assert_array_equal(L["pos"].cpu().numpy(), ref["L"]["pos"])
    np.testing.assert_array_equal(down_u16(send)[:ref["N"]], ref["send"][:ref["N"]])
    # the GPU's own float32 weights feed this combine: widen the bound by
    # their error times the largest routed value
    wtol = weight_tolerance(d["logits"], ref["idx"], ref["w"], w.k).max()
    xmax = np.abs(bf16_value(d["x"])).max()
    assert_bf16_close(down_u16(out), oracle.bf16_round(ref["out"]), ATOL + w.k * wtol * xmax,
                      err_msg=w.name)


# ---------------------------------------------------------------------------
# edge cases and invariants on small shapes
# ---------------------------------------------------------------------------

def _run_small(moe, T, H, E, k, R, capacity=-1, seed=0, logits=None, bias=None, shared=False,
               idx_override=None):
    r = np.random.default_rng(seed)
    if logits is None:
        logits = r.standard_normal((T, E), dtype=np.float32)
    x = synthetic.bf16_bits_from_f32(r.standard_normal((T, H), dtype=np.float32))
    res = synthetic.bf16_bits_from_f32(r.standard_normal((T, H), dtype=np.float32))
    sh = synthetic.bf16_bits_from_f32(r.standard_normal((T, H), dtype=np.float32)) if shared else None
    say(f"small T={T} H={H} E={E} k={k} R={R} C={capacity} seed={seed}")
    if idx_override is None:
        o_idx, o_w = oracle.route_topk(logits, bias, k)
    else:
        o_idx, o_w = idx_override, np.full((T, k), 1.0 / k)
    o_L = oracle.dispatch_layout(o_idx, E, R, capacity)
    N = int(o_L["expert_offsets"][-1])
    o_send = oracle.dispatch_permute(x, o_L["pos"], max(N, 1))
    o_out = oracle.combine_reduce(o_send, o_L["pos"], o_w, sh, res)

    if idx_override is None:
        idx, wt = moe.moe_route_topk(up(logits), None if bias is None else up(bias), k)
    else:
        idx, wt = up(idx_override), up(o_w.astype(np.float32))
    L = moe.moe_dispatch_layout(idx, E, R, capacity)
    rows = T * k if capacity < 0 else min(T * k, E * capacity)
    send = torch.full((max(rows, 1), H), 0x1234, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    moe.moe_dispatch_permute(up(x, True), L["pos"], E, capacity, send=send)
    out = moe.moe_combine_reduce(send, L["pos"], wt, None if sh is None else up(sh, True), up(res, True))
    torch.cuda.synchronize()
    got = dict(idx=idx.cpu().numpy(), w=wt.cpu().numpy(), send=down_u16(send), out=down_u16(out),
               **{n: L[n].cpu().numpy() for n in L if L[n] is not None})
    ref = dict(idx=o_idx, w=o_w, N=N, send=o_send, out=o_out, L=o_L, logits=logits, x=x)
    return got, ref


def _check_small(got, ref, k, weights=True):
    np.testing.assert_array_equal(got["idx"], ref["idx"])
    for name in ("expert_demand", "expert_counts", "expert_offsets", "dest_counts", "dest_offsets", "pos"):
        np.testing.assert_array_equal(got[name], ref["L"][name], err_msg=name)
    N = ref["N"]
    np.testing.assert_array_equal(got["send_src"][:N], ref["L"]["send_src"][:N])
    np.testing.assert_array_equal(got["send"][:N], ref["send"][:N])
    assert np.all(got["send"][N:] == 0x1234)
    if weights:
        tol = weight_tolerance(ref["logits"], ref["idx"], ref["w"], k)
        assert np.all(np.abs(got["w"] - ref["w"]) <= tol)
        xmax = np.abs(bf16_value(ref["x"])).max()
        assert_bf16_close(got["out"], oracle.bf16_round(ref["out"]), ATOL + k * tol.max() * xmax)


SHAPES = [
    # T, H, E, k, R, capacity
    (1, 8, 4, 1, 1, -1),          # single token, one 16-byte chunk per row
    (3, 64, 100, 7, 4, -1),       # E not a multiple of 64, ragged everything
    (77, 7168, 384, 8, 64, -1),   # three full 4 KiB slabs + a half slab
    (1000, 136, 32, 32, 8, -1),   # k = E: a full sort
    (4099, 256, 1024, 32, 16, -1),  # largest E and k
    (5000, 520, 16, 2, 16, 300),  # E / R = 1, capacity
    (333, 64, 30, 5, 3, -1),      # E = 30: two tokens per wave on 4-byte loads, odd T
    (3000, 128, 40, 3, 1, 100),   # R = 1
    (70001, 16, 32, 8, 8, -1),    # 274 tiles: several tiles per scan wave
    (2048, 64, 8, 2, 2, 0),       # capacity 0 drops everything
    (1500, 64, 250, 6, 5, -1),    # E % 4 != 0: 4-byte route loads
    (200, 32, 13, 3, 13, -1),     # E % 4 != 0, one expert per destination
    (512, 16, 64, 8, 8, 70),      # 4096 assignments: the one-block layout, capacity
    (513, 16, 64, 8, 8, 70),      # 4104 assignments: the tiled layout, capacity
    (20000, 16, 64, 4, 8, 900),   # tiled layout, capacity, several tiles
    (1000, 32, 600, 4, 6, 50),    # E > 512 takes the tiled layout at any size
    (16, 65536, 16, 2, 4, -1),    # largest H: 16 slabs of 4096 values per row
    (262144, 8, 64, 8, 8, -1),    # 2^21 assignments: 128 tiles of 16384 (the tile grows past the cap)
    (32768, 8, 1024, 32, 64, -1),  # 2^20 assignments at the largest E and k (8 waves per rank block)
    (3000, 8, 512, 2, 8, -1),     # 8 slots per lane with k <= 2: two route candidates
    (601, 8, 902, 5, 11, -1),     # 4-byte route loads with 15 slots per lane, three candidates
]


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_small_shapes(moe, shape):
    T, H, E, k, R, C = shape
    got, ref = _run_small(moe, T, H, E, k, R, C, seed=T)
    _check_small(got, ref, k)


def test_capacity_zero_returns_residual_exactly(moe):
    T, H, E, k, R = 300, 64, 16, 4, 4
    got, ref = _run_small(moe, T, H, E, k, R, capacity=0, seed=4)
    assert np.all(got["pos"] == -1) and got["expert_offsets"][-1] == 0
    np.testing.assert_array_equal(got["out"], oracle.bf16_round(ref["out"]))


def test_capacity_at_max_demand_is_dropless(moe):
    T, H, E, k, R = 2000, 32, 16, 4, 4
    logits = (np.random.default_rng(9).standard_normal((T, E)) - np.log(np.arange(1, E + 1))).astype(np.float32)
    idx, _ = oracle.route_topk(logits, None, k)
    cmax = int(np.bincount(idx.ravel(), minlength=E).max())
    got_c, _ = _run_small(moe, T, H, E, k, R, capacity=cmax, logits=logits)
    got_d, _ = _run_small(moe, T, H, E, k, R, capacity=-1, logits=logits)
    for name in ("pos", "expert_counts", "expert_offsets", "send_src", "out"):
        np.testing.assert_array_equal(got_c[name], got_d[name], err_msg=name)


def test_constant_logits(moe):
    T, H, E, k, R = 500, 32, 12, 4, 3
    got, ref = _run_small(moe, T, H, E, k, R, capacity=200, logits=np.zeros((T, E), np.float32))
    _check_small(got, ref, k)
    assert np.all(got["idx"] == np.arange(k))
    assert np.all(got["w"] == np.float32(1.0 / k))
    assert np.all((got["pos"] >= 0) == (np.arange(T)[:, None] < 200))


def test_forced_bias_and_special_values(moe):
    T, H, E, k, R = 256, 16, 70, 4, 7
    r = np.random.default_rng(1)
    logits = r.standard_normal((T, E), dtype=np.float32)
    logits[::3, 5] = np.nan
    logits[1::4, 6] = -0.0
    logits[2::4, 6] = 0.0
    logits[::5, 7] = -np.inf
    logits[::7, 8] = logits[::7, 9]   # exact ties
    bias = np.zeros(E, np.float32)
    bias[[3, 66, 41, 12]] = 1e4
    got, ref = _run_small(moe, T, H, E, k, R, logits=logits, bias=bias)
    np.testing.assert_array_equal(got["idx"], ref["idx"])
    assert np.all(np.sort(got["idx"], axis=1) == np.array([3, 12, 41, 66]))
    # selection with special values but no forcing bias
    logits2 = logits.copy()
    logits2[::2, :] = np.nan
    logits2[1::2, 10:] = -np.inf
    got2, ref2 = _run_small(moe, T, H, E, k, R, logits=logits2)
    np.testing.assert_array_equal(got2["idx"], ref2["idx"])


def test_round_robin_indices(moe):
    T, H, E, k, R = 4096, 32, 64, 8, 8
    idx = synthetic.round_robin_idx(T, E, k)
    got, ref = _run_small(moe, T, H, E, k, R, idx_override=idx)
    _check_small(got, ref, k, weights=False)
    per = T * k // E
    assert np.all(got["expert_demand"] == per)


@pytest.mark.parametrize("E", [16, 1024])
def test_zero_tokens(moe, E):
    say(f"zero tokens E={E}")
    k, R, H = 2, 4, 64
    idx, wt = moe.moe_route_topk(torch.empty((0, E), device=DEV), None, k)
    L = moe.moe_dispatch_layout(idx, E, R, -1)
    send = moe.moe_dispatch_permute(torch.empty((0, H), dtype=torch.bfloat16, device=DEV), L["pos"], E)
    out = moe.moe_combine_reduce(send, L["pos"], wt)
    torch.cuda.synchronize()
    assert out.shape == (0, H)
    for name in ("expert_demand", "expert_counts", "expert_offsets", "dest_counts", "dest_offsets"):
        assert np.all(L[name].cpu().numpy() == 0), name


def test_invalid_ids_are_ignored(moe):
    say("invalid ids")
    T, E, k, R = 600, 16, 2, 4
    idx = synthetic.round_robin_idx(T, E, k)
    bad = idx.copy()
    bad[::7, 0] = -3
    bad[::11, 1] = E + 5
    L = moe.moe_dispatch_layout(up(bad), E, R, -1)
    torch.cuda.synchronize()
    pos = L["pos"].cpu().numpy()
    ok = (bad >= 0) & (bad < E)
    assert np.all(pos[~ok] == -1)
    np.testing.assert_array_equal(L["expert_demand"].cpu().numpy(), np.bincount(bad[ok], minlength=E))
    assert np.array_equal(np.sort(pos[ok]), np.arange(ok.sum()))


@pytest.mark.parametrize("E,k,biased", [(200, 6, False), (64, 6, False), (24, 6, False), (100, 6, False),
                                        (30, 6, False), (16, 4, False), (16, 3, True), (64, 6, True),
                                        (512, 10, True), (30, 5, True)])
def test_unnormalised_weights(moe, E, k, biased):
    # E = 16 (k <= 4), 24 and 64 put 16, 8 and 4 tokens in a wave, 100 and 30
    # two; T = 513 leaves the last wave partly empty. With a selection bias
    # the weights still come from the unbiased logits.
    T = 513
    r = np.random.default_rng(2)
    logits = (2 * r.standard_normal((T, E))).astype(np.float32)
    bias = r.uniform(-0.5, 0.5, E).astype(np.float32) if biased else None
    say(f"unnormalised weights T={T} E={E} k={k} bias={biased}")
    idx, wt = moe.moe_route_topk(up(logits), None if bias is None else up(bias), k, normalize=False)
    torch.cuda.synchronize()
    o_idx, o_w = oracle.route_topk(logits, bias, k, normalize=False)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    # full softmax over E: the sum has E terms
    d = np.abs(logits.astype(np.float64).max(axis=1, keepdims=True)
               - np.take_along_axis(logits, o_idx.astype(np.int64), 1))
    tol = (d + E + 5) * 2.0 ** -24 * o_w
    assert np.all(np.abs(wt.cpu().numpy() - o_w) <= tol)


@pytest.mark.parametrize("cfg", CONFIGS)
def test_reproducible(moe, cfg):
    """Two runs of the whole path give the same bits: ids, weights, layout,
    send rows, and the combined rows in bf16 and in fp32."""
    w = synthetic.WORKLOADS[cfg]
    d = inputs(cfg)
    say("reproducible", w.describe())
    sh = None if d["shared"] is None else up(d["shared"], True)
    outs = []
    for _ in range(2):
        idx, wt = moe.moe_route_topk(up(d["logits"]), None if d["bias"] is None else up(d["bias"]), w.k)
        L = gpu_layout(moe, idx, w)
        send = moe.moe_dispatch_permute(up(d["x"], True), L["pos"], w.E, w.capacity)
        out = moe.moe_combine_reduce(send, L["pos"], wt, sh, up(d["residual"], True))
        out32 = moe.moe_combine_reduce(send, L["pos"], wt, sh, up(d["residual"], True), out_fp32=True)
        torch.cuda.synchronize()
        N = int(L["expert_offsets"][-1].item())
        # send_src entries at and past N are never written
        outs.append([t.cpu() for t in (idx, wt, L["expert_counts"], L["expert_offsets"], L["pos"],
                                       L["send_src"][:N], send[:N], out, out32)])
    for a, b in zip(*outs):
        assert np.array_equal(a.contiguous().view(torch.uint8).numpy(), b.contiguous().view(torch.uint8).numpy())


@pytest.mark.parametrize("cfg,capacity", [(1, -1), (1, 20), (2, -1), (2, 3), (3, 615)])
def test_layout_paths_agree(moe, cfg, capacity):
    """The one-block layout (at most 4096 assignments, E <= 512) and the tiled
    two-pass layout give the same counts, offsets, positions and send rows
    for the same assignments: the ids are laid out once with the workload's
    E and again with E' = 1024 experts, which takes the tiled path (experts
    past E receive nothing). The capacity-limited workload (32768
    assignments) goes the other way: a first slice of its tokens fits the
    one-block path."""
    w = synthetic.WORKLOADS[cfg]
    d = inputs(cfg)
    o_idx, _ = oracle.route_topk(d["logits"], d["bias"], w.k)
    if w.T * w.k > 4096:
        o_idx = o_idx[:4096 // w.k]
    T, E = o_idx.shape[0], w.E
    say(f"layout paths agree {w.name} T={T} C={capacity}")
    assert T * w.k <= 4096 and moe.moe_layout_workspace_size(T, E, w.k, w.R) == 0
    assert moe.moe_layout_workspace_size(T, 1024, w.k, 1) > 0
    small = moe.moe_dispatch_layout(up(o_idx), E, w.R, capacity)
    tiled = moe.moe_dispatch_layout(up(o_idx), 1024, 1, capacity)
    torch.cuda.synchronize()
    ref = oracle.dispatch_layout(o_idx, E, w.R, capacity)
    N = int(ref["expert_offsets"][-1])
    for name, n in (("expert_demand", E), ("expert_counts", E), ("expert_offsets", E + 1)):
        np.testing.assert_array_equal(small[name].cpu().numpy()[:n], ref[name][:n], err_msg=name)
        np.testing.assert_array_equal(tiled[name].cpu().numpy()[:n], ref[name][:n], err_msg=name)
    assert np.all(tiled["expert_counts"].cpu().numpy()[E:] == 0)
    assert np.all(tiled["expert_offsets"].cpu().numpy()[E:] == N)
    for L in (small, tiled):
        np.testing.assert_array_equal(L["pos"].cpu().numpy(), ref["pos"])
        np.testing.assert_array_equal(L["send_src"][:N].cpu().numpy(), ref["send_src"][:N])


def _lanes_per_token(E, k, n_groups=0):
    """Lanes of one token in the route kernel, by the launcher's rule (rows
    16-byte aligned): with 16-byte loads (E % 4 == 0) a token takes the
    smallest power of two >= 4 lanes that holds its row in runs of four, its
    k ids and one lane per group, while that is at most 16 (4, 8 or 16
    tokens per wave); else 32 lanes for rows of at most 128 experts (32 with
    4-byte loads) and at most 32 groups; else the whole wave."""
    vec4 = E % 4 == 0
    seg = 4
    while seg < (E + 3) // 4 or seg < k or seg < n_groups:
        seg *= 2
    if vec4 and seg <= 16:
        return seg
    if (E <= 128 if vec4 else E <= 32) and n_groups <= 32:
        return 32
    return 64


def _lane_experts(E, gl, hw):
    """Experts whose logits in-token lane gl holds when a token has hw lanes:
    runs of four (4gl..4gl+3, then + 4hw) with 16-byte loads (E % 4 == 0),
    else gl + hw*i."""
    if E % 4 == 0:
        ids = [4 * hw * q + 4 * gl + c for q in range((E + 4 * hw - 1) // (4 * hw)) for c in range(4)]
    else:
        ids = [gl + hw * i for i in range((E + hw - 1) // hw)]
    return np.array([e for e in ids if e < E], dtype=np.int64)


def test_lane_model():
    """The lane model above against the tokens-per-wave cases the launcher
    documents: 16, 8 and 4 tokens per wave for E <= 16, 32 and 64 with 16-byte
    loads, two for E <= 128, one above; k and the group count can widen it."""
    assert _lanes_per_token(16, 4) == 4 and _lanes_per_token(16, 5) == 8
    assert _lanes_per_token(32, 8) == 8 and _lanes_per_token(64, 8) == 16
    assert _lanes_per_token(64, 17) == 32 and _lanes_per_token(128, 16) == 32
    assert _lanes_per_token(512, 10) == 64 and _lanes_per_token(30, 6) == 32
    assert _lanes_per_token(100, 7) == 32 and _lanes_per_token(32, 5, 16) == 16
    # every expert is held by exactly one in-token lane
    for E, hw in ((512, 64), (64, 16), (30, 32), (100, 32), (16, 4), (902, 64)):
        got = np.sort(np.concatenate([_lane_experts(E, gl, hw) for gl in range(hw)]))
        np.testing.assert_array_equal(got, np.arange(E))


@pytest.mark.parametrize("E,k", [(512, 10), (512, 3), (512, 2), (1024, 32), (1024, 1), (300, 16),
                                 (902, 5), (902, 2), (64, 8), (128, 16), (100, 7), (30, 6),
                                 (32, 6), (32, 8), (16, 3), (16, 4), (64, 12)])
def test_route_candidate_rescans(moe, E, k):
    """Rows that make one lane win round after round (so it must refill its
    candidates from its registers, possibly several times), rows of ties and
    special values, and all-equal rows: on row widths whose lanes hold 8 or
    more slots (three candidates when k >= 3), on rows of at most 128
    experts, where each 32-lane half of a wave routes its own token, and on
    rows of 16 to 64 experts, where 16, 8 or 4 tokens share a wave. The
    planted winner sits on a lane inside the token's own lanes."""
    T = 1024
    r = np.random.default_rng(E * 100 + k)
    pool = np.array([0.0, -0.0, 1.0, -1.0, 0.5, 2.0, np.inf, -np.inf, np.nan], np.float32)
    logits = r.choice(pool, size=(T, E)).astype(np.float32)        # rows 0, 4, ...: ties everywhere
    logits[1::4] = r.standard_normal((len(range(1, T, 4)), E), dtype=np.float32)
    top = r.standard_normal((len(range(2, T, 4)), E), dtype=np.float32) - 10.0
    hw = _lanes_per_token(E, k)
    lanes = [gl for gl in range(hw) if _lane_experts(E, gl, hw).size]   # lanes past the row hold padding
    for n, row in enumerate(range(2, T, 4)):
        ids = _lane_experts(E, lanes[n % len(lanes)], hw)           # one lane holds the best
        top[n, ids] = 10.0 + r.standard_normal(len(ids), dtype=np.float32)
        if n % 2:
            top[n, ids[::2]] = 10.0                                  # with exact ties inside it
    logits[2::4] = top
    logits[3::4] = 0.0                                               # all equal: ids 0..k-1
    say(f"route candidate rescans T={T} E={E} k={k}")
    idx, wt = moe.moe_route_topk(up(logits), None, k)
    torch.cuda.synchronize()
    o_idx, o_w = oracle.route_topk(logits, None, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    assert np.all(o_idx[3::4] == np.arange(k))
    fin = np.all(np.isfinite(np.take_along_axis(logits, o_idx.astype(np.int64), axis=1)), axis=1)
    tol = weight_tolerance(logits[fin], o_idx[fin], o_w[fin], k)
    assert np.all(np.abs(wt.cpu().numpy()[fin] - o_w[fin]) <= tol)


@pytest.mark.parametrize("E", [512, 384])
def test_route_misaligned_rows(moe, E):
    """Logit rows that are only 4-byte aligned take the 4-byte load path."""
    T, k = 777, 8
    r = np.random.default_rng(E)
    logits = r.standard_normal((T, E), dtype=np.float32)
    bias = r.uniform(-0.1, 0.1, E).astype(np.float32)
    say(f"route misaligned rows T={T} E={E} k={k}")
    flat = torch.zeros(T * E + 1, dtype=torch.float32, device=DEV)
    flat[1:] = up(logits.ravel())
    view = flat[1:].view(T, E)
    assert view.data_ptr() % 16 != 0
    idx, wt = moe.moe_route_topk(view, up(bias), k)
    torch.cuda.synchronize()
    o_idx, o_w = oracle.route_topk(logits, bias, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    assert np.all(np.abs(wt.cpu().numpy() - o_w) <= weight_tolerance(logits, o_idx, o_w, k))


GROUPED = [
    # T, E, k, n_groups, topk_groups, bias
    (32768, 512, 10, 8, 4, None),      # fine-grained shape, 8 groups of 64, at most 4
    (4096, 384, 8, 64, 4, "uniform"),  # one group per destination of 6 experts
    (3000, 256, 8, 8, 4, "uniform"),   # groups of 32 in one 16-byte slot quad
    (2000, 320, 8, 20, 4, "uniform"),  # groups of 16, E not a multiple of 256
    (700, 960, 9, 30, 5, None),        # groups of 32, 4 slot quads, last one partial
    (1500, 1024, 12, 16, 3, "uniform"),  # groups of 64, 16 slots per lane
    (513, 192, 6, 12, 2, None),        # groups of 16, one partial slot quad
    (999, 256, 8, 32, 8, "uniform"),
    (500, 100, 7, 4, 2, None),         # E % 4 == 0 but tiny groups of 25
    (333, 70, 6, 7, 2, "uniform"),     # 4-byte route path
    (200, 64, 4, 64, 4, None),         # one expert per group: plain top-k
    (300, 64, 6, 8, 8, None),          # every group allowed: plain top-k
    (777, 32, 5, 16, 3, "uniform"),    # 16 groups need 16 lanes: four tokens per wave, odd T
    (901, 32, 4, 8, 3, "uniform"),     # eight tokens per wave, 16-byte loads, odd T
    (555, 16, 3, 4, 2, None),          # sixteen tokens per wave
    (401, 30, 4, 5, 2, None),          # two tokens per wave, 4-byte loads, odd T
]


@pytest.mark.parametrize("case", GROUPED, ids=[str(c) for c in GROUPED])
def test_route_topk_grouped(moe, case):
    T, E, k, G, M, b = case
    r = np.random.default_rng(T + E + G)
    logits = r.standard_normal((T, E), dtype=np.float32)
    logits[::13, 3] = np.nan
    logits[::7, E // 2] = logits[::7, E // 2 + 1]            # exact ties
    bias = r.uniform(-0.1, 0.1, E).astype(np.float32) if b else None
    say(f"route_topk_grouped T={T} E={E} k={k} groups={G} topk_groups={M}")
    idx, wt = moe.moe_route_topk_grouped(up(logits), None if bias is None else up(bias), k, G, M)
    torch.cuda.synchronize()
    o_idx, o_w = oracle.route_topk_grouped(logits, bias, k, G, M)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    finite = np.isfinite(o_w).all(axis=1)
    tol = weight_tolerance(logits, o_idx, o_w, k)
    assert np.all(np.abs(wt.cpu().numpy() - o_w)[finite] <= tol[finite])


@pytest.mark.parametrize("E,k,G,M", [(512, 10, 8, 4), (1024, 12, 16, 3), (384, 8, 64, 4), (120, 6, 8, 3),
                                     (64, 8, 8, 3), (32, 6, 8, 4)])
def test_route_grouped_ties_and_specials(moe, E, k, G, M):
    """Group-limited routing on rows full of ties, signed zeros, infinities
    and NaNs (group maxima tie too), on rows where one lane holds the best
    experts of its groups, and on all-equal rows (the lowest groups and ids
    win)."""
    T = 1024
    r = np.random.default_rng(E + k + G)
    pool = np.array([0.0, -0.0, 1.0, -1.0, 2.0, np.inf, -np.inf, np.nan], np.float32)
    logits = r.choice(pool, size=(T, E)).astype(np.float32)
    logits[1::3] = r.standard_normal((len(range(1, T, 3)), E), dtype=np.float32) - 10.0
    hw = _lanes_per_token(E, k, G)
    lanes = [gl for gl in range(hw) if _lane_experts(E, gl, hw).size]
    for n, row in enumerate(range(1, T, 3)):
        ids = _lane_experts(E, lanes[n % len(lanes)], hw)
        logits[row, ids] = 10.0 + np.round(r.standard_normal(len(ids)), 1).astype(np.float32)
    logits[2::3] = 0.0
    bias = np.where(r.random(E) < 0.5, 0.0, 1.0).astype(np.float32)   # ties survive the bias
    say(f"route grouped ties T={T} E={E} k={k} groups={G} topk_groups={M}")
    for b in (None, bias):
        idx, wt = moe.moe_route_topk_grouped(up(logits), None if b is None else up(b), k, G, M)
        torch.cuda.synchronize()
        o_idx, o_w = oracle.route_topk_grouped(logits, b, k, G, M)
        np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
        fin = np.all(np.isfinite(np.take_along_axis(logits, o_idx.astype(np.int64), axis=1)), axis=1)
        tol = weight_tolerance(logits[fin], o_idx[fin], o_w[fin], k)
        assert np.all(np.abs(wt.cpu().numpy()[fin] - o_w[fin]) <= tol)
        if b is None:
            # all-equal rows: groups 0..M-1 tie and win, and inside them the lowest ids
            assert np.all(o_idx[2::3] == np.arange(k))


# ---------------------------------------------------------------------------
# the permutes' prefetch of x (k >= 4, the token 4096 ahead): batches just
# past the prefetch distance, tokens with every replica dropped, and
# capacity limits, checked row by row against the oracle
# ---------------------------------------------------------------------------

PREFETCH_TOKENS = 4096   # tokens ahead that a permute block loads for k >= 4


@pytest.mark.parametrize("T,k,capacity", [
    (PREFETCH_TOKENS + 1, 4, -1),       # one token past the distance
    (PREFETCH_TOKENS + 13, 8, 40),      # capacity: most late tokens fully dropped
    (3 * PREFETCH_TOKENS + 7, 5, 300),  # several distances, partial drops
    (2 * PREFETCH_TOKENS, 3, -1),       # k = 3: no prefetch, same results
])
def test_permutes_around_prefetch(moe, T, k, capacity):
    H, E, R = 288, 64, 8  # H = 288: part of one slab, for both payloads
    say(f"permutes around the prefetch T={T} k={k} capacity={capacity} H={H} E={E}")
    rng = np.random.default_rng(T + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, :4] += 3.0  # skew: the first experts overflow a capacity
    x = synthetic.normal_bf16(T, 1, (T, H))
    idx, _ = oracle.route_topk(logits, None, k)
    L = oracle.dispatch_layout(idx, E, R, capacity)
    rows = T * k if capacity < 0 else min(T * k, E * capacity)
    ref = oracle.dispatch_permute(x, L["pos"], rows, fill=0x5A5A)
    if capacity >= 0:
        dropped_tokens = int(np.all(L["pos"] < 0, axis=1).sum())
        assert dropped_tokens > 0, "the case must hold tokens with every replica dropped"
    pos = up(L["pos"])
    send = torch.full((rows, H), 0x5A5A, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    moe.moe_dispatch_permute(up(x, True), pos, E, capacity, send=send)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(down_u16(send), ref)
    rb = oracle.fp8_row_bytes(H)
    ref8 = oracle.dispatch_permute_fp8(x, L["pos"], rows, rb, fill=0xA5)
    send8 = torch.full((rows, rb), 0xA5, dtype=torch.uint8, device=DEV)
    moe.moe_dispatch_permute_fp8(up(x, True), pos, E, capacity, send=send8)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(send8.cpu().numpy(), ref8)


# ---------------------------------------------------------------------------
# token counts past the grid's limit: the launchers split the work
# ---------------------------------------------------------------------------

MAX_ROW_BLOCKS = 1 << 22   # blocks per launch of the row kernels before the launcher splits


@pytest.mark.parametrize("k", [2, 4])
def test_row_kernels_past_grid_limit(moe, k):
    """Permute, FP8 permute and combine over 2^22 + 3 tokens (one block per
    token, so the launcher issues two launches with offset pointers): every
    send row against its token's row, and sampled tokens on both sides of the
    split against the oracle. With k = 4 the permutes' prefetch of the token
    4096 ahead reaches across the split into the second launch's tokens."""
    T, H, E = MAX_ROW_BLOCKS + 3, 32, 8
    say(f"row kernels past the grid limit T={T} H={H} k={k}")
    gen = torch.Generator(device=DEV).manual_seed(11)
    x = torch.randint(-16000, 16000, (T, H), dtype=torch.int16, device=DEV, generator=gen)
    x = (x & 0x3FFF).view(torch.bfloat16)                     # finite values below 2
    res = torch.randn((T, H), device=DEV, generator=gen).to(torch.bfloat16)
    # identity-like layout: replica j of token t goes to row j*T + t (distinct, dropless)
    tt = torch.arange(T, dtype=torch.int32, device=DEV)
    pos = torch.stack([tt + j * T for j in range(k)], dim=1).contiguous()
    wt = torch.rand((T, k), device=DEV, generator=gen)
    send = moe.moe_dispatch_permute(x, pos, E)
    out = moe.moe_combine_reduce(send, pos, wt, None, res)
    out32 = moe.moe_combine_reduce(send, pos, wt, None, res, out_fp32=True)
    torch.cuda.synchronize()
    xi = x.view(torch.int16)
    for j in range(k):
        assert torch.equal(send[j * T:(j + 1) * T].view(torch.int16), xi), f"replica {j}"
    del send
    sample = np.unique(np.concatenate([np.arange(4), np.arange(MAX_ROW_BLOCKS - 4, T),
                                       np.random.default_rng(3).integers(0, T, 200)]))
    s = torch.from_numpy(sample).to(DEV)
    xs, rs = down_u16(x[s]), down_u16(res[s])
    ws = wt[s].cpu().numpy().astype(np.float64)
    n = len(sample)
    npos = np.stack([np.arange(n) + j * n for j in range(k)], 1).astype(np.int32)
    ref = oracle.combine_reduce(np.concatenate([xs] * k), npos, ws, None, rs)
    got32 = out32[s].cpu().numpy().astype(np.float64)
    assert np.abs(got32 - ref).max() <= 1e-5
    assert_bf16_close(down_u16(out[s]), oracle.bf16_round(ref), 1e-5, err_msg="combine past the grid limit")
    del out, out32
    send8 = moe.moe_dispatch_permute_fp8(x, pos, E)
    torch.cuda.synchronize()
    rows8 = oracle.dispatch_permute_fp8(xs, np.arange(n, dtype=np.int32).reshape(-1, 1), n)
    for j in range(k):
        np.testing.assert_array_equal(send8[s + j * T].cpu().numpy(), rows8)


def test_route_past_grid_limit(moe):
    """The routing kernel over 2^24 + 5 tokens of 256 experts (one wave per
    token, four per block: past 2^22 blocks the launcher splits the tokens):
    sampled tokens on both sides of the split against the oracle."""
    T, E, k = 4 * MAX_ROW_BLOCKS + 5, 256, 2
    say(f"route past the grid limit T={T} E={E} k={k}")
    gen = torch.Generator(device=DEV).manual_seed(12)
    logits = torch.randn((T, E), device=DEV, generator=gen)
    idx, wt = moe.moe_route_topk(logits, None, k)
    torch.cuda.synchronize()
    cut = 4 * MAX_ROW_BLOCKS
    sample = np.unique(np.concatenate([np.arange(3), np.arange(cut - 3, T),
                                       np.random.default_rng(4).integers(0, T, 300)]))
    s = torch.from_numpy(sample).to(DEV)
    lg = logits[s].cpu().numpy()
    o_idx, o_w = oracle.route_topk(lg, None, k)
    np.testing.assert_array_equal(idx[s].cpu().numpy(), o_idx)
    assert np.all(np.abs(wt[s].cpu().numpy() - o_w) <= weight_tolerance(lg, o_idx, o_w, k))
    del logits


@pytest.mark.parametrize("cfg", [3, 5])
def test_split_batch_matches_whole(moe, cfg):
    """Grid-size independence: routing, permute and combine of a workload in
    one launch each, and of its two halves in separate launches (a grid of
    half the blocks each, on offset views), give the same bits token by
    token."""
    w = synthetic.WORKLOADS[cfg]
    d = inputs(cfg)
    ref = oracle_path(cfg)
    say("split batch", w.describe())
    lg = up(d["logits"])
    x, res = up(d["x"], True), up(d["residual"], True)
    sh = None if d["shared"] is None else up(d["shared"], True)
    idx, wt = moe.moe_route_topk(lg, None, w.k)
    h = w.T // 2 + 1                                            # halves of unequal size
    idx_a, wt_a = moe.moe_route_topk(lg[:h], None, w.k)
    idx_b, wt_b = moe.moe_route_topk(lg[h:], None, w.k)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([idx_a, idx_b]), idx)
    assert torch.equal(torch.cat([wt_a, wt_b]).view(torch.int32), wt.view(torch.int32))
    pos = up(ref["L"]["pos"])
    rows = send_rows_bound(w)
    send = moe.moe_dispatch_permute(x, pos, w.E, w.capacity)
    send2 = torch.full_like(send.view(torch.int16), 0x5A5A).view(torch.bfloat16)
    # each half writes its own tokens' rows (both halves stay within the bound)
    moe.moe_dispatch_permute(x[:h], pos[:h], w.E, w.capacity, send=send2, send_rows=rows)
    moe.moe_dispatch_permute(x[h:], pos[h:], w.E, w.capacity, send=send2, send_rows=rows)
    out = moe.moe_combine_reduce(send, pos, wt, sh, res)
    out_a = moe.moe_combine_reduce(send, pos[:h], wt[:h], None if sh is None else sh[:h], res[:h])
    out_b = moe.moe_combine_reduce(send, pos[h:], wt[h:], None if sh is None else sh[h:], res[h:])
    torch.cuda.synchronize()
    N = ref["N"]
    assert torch.equal(send2[:N].view(torch.int16), send[:N].view(torch.int16))
    assert torch.equal(torch.cat([out_a, out_b]).view(torch.int16), out.view(torch.int16))
