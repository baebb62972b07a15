"""GPU parity of the FP8 dispatch payload against the CPU oracle.

Codes and scale bytes are integers decided by floating point; both sides
decide them from the exact x / 2^e, so the bar is bit-exact for every byte
of every written row, with untouched rows and padding checked by a canary.
The decode to bf16 is exact (or a correctly rounded subnormal), so it is
bit-exact too. Combine after an FP8 dispatch keeps the combine bar.
Every test prints the case it runs before touching the GPU.
"""

import concurrent.futures
import functools
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tolerance import assert_bf16_close

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FILL = 0xA5
ATOL = 1e-5


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


def gpu_quantize(moe, x_u16):
    """Quantise rows through the FP8 permute with the identity map (k = 1)."""
    T, H = x_u16.shape
    pos = up(np.arange(T, dtype=np.int32).reshape(T, 1))
    send = torch.full((T, moe.moe_fp8_row_bytes(H)), FILL, dtype=torch.uint8, device=DEV)
    moe.moe_dispatch_permute_fp8(up_bf16(x_u16), pos, 1, send=send)
    torch.cuda.synchronize()
    return send.cpu().numpy()


def check_rows(send, x_u16, H):
    codes, scales = oracle.fp8_quantize_rows(x_u16)
    np.testing.assert_array_equal(send[:, :H], codes)
    np.testing.assert_array_equal(send[:, H:H + H // 32], scales)
    assert np.all(send[:, H + H // 32:] == 0), "padding not zero"


def finite_bf16_patterns():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return b[(b & 0x7F80) != 0x7F80]


def test_every_bf16_pattern(moe):
    """All 65280 finite bf16 patterns, once in order (narrow blocks) and once
    shuffled (tiny values in blocks with a large maximum)."""
    pats = finite_bf16_patterns()
    pad = np.zeros(-pats.size % 512, np.uint16)          # up to 128 rows of 512
    r = np.random.default_rng(0)
    for name, arr in (("ordered", pats), ("shuffled", r.permutation(pats))):
        x = np.concatenate([arr, pad]).reshape(-1, 512)
        say(f"fp8 quantise every bf16 pattern ({name}) rows={x.shape[0]} H=512")
        check_rows(gpu_quantize(moe, x), x, 512)


@pytest.mark.parametrize("H", [2048, 7168])
def test_wide_dynamic_range(moe, H):
    """Block maxima from 2^-135 (bf16 subnormals, scale byte 0) to 2^120."""
    r = np.random.default_rng(H)
    n = 64
    x = r.standard_normal((n, H)).astype(np.float32)
    x *= (2.0 ** r.integers(-135, 121, size=(n, H // 32, 1))).repeat(32, axis=2).reshape(n, H)
    x = synthetic.bf16_bits_from_f32(x)
    x[0, :32] = 0
    x[1, :32] = 0x8000
    x[2, :32] = 0x0001
    x[3, :32] = 0x7F7F                     # largest finite bf16
    x[4, 32:64] = np.where(np.arange(32) % 2 == 0, 0x43E0, 0xC3E0)   # +-448
    say(f"fp8 quantise wide dynamic range H={H}")
    check_rows(gpu_quantize(moe, x), x, H)


@pytest.mark.parametrize("H", [32, 96, 160, 544, 4128, 65536])
def test_partial_wave_widths(moe, H):
    """Widths that leave lanes of the last wave (or slab) idle; the scale
    line is zero after the row's last scale byte. H = 65536, the largest
    width, gives 16 slabs and 16 scale lines per row."""
    r = np.random.default_rng(H)
    x = synthetic.bf16_bits_from_f32(r.standard_normal((37, H)).astype(np.float32) * 3)
    say(f"fp8 quantise partial-wave width H={H}")
    check_rows(gpu_quantize(moe, x), x, H)


def test_dequant_every_code_and_scale(moe):
    """All 254 finite codes under every scale byte 0..247 (the range the
    quantiser produces), through moe_fp8_dequant."""
    codes_all = np.arange(256, dtype=np.uint8)
    codes_all = codes_all[(codes_all & 0x7F) != 0x7F]
    H = 256
    reps = -(-codes_all.size // H) + 1
    rows = []
    scales = []
    for s in range(248):
        c = np.resize(np.roll(codes_all, s), H * reps).reshape(reps, H)
        rows.append(c)
        scales.append(np.full((reps, H // 32), s, np.uint8))
    codes = np.concatenate(rows)
    sc = np.concatenate(scales)
    rb = moe.moe_fp8_row_bytes(H)
    buf = np.zeros((codes.shape[0], rb), np.uint8)
    buf[:, :H] = codes
    buf[:, H:H + H // 32] = sc
    say(f"fp8 dequant every code x scale rows={codes.shape[0]}")
    out = moe.moe_fp8_dequant(up(buf), H)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(down_u16(out), oracle.fp8_dequant_rows(codes, sc))


def test_dequant_stops_at_n_rows(moe):
    r = np.random.default_rng(1)
    H, rows, N = 64, 40, 23
    x = synthetic.bf16_bits_from_f32(r.standard_normal((rows, H)).astype(np.float32))
    send = gpu_quantize(moe, x)
    say("fp8 dequant bounded by a device row count")
    out = torch.full((rows, H), 0x5A5A, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    moe.moe_fp8_dequant(up(send), H, n_rows=up(np.array([N], np.int32)), out=out)
    torch.cuda.synchronize()
    got = down_u16(out)
    c, s = oracle.fp8_quantize_rows(x[:N])
    np.testing.assert_array_equal(got[:N], oracle.fp8_dequant_rows(c, s))
    assert np.all(got[N:] == 0x5A5A)


def quantize_tokens(x_u16):
    """The oracle's FP8 row of every token (its permute with an identity
    map), computed in row chunks on a few host threads: the oracle is
    single-threaded C and its calls release the interpreter lock."""
    T = x_u16.shape[0]
    chunk = max(1, -(-T // 64))

    def rows(a):
        return oracle.dispatch_permute_fp8(a, np.arange(a.shape[0], dtype=np.int32).reshape(-1, 1), a.shape[0])

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(rows, [x_u16[i:i + chunk] for i in range(0, T, chunk)]))
    return np.concatenate(parts) if parts else np.zeros((0, oracle.fp8_row_bytes(x_u16.shape[1])), np.uint8)


@functools.lru_cache(maxsize=3)
def token_rows(cfg):
    w, d, _, _, _ = routed(cfg)
    return quantize_tokens(d["x"])


@functools.lru_cache(maxsize=8)
def routed(cfg):
    w = synthetic.WORKLOADS[cfg]
    d = synthetic.make_inputs(w, seed=0)
    idx, wt = oracle.route_topk(d["logits"], d["bias"], w.k)
    L = oracle.dispatch_layout(idx, w.E, w.R, w.capacity)
    return w, d, idx, wt, L


def send_rows_bound(w):
    return w.T * w.k if w.capacity < 0 else min(w.T * w.k, w.E * w.capacity)


@pytest.mark.parametrize("cfg", sorted(synthetic.WORKLOADS))
def test_permute_fp8_workloads(moe, cfg):
    """Every workload: the oracle's positions drive the GPU FP8 permute.
    Small workloads are compared whole. On the large ones every kept row is
    compared: the oracle quantises each token once (its FP8 row with an
    identity map), and row p must equal the row of token send_src[p]; rows
    past N keep the fill pattern."""
    w, d, idx, wt, L = routed(cfg)
    N = int(L["expert_offsets"][-1])
    rows = send_rows_bound(w)
    rb = moe.moe_fp8_row_bytes(w.H)
    say("permute_fp8", w.describe(), f"N={N} rows={rows}")
    send_t = torch.full((rows, rb), FILL, dtype=torch.uint8, device=DEV)
    moe.moe_dispatch_permute_fp8(up_bf16(d["x"]), up(L["pos"]), w.E, w.capacity, send=send_t)
    torch.cuda.synchronize()
    if w.T * w.H <= 1 << 20:
        send = send_t.cpu().numpy()
        ref = oracle.dispatch_permute_fp8(d["x"], L["pos"], rows, fill=FILL)
        np.testing.assert_array_equal(send, ref)
        return
    expect = up(token_rows(cfg))[up(L["send_src"][:N].astype(np.int64))]
    assert torch.equal(send_t[:N], expect), "kept FP8 rows differ from the oracle's"
    if N < rows:
        assert bool((send_t[N:] == FILL).all()), "rows past N written"


@pytest.mark.parametrize("cfg", sorted(synthetic.WORKLOADS))
def test_fp8_end_to_end(moe, cfg):
    """route -> layout -> FP8 permute -> decode (identity expert) -> combine,
    all on the GPU, against the oracle's same chain, on every workload. On
    the large workloads the oracle's send rows are its per-token FP8 rows
    placed by its send_src (each kept replica's row is its token's quantised
    row), and its decoded rows likewise: the oracle's own permute quantises
    every replica again, k times the work for the same bytes."""
    w, d, _, _, _ = routed(cfg)
    say("fp8 end to end", w.describe())
    idx, wt = moe.moe_route_topk(up(d["logits"]), None if d["bias"] is None else up(d["bias"]), w.k)
    L = moe.moe_dispatch_layout(idx, w.E, w.R, w.capacity)
    rows = send_rows_bound(w)
    send = moe.moe_dispatch_permute_fp8(up_bf16(d["x"]), L["pos"], w.E, w.capacity)
    y = moe.moe_fp8_dequant(send, w.H, n_rows=L["expert_offsets"][w.E:])
    out = moe.moe_combine_reduce(y, L["pos"], wt, None if d["shared"] is None else up_bf16(d["shared"]),
                                 up_bf16(d["residual"]))
    torch.cuda.synchronize()
    o_idx, o_w = oracle.route_topk(d["logits"], d["bias"], w.k)
    np.testing.assert_array_equal(idx.cpu().numpy(), o_idx)
    OL = oracle.dispatch_layout(o_idx, w.E, w.R, w.capacity)
    np.testing.assert_array_equal(L["pos"].cpu().numpy(), OL["pos"])
    N = int(OL["expert_offsets"][-1])
    H = w.H
    if w.T * H <= 1 << 20:
        o_send = oracle.dispatch_permute_fp8(d["x"], OL["pos"], rows)[:N]
        o_y = oracle.fp8_dequant_rows(o_send[:, :H], o_send[:, H:H + H // 32])
    else:
        tok = token_rows(cfg)
        src = OL["send_src"][:N].astype(np.int64)
        o_send = tok[src]
        o_y = oracle.fp8_dequant_rows(tok[:, :H], tok[:, H:H + H // 32])[src]
    assert torch.equal(send[:N], up(o_send)), "FP8 send rows differ from the oracle's"
    del o_send
    assert torch.equal(y[:N].view(torch.int16), up(o_y.view(np.int16))), "decoded rows differ from the oracle's"
    ref = oracle.combine_reduce(o_y, OL["pos"], o_w, d["shared"], d["residual"])
    # the GPU's own float32 weights feed this combine: widen the bound by
    # their error (the float32 softmax bound) times the largest routed value
    sel = np.take_along_axis(d["logits"].astype(np.float64), o_idx.astype(np.int64), axis=1)
    wtol = ((np.abs(sel - sel.max(axis=1, keepdims=True)) + w.k + 5) * 2.0 ** -24 * o_w).max()
    ymax = np.abs(oracle.bf16_to_f64(o_y)).max() if N else 0.0
    assert_bf16_close(down_u16(out), oracle.bf16_round(ref), ATOL + w.k * wtol * ymax, err_msg=w.name)


def test_zero_tokens_and_all_dropped(moe):
    say("fp8 permute: zero tokens, and every replica dropped")
    H = 64
    rb = moe.moe_fp8_row_bytes(H)
    empty = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    send = torch.full((4, rb), FILL, dtype=torch.uint8, device=DEV)
    moe.moe_dispatch_permute_fp8(empty, torch.empty((0, 2), dtype=torch.int32, device=DEV), 2, 2, send=send)
    x = up_bf16(np.ones((8, H), np.uint16))
    pos = torch.full((8, 2), -1, dtype=torch.int32, device=DEV)
    moe.moe_dispatch_permute_fp8(x, pos, 2, 2, send=send)
    torch.cuda.synchronize()
    assert bool((send == FILL).all())
