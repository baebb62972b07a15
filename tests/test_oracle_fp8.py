"""Pins for the oracle's FP8 dispatch payload: E4M3 codes with one
power-of-two scale byte (biased exponent, E8M0) per 32 values.

Sources: aicassindra "gpu_moe_all_to_all", "Latency-bound at decode,
bandwidth-bound at prefill" (a lower-precision dispatch payload, since the
expert matmul casts its input anyway); zenaique Q&A
"moe-hide-alltoall-techniques" (shrink the payload). The pages fix neither
format nor scaling; the reading pinned here: OCP E4M3, one scale 2^e per
32 values along H, e the smallest integer >= -127 with amax <= 448 * 2^e,
codes rounded to nearest with ties to even.

Independent references: torch's float8_e4m3fn dtype (decode of all codes,
rounding of float32 values), math.frexp for the block exponent, a value
worked by hand in tests/golden/fp8_block.json, and bounds from the format.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_block.json")


def torch_e4m3_codes(values):
    """torch's own float32 -> float8_e4m3fn conversion, as code bytes."""
    t = torch.tensor(np.asarray(values, np.float32), dtype=torch.float32)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def all_e4m3_values():
    codes = np.arange(256, dtype=np.uint8)
    return codes, torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch(orc):
    codes, ref = all_e4m3_values()
    got = orc.e4m3_value(codes)
    nan = np.isnan(ref)
    assert list(codes[nan]) == [0x7F, 0xFF]
    assert np.all(np.isnan(got[nan]))
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_round_representable_and_midpoints(orc):
    """Every finite code maps to itself; every midpoint between neighbours
    goes to the even code (checked against torch, which rounds to nearest
    even: midpoints have 5 significant bits, exact in float32)."""
    codes, vals = all_e4m3_values()
    finite = ~np.isnan(vals)
    got = orc.e4m3_round(vals[finite])
    # -0.0 and +0.0 keep their codes
    np.testing.assert_array_equal(got, codes[finite])
    pos = np.unique(vals[finite & (vals >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2
    for sign in (1.0, -1.0):
        m = sign * mids
        g = orc.e4m3_round(m)
        np.testing.assert_array_equal(g, torch_e4m3_codes(m))
        lo = orc.e4m3_round(sign * pos[:-1])
        hi = orc.e4m3_round(sign * pos[1:])
        even = np.where(lo % 2 == 0, lo, hi)
        np.testing.assert_array_equal(g, even)


def test_round_matches_torch_on_bf16_grid(orc):
    """All finite bf16 values within +-448 (they include the subnormal
    range, the subnormal/normal boundary and many ties)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) <= 448)]
    np.testing.assert_array_equal(orc.e4m3_round(v.astype(np.float64)), torch_e4m3_codes(v))


def test_round_random_float32(orc):
    r = np.random.default_rng(3)
    v = np.concatenate([r.uniform(-448, 448, 4000), r.uniform(-1, 1, 4000) * 2.0 ** r.integers(-14, 0, 4000)])
    v = v.astype(np.float32)
    np.testing.assert_array_equal(orc.e4m3_round(v.astype(np.float64)), torch_e4m3_codes(v))


def frexp_exponent(amax):
    """Closed form: amax = m * 2^E with m in [0.5, 1) needs
    e = E - 9 + (m > 0.875), clamped to -127 (448 = 0.875 * 2^9)."""
    if amax == 0:
        return -127
    m, E = math.frexp(amax)
    return max(-127, E - 9 + (1 if m > 0.875 else 0))


def test_block_exponent_closed_forms(orc):
    assert orc.fp8_block_exponent(448.0) == 0
    assert orc.fp8_block_exponent(448.0 * 2 ** 5) == 5
    assert orc.fp8_block_exponent(450.0) == 1          # next bf16 above 448
    assert orc.fp8_block_exponent(224.0) == -1
    assert orc.fp8_block_exponent(1.0) == -8
    assert orc.fp8_block_exponent(0.0) == -127
    assert orc.fp8_block_exponent(2.0 ** -130) == -127
    assert orc.fp8_block_exponent(float(np.finfo(np.float32).max)) == 120
    r = np.random.default_rng(4)
    for a in np.concatenate([r.uniform(0, 10, 300), 2.0 ** r.uniform(-140, 127, 300)]):
        assert orc.fp8_block_exponent(float(a)) == frexp_exponent(float(a)), a


def bf16_rows(r, n, H, wide=False):
    x = r.standard_normal((n, H)).astype(np.float32)
    if wide:  # per-block magnitudes from 2^-135 to 2^120
        x *= (2.0 ** r.integers(-135, 120, size=(n, H // 32, 1))).repeat(32, axis=2).reshape(n, H)
    return synthetic.bf16_bits_from_f32(x)


@pytest.mark.parametrize("wide", [False, True])
def test_quantize_rows_invariants(orc, wide):
    r = np.random.default_rng(5 + wide)
    n, H = 16, 256
    x = bf16_rows(r, n, H, wide)
    x[0, :32] = 0                       # an all-zero block
    x[1, 32:64] = 0x8000                # a block of -0.0
    x[2, 64:96] = 0x0001                # a block of the smallest subnormal
    codes, scales = orc.fp8_quantize_rows(x)
    xv = orc.bf16_to_f64(x).reshape(n, H // 32, 32)
    e = scales.astype(np.int64) - 127
    amax = np.abs(xv).max(axis=2)
    # the scale is minimal: amax fits at e and not at e - 1 (unless e is the floor)
    assert np.all(amax <= 448.0 * np.exp2(e))
    assert np.all((e == -127) | (amax > 448.0 * np.exp2(e - 1)))
    # codes are torch's rounding of x / 2^e (exact in float32 for |x / 2^e| >= 2^-126)
    q = (xv / np.exp2(e)[..., None]).reshape(n, H)
    np.testing.assert_array_equal(codes, torch_e4m3_codes(q))
    assert codes[0, 0] == 0x00 and codes[1, 32] == 0x80
    # decoded error: half a step of E4M3 at the value's binade
    dq = orc.e4m3_value(codes).reshape(n, H // 32, 32) * np.exp2(e)[..., None]
    step = np.where(np.abs(xv) >= np.exp2(e - 6)[..., None],
                    np.exp2(np.floor(np.log2(np.maximum(np.abs(xv), 1e-300))) - 3), np.exp2(e - 9)[..., None])
    assert np.all(np.abs(dq - xv) <= step / 2)


def test_representable_values_round_trip(orc):
    """x = value(code) * 2^e with a block maximum that forces e come back
    bit for bit through quantize and dequantize."""
    r = np.random.default_rng(6)
    codes_all, vals = all_e4m3_values()
    finite = vals[~np.isnan(vals)]
    n, H = 8, 128
    e = r.integers(-100, 100, size=(n, H // 32))
    v = r.choice(finite, size=(n, H // 32, 32))
    v[:, :, 0] = 448.0 * r.choice([-1.0, 1.0], size=(n, H // 32))    # forces the exponent
    x_f64 = (v * np.exp2(e)[..., None]).reshape(n, H)
    x = orc.bf16_round(x_f64)
    np.testing.assert_array_equal(orc.bf16_to_f64(x), x_f64)          # exact in bf16
    codes, scales = orc.fp8_quantize_rows(x)
    np.testing.assert_array_equal(scales.astype(np.int64) - 127, e)
    np.testing.assert_array_equal(orc.fp8_dequant_rows(codes, scales), x)


def test_dequant_matches_definition(orc):
    r = np.random.default_rng(7)
    codes_all, vals = all_e4m3_values()
    ok = codes_all[~np.isnan(vals)]
    n, H = 4, 64
    codes = r.choice(ok, size=(n, H)).astype(np.uint8)
    scales = r.integers(0, 248, size=(n, H // 32)).astype(np.uint8)
    got = orc.fp8_dequant_rows(codes, scales)
    exact = orc.e4m3_value(codes) * np.exp2(scales.astype(np.int64) - 127).repeat(32, axis=1)
    # torch's float64 -> bfloat16 rounding of the exact product
    ref = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_golden_block(orc):
    case = json.load(open(GOLDEN))
    x = orc.bf16_round(np.array([case["x"]], np.float64))
    np.testing.assert_array_equal(orc.bf16_to_f64(x)[0], case["x"])
    codes, scales = orc.fp8_quantize_rows(x)
    assert list(scales[0]) == case["scale_bytes"]
    assert [int(c) for c in codes[0]] == case["codes"]
    np.testing.assert_array_equal(orc.bf16_to_f64(orc.fp8_dequant_rows(codes, scales))[0], case["dequant"])


def test_permute_fp8_is_quantised_permute(orc):
    """Row pos[t][j] holds quantize(x[t]) codes, then scale bytes, then zero
    padding; dropped replicas leave their rows (and rows past N) at the fill."""
    r = np.random.default_rng(8)
    T, H, E, k, R = 40, 96, 8, 3, 2
    x = bf16_rows(r, T, H)
    logits = r.standard_normal((T, E)).astype(np.float32)
    idx, _ = orc.route_topk(logits, None, k)
    L = orc.dispatch_layout(idx, E, R, 12)                         # capacity 12: drops
    N = int(L["expert_offsets"][-1])
    assert N < T * k
    rows = N + 3
    send = orc.dispatch_permute_fp8(x, L["pos"], rows, fill=0xA5)
    rb = orc.fp8_row_bytes(H)
    assert rb == 96 + 128 and send.shape == (rows, rb)
    codes, scales = orc.fp8_quantize_rows(x)
    for t in range(T):
        for j in range(k):
            p = L["pos"][t, j]
            if p >= 0:
                np.testing.assert_array_equal(send[p, :H], codes[t])
                np.testing.assert_array_equal(send[p, H:H + H // 32], scales[t])
    assert np.all(send[:N, H + H // 32:] == 0)
    assert np.all(send[N:] == 0xA5)
    # same rows as quantising the bf16 send buffer
    bf = orc.dispatch_permute(x, L["pos"], N)
    c2, s2 = orc.fp8_quantize_rows(bf)
    np.testing.assert_array_equal(send[:N, :H], c2)
    np.testing.assert_array_equal(send[:N, H:H + H // 32], s2)


def test_rejections(orc):
    with pytest.raises(ValueError):
        orc.fp8_quantize_rows(np.zeros((1, 48), np.uint16))          # H % 32 != 0
    bad = np.zeros((1, 32), np.uint16)
    bad[0, 3] = 0x7F80                                                # +inf
    with pytest.raises(ValueError):
        orc.fp8_quantize_rows(bad)
    with pytest.raises(ValueError):
        orc.e4m3_round([449.0])
    with pytest.raises(ValueError):
        orc.fp8_dequant_rows(np.full((1, 32), 0x7F, np.uint8), np.zeros((1, 1), np.uint8))
