"""Property-based pins for the oracle (hypothesis draws the inputs).

Every property states a definition written independently of the oracle:
brute-force enumeration of selections, Python sorting, exact rational
arithmetic (fractions.Fraction) for the roundings and the weighted sum, and
plain loops for the layouts. Hypothesis searches tiny shapes and awkward
values (subnormals, signed zeros, infinities, NaN, exact ties) that fixed
seeds rarely reach, and shrinks any failure to a minimal case.

Sources: ai-from-scratch "19. All-to-all" (intro: each token names k expert
ids; "Why the router can ruin your day": the balancing bias only selects;
"DeepSeek's numbers": at most a few nodes per token), aicassindra
"gpu_moe_all_to_all" ("Two collectives per layer": rows leave grouped by
destination and come back to be summed with their gate weights; "Capacity
factor": replicas past an expert's capacity are dropped).
"""

import bisect
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

SETTINGS = settings(max_examples=150, deadline=None, database=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])

F32 = st.floats(width=32, allow_nan=True, allow_infinity=True)
SPECIAL = st.sampled_from([math.nan, math.inf, -math.inf, 0.0, -0.0, 1.0, -1.0])


# ---------------------------------------------------------------------------
# top-k selection
# ---------------------------------------------------------------------------

def _better(a, b):
    """(value, id) pair a ranks before b: numbers above NaN, larger first,
    then the lower id."""
    (va, ea), (vb, eb) = a, b
    if math.isnan(va) != math.isnan(vb):
        return math.isnan(vb)
    if not math.isnan(va) and va != vb:
        return va > vb
    return ea < eb


def _brute_topk(s, allowed, k):
    """The ordered k-tuple of distinct allowed experts whose first member
    ranks before every other allowed expert, the second before every other
    remaining one, and so on; found by trying every ordered tuple."""
    for tup in itertools.permutations(allowed, k):
        ok = True
        rest = set(allowed)
        for e in tup:
            rest.discard(e)
            if any(_better((float(s[o]), o), (float(s[e]), e)) for o in rest):
                ok = False
                break
        if ok:
            return list(tup)
    raise AssertionError("no ordered tuple satisfies the selection rule")


@st.composite
def route_case(draw, grouped=False):
    if grouped:
        G = draw(st.sampled_from([1, 2, 3]))
        gs = draw(st.integers(1, 3))
        E = G * gs
        M = draw(st.integers(1, G))
        k = draw(st.integers(1, min(M * gs, 3)))
    else:
        E = draw(st.integers(1, 6))
        k = draw(st.integers(1, min(E, 3)))
        G = M = 0
    T = draw(st.integers(1, 4))
    # a small pool makes exact ties likely; F32 reaches subnormals and specials
    pool = draw(st.lists(st.one_of(SPECIAL, F32), min_size=1, max_size=4))
    logits = np.array([[draw(st.sampled_from(pool)) for _ in range(E)] for _ in range(T)], np.float32)
    bias = None
    if draw(st.booleans()):
        bias = np.array([draw(st.floats(-2, 2, width=32)) for _ in range(E)], np.float32)
    return logits, bias, k, G, M


@SETTINGS
@given(route_case())
def test_route_selection_property(orc, case):
    logits, bias, k, _, _ = case
    T, E = logits.shape
    idx, w = orc.route_topk(logits, bias, k)
    for t in range(T):
        s = logits[t] if bias is None else (logits[t] + bias).astype(np.float32)
        assert list(idx[t]) == _brute_topk(s, list(range(E)), k)
        if np.all(np.isfinite(logits[t])):
            # softmax over the chosen unbiased logits, exact up to float64 rounding
            z = logits[t].astype(np.float64)[idx[t]]
            ref = np.exp(z - z.max())
            np.testing.assert_allclose(w[t], ref / ref.sum(), rtol=1e-12, atol=0)
            assert abs(w[t].sum() - 1.0) <= 4 * k * 2.0 ** -52


@SETTINGS
@given(route_case(grouped=True))
def test_grouped_route_property(orc, case):
    logits, bias, k, G, M = case
    T, E = logits.shape
    gs = E // G
    idx, w = orc.route_topk_grouped(logits, bias, k, G, M)
    for t in range(T):
        s = logits[t] if bias is None else (logits[t] + bias).astype(np.float32)
        # a group ranks by its best member; keep the M best groups
        best = [_brute_topk(s, list(range(g * gs, (g + 1) * gs)), 1)[0] for g in range(G)]
        order = _brute_topk({g: s[best[g]] for g in range(G)}, list(range(G)), G)
        # equal best scores: the group holding the lower expert id first,
        # which is the lower group id since groups are contiguous
        groups = set(order[:M])
        allowed = [e for e in range(E) if e // gs in groups]
        assert list(idx[t]) == _brute_topk(s, allowed, k)
        if np.all(np.isfinite(logits[t])):
            # gate weights come from the unbiased logits of the chosen experts
            z = logits[t].astype(np.float64)[idx[t]]
            ref = np.exp(z - z.max())
            np.testing.assert_allclose(w[t], ref / ref.sum(), rtol=1e-12, atol=0)


# ---------------------------------------------------------------------------
# dispatch layout with capacity
# ---------------------------------------------------------------------------

@st.composite
def layout_case(draw):
    R = draw(st.integers(1, 3))
    El = draw(st.integers(1, 3))
    E = R * El
    k = draw(st.integers(1, min(E, 3)))
    T = draw(st.integers(0, 8))
    idx = np.array([draw(st.permutations(range(E)))[:k] for _ in range(T)], np.int32).reshape(T, k)
    C = draw(st.integers(-1, T))
    return idx, E, R, C


@SETTINGS
@given(layout_case())
def test_layout_property(orc, case):
    idx, E, R, C = case
    T, k = idx.shape
    L = orc.dispatch_layout(idx, E, R, C)
    # token order decides who keeps a slot: walk the replicas in (t, j) order
    seen = [0] * E
    kept = [[] for _ in range(E)]          # (t, j) of the replicas each expert keeps
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if C < 0 or seen[e] < C:
                kept[e].append((t, j))
            seen[e] += 1
    assert list(L["expert_demand"]) == seen
    assert list(L["expert_counts"]) == [len(v) for v in kept]
    start, pos = 0, -np.ones((T, k), np.int64)
    for e in range(E):                     # send rows: expert-major, token order inside
        assert L["expert_offsets"][e] == start
        for n, (t, j) in enumerate(kept[e]):
            pos[t, j] = start + n
        start += len(kept[e])
    assert L["expert_offsets"][E] == start
    np.testing.assert_array_equal(L["pos"], pos)
    El = E // R
    for r in range(R + 1):                 # rank r owns experts r*El .. r*El+El-1
        assert L["dest_offsets"][r] == L["expert_offsets"][r * El]
    for r in range(R):
        assert L["dest_counts"][r] == L["dest_offsets"][r + 1] - L["dest_offsets"][r]
    src = L["send_src"][:start]
    for t in range(T):
        for j in range(k):
            if pos[t, j] >= 0:
                assert src[pos[t, j]] == t


# ---------------------------------------------------------------------------
# receive-side regroup
# ---------------------------------------------------------------------------

@SETTINGS
@given(st.integers(1, 4).flatmap(lambda S: st.integers(1, 4).flatmap(
    lambda El: st.lists(st.integers(0, 4), min_size=S * El, max_size=S * El).map(
        lambda v: np.array(v, np.int32).reshape(S, El)))))
def test_regroup_property(orc, cnt):
    S, El = cnt.shape
    L = orc.recv_regroup_layout(cnt)
    N = int(cnt.sum())
    # expert-major destination: expert l's block lists source 0's rows, then source 1's, ...
    dest = []
    for s in range(S):
        for l in range(El):
            for i in range(int(cnt[s, l])):
                dest.append(int(cnt[:, :l].sum()) + int(cnt[:s, l].sum()) + i)
    np.testing.assert_array_equal(L["recv_pos"], np.array(dest, np.int32).reshape(N))
    assert list(L["local_expert_offsets"]) == [int(cnt[:, :l].sum()) for l in range(El + 1)]
    assert list(L["source_offsets"]) == [int(cnt[:s].sum()) for s in range(S + 1)]
    # the scatter is a bijection: gathering with the same map restores the rows
    src = np.arange(N * 2, dtype=np.uint16).reshape(N, 2)
    back = orc.gather_rows(orc.scatter_rows(src, L["recv_pos"], N), L["recv_pos"])
    np.testing.assert_array_equal(back, src)


# ---------------------------------------------------------------------------
# combine: exact rational reference
# ---------------------------------------------------------------------------

BF16_BITS = st.integers(0, 0xFFFF).filter(lambda b: (b & 0x7F80) != 0x7F80)   # finite


@st.composite
def combine_case(draw):
    T = draw(st.integers(1, 3))
    k = draw(st.integers(1, 3))
    H = draw(st.integers(1, 3))
    rows = draw(st.integers(1, 6))
    y = np.array(draw(st.lists(BF16_BITS, min_size=rows * H, max_size=rows * H)), np.uint16).reshape(rows, H)
    pos = np.array(draw(st.lists(st.integers(-1, rows - 1), min_size=T * k, max_size=T * k)),
                   np.int32).reshape(T, k)
    w = np.array(draw(st.lists(st.floats(0, 1), min_size=T * k, max_size=T * k)), np.float64).reshape(T, k)
    extra = lambda: (np.array(draw(st.lists(BF16_BITS, min_size=T * H, max_size=T * H)), np.uint16)
                     .reshape(T, H) if draw(st.booleans()) else None)
    return y, pos, w, extra(), extra()


def _bf16_exact(b):
    return Fraction(float(np.array([int(b) << 16], np.uint32).view(np.float32)[0]))


@SETTINGS
@given(combine_case())
def test_combine_exact_sum_property(orc, case):
    y, pos, w, shared, residual = case
    T, k = pos.shape
    H = y.shape[1]
    out = orc.combine_reduce(y, pos, w, shared, residual)
    for t in range(T):
        for h in range(H):
            terms = [Fraction(float(w[t, j])) * _bf16_exact(y[pos[t, j], h]) for j in range(k) if pos[t, j] >= 0]
            terms += [_bf16_exact(a[t, h]) for a in (shared, residual) if a is not None]
            exact = sum(terms, Fraction(0))
            # k products and up to k+1 additions, each rounded once in float64;
            # a product that underflows is off by at most half the smallest
            # subnormal, 2^-1075 (additions of subnormals are exact)
            bound = (Fraction((2 * k + 2) * 2.0 ** -53) * sum((abs(x) for x in terms), Fraction(0))
                     + k * Fraction(2) ** -1075)
            assert abs(Fraction(float(out[t, h])) - exact) <= bound, (t, h, terms)


# ---------------------------------------------------------------------------
# roundings: nearest, ties to even, against exact enumeration
# ---------------------------------------------------------------------------

def _nearest_even(v, candidates):
    """candidates: list of (exact value, code) sorted by value; the nearest
    to v, a tie going to the code with an even last mantissa bit."""
    fv = Fraction(v)
    best = min(abs(c[0] - fv) for c in candidates)
    near = [c for c in candidates if abs(c[0] - fv) == best]
    if len(near) == 1:
        return near
    return [c for c in near if c[1] % 2 == 0]


def _e4m3_table():
    tab = []
    for c in range(256):
        s, ex, m = c >> 7, (c >> 3) & 15, c & 7
        if ex == 15 and m == 7:
            continue                               # the NaN codes
        mag = Fraction(m, 8) * Fraction(2) ** -6 if ex == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (ex - 7)
        tab.append((-mag if s else mag, c))
    return tab


E4M3 = _e4m3_table()
E4M3_VALUE = {c: v for v, c in E4M3}
E4M3_SORTED = sorted(E4M3)


def _e4m3_nearby(q):
    """The table entries around q (both zeros included near zero): enough
    for the nearest-value search, far cheaper than the whole table."""
    i = bisect.bisect_left(E4M3_SORTED, (q, -1))
    return E4M3_SORTED[max(i - 3, 0):i + 3]


# exact midpoints between neighbouring codes, where the tie rule decides
E4M3_MIDPOINTS = sorted({float((a[0] + b[0]) / 2) for a, b in zip(E4M3_SORTED, E4M3_SORTED[1:])
                         if a[0] != b[0]})


@SETTINGS
@given(st.one_of(st.floats(-448, 448, allow_subnormal=True), st.sampled_from(E4M3_MIDPOINTS)))
def test_e4m3_round_nearest_even_property(orc, v):
    code = int(orc.e4m3_round(np.array([v]))[0])
    want = _nearest_even(v, E4M3)
    if v == 0 or all(c[0] == 0 for c in want):
        # zero keeps the sign of the value it came from
        assert code in (0x00, 0x80) and (code == 0x80) == (math.copysign(1, v) < 0)
    else:
        assert code in [c[1] for c in want], (v, code, want)


def _bf16_neighbours(v):
    """The two bf16 values that bracket v (as exact fractions with their bit
    patterns), from the float32 grid: bf16 is float32 with 16 low bits zero."""
    f = np.array([v], np.float64).astype(np.float32)
    b = int(f.view(np.uint32)[0]) & 0xFFFF0000
    out = []
    for d in (-0x10000, 0, 0x10000, 0x20000):
        u = (b + d) & 0xFFFFFFFF
        x = float(np.array([u], np.uint32).view(np.float32)[0])
        if math.isfinite(x):
            out.append((Fraction(x), u >> 16))
    return out


MAX_BF16 = float(np.array([0x7F7F0000], np.uint32).view(np.float32)[0])


@SETTINGS
@given(st.floats(-MAX_BF16, MAX_BF16, allow_subnormal=True))
def test_bf16_round_nearest_even_property(orc, v):
    got = int(orc.bf16_round(np.array([v]))[0])
    cands = _bf16_neighbours(v)
    want = _nearest_even(v, cands)
    if all(c[0] == 0 for c in want):
        assert got in (0x0000, 0x8000) and (got == 0x8000) == (math.copysign(1, v) < 0)
    else:
        assert got in [c[1] for c in want], (v, hex(got), want)


@pytest.mark.parametrize("v,bits", [(MAX_BF16, 0x7F7F), (-MAX_BF16, 0xFF7F), (math.inf, 0x7F80),
                                    (2.0 ** 128, 0x7F80), (2.0 ** -133, 0x0001), (2.0 ** -134, 0x0000),
                                    (3 * 2.0 ** -134, 0x0002), (3 * 2.0 ** -135, 0x0001)])
def test_bf16_round_edges(orc, v, bits):
    # the largest finite bf16 is (2 - 2^-7) * 2^127; 2^128 lies past its half
    # step and overflows; the smallest subnormal is 2^-133, its half ties to
    # zero (even), 1.5 times it rounds to 2^-132 (even) and 0.75 times it
    # rounds up to it
    assert int(orc.bf16_round(np.array([v]))[0]) == bits


# ---------------------------------------------------------------------------
# dispatch permute (bf16 and FP8 payloads)
# ---------------------------------------------------------------------------

@st.composite
def permute_case(draw, H_choices=(1, 2, 5)):
    T = draw(st.integers(1, 4))
    k = draw(st.integers(1, 3))
    H = draw(st.sampled_from(H_choices))
    # distinct send rows for the kept replicas, -1 for the dropped ones
    rows = draw(st.integers(T * k, T * k + 3))
    slots = draw(st.permutations(range(rows)))[:T * k]
    drop = draw(st.lists(st.booleans(), min_size=T * k, max_size=T * k))
    pos = np.array([-1 if d else p for p, d in zip(slots, drop)], np.int32).reshape(T, k)
    x = np.array(draw(st.lists(BF16_BITS, min_size=T * H, max_size=T * H)), np.uint16).reshape(T, H)
    return x, pos, rows


@SETTINGS
@given(permute_case(), st.integers(0, 0xFFFF))
def test_permute_property(orc, case, fill):
    x, pos, rows = case
    send = orc.dispatch_permute(x, pos, rows, fill)
    want = np.full((rows, x.shape[1]), fill, np.uint16)
    for t, j in zip(*np.nonzero(pos >= 0)):
        want[pos[t, j]] = x[t]
    np.testing.assert_array_equal(send, want)


def _bf16_of_bits(b):
    return Fraction(float(np.array([int(b) << 16], np.uint32).view(np.float32)[0]))


@st.composite
def fp8_rows(draw):
    """bf16 rows of whole 32-value blocks; some blocks are E4M3 grid values
    times a power of two, so that a block maximum can sit exactly on 448 * 2^e."""
    n = draw(st.integers(1, 2))
    nb = draw(st.integers(1, 2))
    out = []
    for _ in range(n * nb):
        if draw(st.booleans()):
            out += draw(st.lists(BF16_BITS, min_size=32, max_size=32))
        else:
            e = draw(st.integers(-120, 120))
            vals = draw(st.lists(st.sampled_from([v for v, _ in E4M3]), min_size=32, max_size=32))
            f = np.array([float(v * Fraction(2) ** e) for v in vals], np.float32)   # exact in bf16
            out += list((f.view(np.uint32) >> 16).astype(np.int64))
    return np.array(out, np.uint16).reshape(n, nb * 32)


@SETTINGS
@given(fp8_rows())
def test_fp8_quantize_property(orc, x):
    n, H = x.shape
    codes, scales = orc.fp8_quantize_rows(x)
    deq = orc.fp8_dequant_rows(codes, scales)
    for r in range(n):
        for b in range(H // 32):
            v = [_bf16_of_bits(x[r, b * 32 + i]) for i in range(32)]
            amax = max(abs(a) for a in v)
            e = int(scales[r, b]) - 127
            # the smallest e >= -127 whose range 448 * 2^e holds the block
            assert amax <= 448 * Fraction(2) ** e
            assert e == -127 or amax > 448 * Fraction(2) ** (e - 1)
            for i in range(32):
                c = int(codes[r, b * 32 + i])
                q = v[i] / Fraction(2) ** e
                want = _nearest_even(q, _e4m3_nearby(q))
                if all(a[0] == 0 for a in want):
                    neg = (int(x[r, b * 32 + i]) >> 15) == 1
                    assert c == (0x80 if neg else 0x00)
                else:
                    assert c in [a[1] for a in want], (r, b, i, q, c)
                # decode: the bf16 nearest to value(code) * 2^e
                val = E4M3_VALUE[c] * Fraction(2) ** e
                got = int(deq[r, b * 32 + i])
                if val == 0:
                    assert got & 0x7FFF == 0
                else:
                    assert got in [a[1] for a in _nearest_even(val, _bf16_neighbours(float(val)))]


@SETTINGS
@given(permute_case(H_choices=(32, 64)), st.integers(0, 255))
def test_fp8_permute_property(orc, case, fill):
    x, pos, rows = case
    H = x.shape[1]
    rb = orc.fp8_row_bytes(H)
    send = orc.dispatch_permute_fp8(x, pos, rows, fill=fill)
    codes, scales = orc.fp8_quantize_rows(x)
    want = np.full((rows, rb), fill, np.uint8)
    for t, j in zip(*np.nonzero(pos >= 0)):
        # codes, then the block scale bytes, then zero padding
        want[pos[t, j]] = np.concatenate([codes[t], scales[t], np.zeros(rb - H - H // 32, np.uint8)])
    np.testing.assert_array_equal(send, want)


# ---------------------------------------------------------------------------
# stand-in expert linear map
# ---------------------------------------------------------------------------

# bf16 values with exponents in [-8, 8]: products carry 16 significant bits
# over 32 binades, so a sum of up to 8 of them is exact in float64 and the
# one rounding left is the final one to bf16
BF16_NARROW = st.tuples(st.integers(0, 1), st.integers(127 - 8, 127 + 8), st.integers(0, 127)).map(
    lambda t: (t[0] << 15) | (t[1] << 7) | t[2]) | st.just(0)


@SETTINGS
@given(st.integers(1, 2), st.integers(1, 3), st.integers(1, 8), st.integers(1, 3), st.data())
def test_expert_linear_property(orc, S, El, H, H_out, data):
    cnt = np.array(data.draw(st.lists(st.integers(0, 2), min_size=S * El, max_size=S * El)),
                   np.int32).reshape(S, El)
    N = int(cnt.sum())
    recv = np.array(data.draw(st.lists(BF16_NARROW, min_size=N * H, max_size=N * H)), np.uint16).reshape(N, H)
    W = np.array(data.draw(st.lists(BF16_NARROW, min_size=El * H_out * H, max_size=El * H_out * H)),
                 np.uint16).reshape(El, H_out, H)
    y = orc.expert_linear(recv, cnt, W)
    # received rows are source-major: source s's rows for expert 0, then expert 1, ...
    experts = [l for s in range(S) for l in range(El) for _ in range(int(cnt[s, l]))]
    for n, l in enumerate(experts):
        for o in range(H_out):
            acc = sum((_bf16_of_bits(recv[n, h]) * _bf16_of_bits(W[l, o, h]) for h in range(H)), Fraction(0))
            got = int(y[n, o])
            if acc == 0:
                assert got & 0x7FFF == 0
            else:
                assert got in [a[1] for a in _nearest_even(acc, _bf16_neighbours(float(acc)))], (n, o)
