"""Python face of the plain CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The HIP library and its binding never
import this package, and this package imports nothing from them.

The functions take and return numpy arrays. bf16 tensors are uint16 bit
patterns; gate weights and combined rows are float64. Each function states
the passage it follows in oracle.c, which it calls one-to-one.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB points the wrapper at another build of oracle.c (the mutation
# test uses it to load deliberately broken copies).
LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

GCC_FLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
             "-fno-builtin", "-shared", "-fPIC", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (single-threaded, no SIMD intrinsics)."""
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", *GCC_FLAGS, SRC_PATH, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        lib.oracle_route_topk.argtypes = [P, P, i64, i32, i32, i32, P, P]
        lib.oracle_route_topk_grouped.argtypes = [P, P, i64, i32, i32, i32, i32, i32, P, P]
        lib.oracle_dispatch_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, P]
        lib.oracle_dispatch_permute.argtypes = [P, P, i64, i32, i32, P, i64]
        lib.oracle_recv_regroup_layout.argtypes = [P, i32, i32, P, P, P]
        lib.oracle_scatter_rows.argtypes = [P, P, i64, i32, P, i64]
        lib.oracle_gather_rows.argtypes = [P, i64, P, i64, i32, P]
        lib.oracle_combine_reduce.argtypes = [P, i64, P, P, P, P, i64, i32, i32, P, i64, P]
        lib.oracle_bf16_round.argtypes = [ctypes.c_double]
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_bf16_round_array.argtypes = [P, i64, P]
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_round.argtypes = [ctypes.c_double]
        lib.oracle_fp8_block_exponent.argtypes = [ctypes.c_double]
        lib.oracle_fp8_quantize_rows.argtypes = [P, i64, i32, P, P]
        lib.oracle_fp8_dequant_rows.argtypes = [P, P, i64, i32, P]
        lib.oracle_dispatch_permute_fp8.argtypes = [P, P, i64, i32, i32, P, i64, i64]
        lib.oracle_expert_linear.argtypes = [P, P, i32, i32, i32, i32, P, P]
        for f in ("oracle_route_topk", "oracle_route_topk_grouped", "oracle_dispatch_layout",
                  "oracle_dispatch_permute", "oracle_combine_reduce", "oracle_recv_regroup_layout",
                  "oracle_scatter_rows", "oracle_gather_rows", "oracle_e4m3_round",
                  "oracle_fp8_block_exponent", "oracle_fp8_quantize_rows", "oracle_fp8_dequant_rows",
                  "oracle_dispatch_permute_fp8", "oracle_expert_linear"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def route_topk(logits: np.ndarray, bias: Optional[np.ndarray], k: int,
               normalize: bool = True):
    """Top-k experts per token (ties to the lower id, descending order) and
    float64 gate weights from the unbiased logits; see oracle_route_topk."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    bias = None if bias is None else _c(bias, np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    rc = _load().oracle_route_topk(_ptr(logits), _ptr(bias), T, E, k,
                                   1 if normalize else 0, _ptr(idx), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_route_topk rejected its arguments")
    return idx, w


def route_topk_grouped(logits: np.ndarray, bias: Optional[np.ndarray], k: int,
                       n_groups: int, topk_groups: int, normalize: bool = True):
    """Group-limited top-k: the best topk_groups expert groups (ranked by their
    best score), then the top k experts inside them; see
    oracle_route_topk_grouped."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    bias = None if bias is None else _c(bias, np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    rc = _load().oracle_route_topk_grouped(_ptr(logits), _ptr(bias), T, E, k, n_groups,
                                           topk_groups, 1 if normalize else 0, _ptr(idx), _ptr(w))
    if rc != 0:
        raise ValueError("oracle_route_topk_grouped rejected its arguments")
    return idx, w


def dispatch_layout(topk_idx: np.ndarray, E: int, R: int, capacity: int = -1,
                    with_send_src: bool = True) -> dict:
    """Counts, offsets, token-order capacity drops and send positions; see
    oracle_dispatch_layout."""
    topk_idx = _c(topk_idx, np.int32)
    T, k = topk_idx.shape
    out = {
        "expert_demand": np.empty(E, np.int32),
        "expert_counts": np.empty(E, np.int32),
        "expert_offsets": np.empty(E + 1, np.int32),
        "dest_counts": np.empty(R, np.int32),
        "dest_offsets": np.empty(R + 1, np.int32),
        "pos": np.empty((T, k), np.int32),
        "send_src": np.full(T * k, -1, np.int32) if with_send_src else None,
    }
    rc = _load().oracle_dispatch_layout(
        _ptr(topk_idx), T, E, k, R, capacity,
        _ptr(out["expert_demand"]), _ptr(out["expert_counts"]),
        _ptr(out["expert_offsets"]), _ptr(out["dest_counts"]),
        _ptr(out["dest_offsets"]), _ptr(out["pos"]), _ptr(out["send_src"]))
    if rc != 0:
        raise ValueError("oracle_dispatch_layout rejected its arguments")
    return out


def dispatch_permute(x: np.ndarray, pos: np.ndarray, send_rows: int,
                     fill: int = 0) -> np.ndarray:
    """send[pos[t, j]] = x[t] for kept replicas; other rows hold `fill`."""
    x = _c(x, np.uint16)
    pos = _c(pos, np.int32)
    T, H = x.shape
    k = pos.shape[1]
    send = np.full((send_rows, H), fill, np.uint16)
    rc = _load().oracle_dispatch_permute(_ptr(x), _ptr(pos), T, H, k, _ptr(send), send_rows)
    if rc != 0:
        raise ValueError("oracle_dispatch_permute: position outside the send buffer")
    return send


def recv_regroup_layout(cnt: np.ndarray) -> dict:
    """Expert-major layout of a source-major receive buffer with cnt[s][l]
    rows of local expert l from source s; see oracle_recv_regroup_layout."""
    cnt = _c(cnt, np.int32)
    S, El = cnt.shape
    N = int(cnt.sum())
    out = {"local_expert_offsets": np.empty(El + 1, np.int32),
           "source_offsets": np.empty(S + 1, np.int32),
           "recv_pos": np.empty(N, np.int32)}
    rc = _load().oracle_recv_regroup_layout(_ptr(cnt), S, El, _ptr(out["local_expert_offsets"]),
                                            _ptr(out["source_offsets"]), _ptr(out["recv_pos"]))
    if rc != 0:
        raise ValueError("oracle_recv_regroup_layout rejected its arguments")
    return out


def scatter_rows(src: np.ndarray, row_map: np.ndarray, dst_rows: int, fill: int = 0) -> np.ndarray:
    """dst[row_map[i]] = src[i]; rows no entry points at hold `fill`."""
    src = _c(src, np.uint16)
    row_map = _c(row_map, np.int32)
    n, H = src.shape
    dst = np.full((dst_rows, H), fill, np.uint16)
    if _load().oracle_scatter_rows(_ptr(src), _ptr(row_map), n, H, _ptr(dst), dst_rows) != 0:
        raise ValueError("oracle_scatter_rows: target row out of range")
    return dst


def gather_rows(src: np.ndarray, row_map: np.ndarray) -> np.ndarray:
    """dst[i] = src[row_map[i]]."""
    src = _c(src, np.uint16)
    row_map = _c(row_map, np.int32)
    H = src.shape[1]
    dst = np.empty((row_map.shape[0], H), np.uint16)
    if _load().oracle_gather_rows(_ptr(src), src.shape[0], _ptr(row_map), row_map.shape[0], H,
                                  _ptr(dst)) != 0:
        raise ValueError("oracle_gather_rows: source row out of range")
    return dst


def combine_reduce(y: np.ndarray, pos: np.ndarray, w: np.ndarray,
                   shared: Optional[np.ndarray], residual: Optional[np.ndarray],
                   tokens: Optional[np.ndarray] = None) -> np.ndarray:
    """float64 gate-weighted sum over kept replicas + shared + residual; see
    oracle_combine_reduce. With `tokens`, only those rows are computed."""
    y = _c(y, np.uint16)
    pos = _c(pos, np.int32)
    w = _c(w, np.float64)
    T, k = pos.shape
    H = y.shape[1]
    shared = None if shared is None else _c(shared, np.uint16)
    residual = None if residual is None else _c(residual, np.uint16)
    tok = None if tokens is None else _c(tokens, np.int64)
    rows = T if tok is None else tok.shape[0]
    out = np.empty((rows, H), np.float64)
    rc = _load().oracle_combine_reduce(
        _ptr(y), y.shape[0], _ptr(pos), _ptr(w), _ptr(shared), _ptr(residual),
        T, H, k, _ptr(tok), rows, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_combine_reduce rejected its arguments")
    return out


def bf16_round(a) -> np.ndarray:
    """Nearest bf16 (ties to even) of each float64 value, as uint16 bits."""
    a = _c(a, np.float64)
    out = np.empty(a.shape, np.uint16)
    _load().oracle_bf16_round_array(_ptr(a), a.size, _ptr(out))
    return out


def bf16_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns as float64."""
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# FP8 dispatch payload (E4M3 codes, one power-of-two scale byte per 32 values)
# ---------------------------------------------------------------------------

def e4m3_value(codes) -> np.ndarray:
    """Value of each E4M3 code (NaN for the NaN codes); oracle_e4m3_value."""
    c = np.asarray(codes, np.uint8)
    f = _load().oracle_e4m3_value
    return np.array([f(int(v)) for v in c.ravel()], np.float64).reshape(c.shape)


def e4m3_round(values) -> np.ndarray:
    """Nearest E4M3 code of each value (|v| <= 448), ties to even; oracle_e4m3_round."""
    v = np.asarray(values, np.float64)
    f = _load().oracle_e4m3_round
    out = np.array([f(float(a)) for a in v.ravel()], np.int32)
    if np.any(out < 0):
        raise ValueError("oracle_e4m3_round: value outside the E4M3 range or NaN")
    return out.astype(np.uint8).reshape(v.shape)


def fp8_block_exponent(amax: float) -> int:
    """Smallest e >= -127 with amax <= 448 * 2^e; oracle_fp8_block_exponent."""
    return int(_load().oracle_fp8_block_exponent(float(amax)))


def fp8_quantize_rows(x: np.ndarray):
    """(codes [n, H] uint8, scale bytes [n, H/32] uint8) of bf16 rows x [n, H]."""
    x = _c(x, np.uint16)
    n, H = x.shape
    codes = np.empty((n, H), np.uint8)
    scales = np.empty((n, max(H // 32, 1)), np.uint8)
    if _load().oracle_fp8_quantize_rows(_ptr(x), n, H, _ptr(codes), _ptr(scales)) != 0:
        raise ValueError("oracle_fp8_quantize_rows: H % 32 != 0 or a non-finite value")
    return codes, scales


def fp8_dequant_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """bf16 bits of value(code) * 2^(scale - 127), ties to even."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    n, H = codes.shape
    out = np.empty((n, H), np.uint16)
    if _load().oracle_fp8_dequant_rows(_ptr(codes), _ptr(scales), n, H, _ptr(out)) != 0:
        raise ValueError("oracle_fp8_dequant_rows: H % 32 != 0 or a NaN code")
    return out


def fp8_row_bytes(H: int) -> int:
    """Bytes of one FP8 send row: H codes, then one 128-byte line per 4096
    values holding that slab's 128 scale bytes (zero-padded in the last)."""
    return H + 128 * ((H + 4095) // 4096)


def dispatch_permute_fp8(x: np.ndarray, pos: np.ndarray, send_rows: int, row_bytes: Optional[int] = None,
                         fill: int = 0) -> np.ndarray:
    """FP8 send buffer [send_rows, row_bytes] uint8: row pos[t][j] holds the
    codes, the scale bytes and zero padding of x[t]; other rows hold `fill`."""
    x = _c(x, np.uint16)
    pos = _c(pos, np.int32)
    T, H = x.shape
    k = pos.shape[1]
    rb = fp8_row_bytes(H) if row_bytes is None else row_bytes
    send = np.full((send_rows, rb), fill, np.uint8)
    if _load().oracle_dispatch_permute_fp8(_ptr(x), _ptr(pos), T, H, k, _ptr(send), send_rows, rb) != 0:
        raise ValueError("oracle_dispatch_permute_fp8 rejected its arguments")
    return send


# ---------------------------------------------------------------------------
# tile-signalled return: stand-in expert computation
# ---------------------------------------------------------------------------

def expert_linear(recv: np.ndarray, cnt: np.ndarray, W: np.ndarray) -> np.ndarray:
    """y [N, H_out] bf16 bits: each received row times its local expert's
    W[l] ([H_out, H]), summed in float64 and rounded once to bf16."""
    recv = _c(recv, np.uint16)
    cnt = _c(cnt, np.int32)
    W = _c(W, np.uint16)
    S, El = cnt.shape
    N = int(cnt.sum())
    H = recv.shape[1]
    H_out = W.shape[1]
    assert W.shape == (El, H_out, H) and recv.shape[0] >= N
    y = np.empty((N, H_out), np.uint16)
    if _load().oracle_expert_linear(_ptr(recv), _ptr(cnt), S, El, H, H_out, _ptr(W), _ptr(y)) != 0:
        raise ValueError("oracle_expert_linear rejected its arguments")
    return y
