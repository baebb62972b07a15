"""The C ABI library loads, exports what include/moe_ep.h declares, and
rejects bad arguments on the host, before anything touches a GPU.

Only argument-validation paths are called here (no GPU in this container):
each call below fails a check that comes before any HIP call, so the
pointers passed are never dereferenced.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ep.h")


@pytest.fixture(scope="module")
def moe():
    import combine_route_topk_amd
    return combine_route_topk_amd


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(moe):
    declared = _declared_functions()
    assert declared == sorted(moe.EXPORTS)
    raw = ctypes.CDLL(moe.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), name


def test_status_strings(moe):
    for code in range(5):
        assert moe.moe_status_string(code).startswith("MOE_")
    assert "unknown" in moe.moe_status_string(99)


FAKE = 0x10000          # never dereferenced: every call below fails validation first
MIS = 0x10002           # misaligned for 4- and 16-byte requirements


def test_route_validation(moe):
    lib = moe.lib
    assert lib.moe_route_topk(FAKE, None, -1, 8, 2, 1, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route_topk(FAKE, None, 4, 8, 0, 1, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_topk(FAKE, None, 4, 8, 9, 1, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_topk(FAKE, None, 4, 2048, 2, 1, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_topk(FAKE, None, 4, 64, 33, 1, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_topk(FAKE, None, 2 ** 29, 64, 4, 1, FAKE, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_topk(FAKE, None, 4, 8, 2, 6, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route_topk(None, None, 4, 8, 2, 1, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route_topk(MIS, None, 4, 8, 2, 1, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route_topk(FAKE, MIS, 4, 8, 2, 1, FAKE, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    # T = 0 is a no-op that needs no pointers and enqueues nothing
    assert lib.moe_route_topk(None, None, 0, 8, 2, 1, None, None, None) == moe.MOE_OK


def test_grouped_route_validation(moe):
    lib = moe.lib
    g = lambda E=64, k=4, G=8, M=2, T=4, flags=1, lg=FAKE: lib.moe_route_topk_grouped(
        lg, None, T, E, k, G, M, flags, FAKE, FAKE, None)
    assert g(G=6) == moe.MOE_ERR_INVALID_ARG          # E % n_groups != 0
    assert g(G=0) == moe.MOE_ERR_INVALID_ARG
    assert g(M=0) == moe.MOE_ERR_INVALID_ARG
    assert g(M=9) == moe.MOE_ERR_INVALID_ARG          # topk_groups > n_groups
    assert g(k=17, M=2) == moe.MOE_ERR_INVALID_ARG    # k > 2 groups x 8 experts
    assert g(E=256, G=128, M=4, k=4) == moe.MOE_ERR_UNSUPPORTED
    assert g(lg=None) == moe.MOE_ERR_INVALID_ARG
    assert g(flags=4) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route_topk_grouped(None, None, 0, 64, 4, 8, 2, 1, None, None, None) == moe.MOE_OK


def test_workspace_size(moe):
    # one E-wide int32 histogram per tile: tiles of at least 512 assignments
    # (E <= 128) or 1024 (larger E), at most 128 of them; up to 4096
    # assignments (E <= 512) need no workspace
    assert moe.moe_layout_workspace_size(32768, 512, 10, 64) == 128 * 512 * 4
    assert moe.moe_layout_workspace_size(8192, 64, 8, 8) == 128 * 64 * 4
    assert moe.moe_layout_workspace_size(4096, 384, 8, 64) == 32 * 384 * 4
    assert moe.moe_layout_workspace_size(4096, 128, 2, 8) == 16 * 128 * 4
    assert moe.moe_layout_workspace_size(512, 384, 8, 64) == 0
    assert moe.moe_layout_workspace_size(256, 16, 2, 4) == 0
    assert moe.moe_layout_workspace_size(256, 1024, 2, 4) == 1 * 1024 * 4
    assert moe.moe_layout_workspace_size(0, 16, 2, 4) == 0
    with pytest.raises(moe.MoeError):
        moe.moe_layout_workspace_size(256, 16, 2, 3)      # E % R != 0
    with pytest.raises(moe.MoeError):
        moe.moe_layout_workspace_size(256, 16, 17, 4)     # k > E


def _layout(lib, T=256, E=16, k=2, R=4, cap=-1, idx=FAKE, pos=FAKE, ws=FAKE, ws_bytes=1 << 20, out=FAKE):
    return lib.moe_dispatch_layout(idx, T, E, k, R, cap, out, out, out, out, out, pos, None,
                                   ws, ws_bytes, None)


def test_layout_validation(moe):
    lib = moe.lib
    assert _layout(lib, R=3) == moe.MOE_ERR_INVALID_ARG
    assert _layout(lib, R=0) == moe.MOE_ERR_INVALID_ARG
    assert _layout(lib, T=-1) == moe.MOE_ERR_INVALID_ARG
    assert _layout(lib, E=2000, R=1) == moe.MOE_ERR_UNSUPPORTED
    assert _layout(lib, k=40) == moe.MOE_ERR_UNSUPPORTED
    assert _layout(lib, idx=None) == moe.MOE_ERR_INVALID_ARG
    assert _layout(lib, pos=MIS) == moe.MOE_ERR_INVALID_ARG
    assert _layout(lib, out=None) == moe.MOE_ERR_INVALID_ARG
    # 65536 assignments take the tiled layout: 128 tiles x 64 experts x 4 bytes
    big = dict(T=8192, E=64, k=8, R=8)
    assert moe.moe_layout_workspace_size(8192, 64, 8, 8) == 32768
    assert _layout(lib, ws=None, **big) == moe.MOE_ERR_WORKSPACE
    assert _layout(lib, ws_bytes=32767, **big) == moe.MOE_ERR_WORKSPACE
    assert _layout(lib, ws=FAKE + 8, **big) == moe.MOE_ERR_WORKSPACE


def test_permute_and_combine_validation(moe):
    lib = moe.lib
    def perm(x=FAKE, pos=FAKE, T=4, H=16, k=2, E=8, C=-1, send=FAKE, rows=8):
        return lib.moe_dispatch_permute(x, pos, T, H, k, E, C, send, rows, None)

    assert perm(H=12) == moe.MOE_ERR_UNSUPPORTED
    assert perm(rows=-1) == moe.MOE_ERR_INVALID_ARG
    assert perm(x=FAKE + 4) == moe.MOE_ERR_INVALID_ARG
    assert perm(x=None) == moe.MOE_ERR_INVALID_ARG
    assert perm(x=None, pos=None, T=0, send=None, rows=0) == moe.MOE_OK
    assert perm(E=0) == moe.MOE_ERR_UNSUPPORTED
    assert perm(E=1) == moe.MOE_ERR_UNSUPPORTED            # k > E
    assert perm(E=2048) == moe.MOE_ERR_UNSUPPORTED
    # the send buffer must hold the bound on the kept rows: T*k dropless,
    # min(T*k, E*capacity) with a capacity
    assert perm(rows=7) == moe.MOE_ERR_INVALID_ARG
    assert perm(C=0, rows=0, send=None, x=None, pos=None) == moe.MOE_ERR_INVALID_ARG  # pointers still required
    assert perm(T=4096, k=8, E=64, C=100, rows=6399) == moe.MOE_ERR_INVALID_ARG     # bound 6400
    assert perm(T=4096, k=8, E=64, C=1000, rows=32767) == moe.MOE_ERR_INVALID_ARG   # bound T*k
    assert perm(T=2 ** 24, k=2, rows=2 ** 25 - 1) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_reduce(FAKE, 8, FAKE, FAKE, None, None, 4, 16, 2, 2, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_reduce(FAKE, 8, FAKE, FAKE, None, None, 4, 0, 2, 0, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_combine_reduce(FAKE, 8, FAKE, FAKE, MIS, None, 4, 16, 2, 0, FAKE, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_reduce(FAKE, 8, FAKE, FAKE, None, None, 4, 16, 2, 0, None, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_combine_reduce(None, 0, None, None, None, None, 0, 16, 2, 0, None, None) == moe.MOE_OK


def test_regroup_workspace_and_validation(moe):
    lib = moe.lib
    assert moe.moe_recv_regroup_workspace_size(64, 8) == (2 * 64 * 8 + 1) * 4
    assert moe.moe_recv_regroup_workspace_size(1, 1) == 3 * 4
    assert moe.moe_recv_regroup_workspace_size(4, 1024) == (2 * 4096 + 1) * 4
    n = ctypes.c_size_t(0)
    for S, El, want in ((0, 8, moe.MOE_ERR_INVALID_ARG), (8, 0, moe.MOE_ERR_INVALID_ARG),
                        (1025, 1, moe.MOE_ERR_UNSUPPORTED), (1, 1025, moe.MOE_ERR_UNSUPPORTED),
                        (128, 64, moe.MOE_ERR_UNSUPPORTED)):
        assert lib.moe_recv_regroup_workspace_size(S, El, ctypes.byref(n)) == want
    assert lib.moe_recv_regroup_workspace_size(4, 4, None) == moe.MOE_ERR_INVALID_ARG

    ws = (2 * 4 * 4 + 1) * 4

    def layout(S=4, El=4, cnt=FAKE, leo=FAKE, so=FAKE, rp=FAKE, max_rows=64, w=FAKE, wb=ws):
        return lib.moe_recv_regroup_layout(cnt, S, El, leo, so, rp, max_rows, w, wb, None)

    assert layout(S=0) == moe.MOE_ERR_INVALID_ARG
    assert layout(S=2048) == moe.MOE_ERR_UNSUPPORTED
    assert layout(max_rows=-1) == moe.MOE_ERR_INVALID_ARG
    assert layout(max_rows=2 ** 31) == moe.MOE_ERR_UNSUPPORTED
    assert layout(cnt=None) == moe.MOE_ERR_INVALID_ARG
    assert layout(leo=None) == moe.MOE_ERR_INVALID_ARG
    assert layout(so=None) == moe.MOE_ERR_INVALID_ARG
    assert layout(rp=None) == moe.MOE_ERR_INVALID_ARG
    assert layout(cnt=MIS) == moe.MOE_ERR_INVALID_ARG
    assert layout(rp=MIS) == moe.MOE_ERR_INVALID_ARG
    assert layout(w=None) == moe.MOE_ERR_WORKSPACE
    assert layout(wb=ws - 4) == moe.MOE_ERR_WORKSPACE
    assert layout(w=FAKE + 4) == moe.MOE_ERR_WORKSPACE

    for fn in (lib.moe_recv_regroup, lib.moe_recv_ungroup):
        assert fn(FAKE, FAKE, FAKE, 0, 64, FAKE, None) == moe.MOE_OK      # nothing to move
        assert fn(FAKE, FAKE, FAKE, -1, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
        assert fn(FAKE, FAKE, FAKE, 2 ** 31, 64, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
        assert fn(FAKE, FAKE, FAKE, 16, 60, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
        assert fn(FAKE, FAKE, FAKE, 16, 0, FAKE, None) == moe.MOE_ERR_UNSUPPORTED
        assert fn(None, FAKE, FAKE, 16, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
        assert fn(FAKE, None, FAKE, 16, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
        assert fn(FAKE, FAKE, None, 16, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
        assert fn(FAKE, FAKE, FAKE, 16, 64, None, None) == moe.MOE_ERR_INVALID_ARG
        assert fn(FAKE + 8, FAKE, FAKE, 16, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG
        assert fn(FAKE, FAKE, FAKE, 16, 64, FAKE + 8, None) == moe.MOE_ERR_INVALID_ARG
        assert fn(FAKE, MIS, FAKE, 16, 64, FAKE, None) == moe.MOE_ERR_INVALID_ARG


def test_fp8_validation(moe):
    lib = moe.lib
    assert moe.moe_fp8_row_bytes(2048) == 2048 + 128      # one scale line per 4096 values
    assert moe.moe_fp8_row_bytes(4096) == 4096 + 128
    assert moe.moe_fp8_row_bytes(7168) == 7168 + 256
    assert moe.moe_fp8_row_bytes(96) == 96 + 128
    assert moe.moe_fp8_row_bytes(65536) == 65536 + 16 * 128
    import oracle
    for H in (32, 96, 2048, 4096, 4128, 7168, 65536):
        assert moe.moe_fp8_row_bytes(H) == oracle.fp8_row_bytes(H)
    n = ctypes.c_int64(0)
    assert lib.moe_fp8_row_bytes(48, ctypes.byref(n)) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_fp8_row_bytes(0, ctypes.byref(n)) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_fp8_row_bytes(64, None) == moe.MOE_ERR_INVALID_ARG

    def perm(x=FAKE, pos=FAKE, T=16, H=64, k=2, E=8, C=-1, send=FAKE, rows=32):
        return lib.moe_dispatch_permute_fp8(x, pos, T, H, k, E, C, send, rows, None)

    assert perm(T=-1) == moe.MOE_ERR_INVALID_ARG
    assert perm(k=0) == moe.MOE_ERR_UNSUPPORTED
    assert perm(H=48) == moe.MOE_ERR_UNSUPPORTED
    assert perm(H=40) == moe.MOE_ERR_UNSUPPORTED
    assert perm(rows=-1) == moe.MOE_ERR_INVALID_ARG
    assert perm(T=0) == moe.MOE_OK
    assert perm(x=None) == moe.MOE_ERR_INVALID_ARG
    assert perm(pos=None) == moe.MOE_ERR_INVALID_ARG
    assert perm(send=None) == moe.MOE_ERR_INVALID_ARG
    assert perm(x=FAKE + 8) == moe.MOE_ERR_INVALID_ARG
    assert perm(send=FAKE + 8) == moe.MOE_ERR_INVALID_ARG
    assert perm(pos=MIS) == moe.MOE_ERR_INVALID_ARG
    assert perm(rows=31) == moe.MOE_ERR_INVALID_ARG             # bound T*k = 32
    assert perm(C=3, rows=23) == moe.MOE_ERR_INVALID_ARG        # bound E*C = 24
    assert perm(E=1) == moe.MOE_ERR_UNSUPPORTED

    def deq(rows=FAKE, n=FAKE, max_rows=16, H=64, out=FAKE):
        return lib.moe_fp8_dequant(rows, n, max_rows, H, out, None)

    assert deq(max_rows=0) == moe.MOE_OK
    assert deq(max_rows=-1) == moe.MOE_ERR_INVALID_ARG
    assert deq(max_rows=2 ** 31) == moe.MOE_ERR_UNSUPPORTED
    assert deq(H=48) == moe.MOE_ERR_UNSUPPORTED
    assert deq(rows=None) == moe.MOE_ERR_INVALID_ARG
    assert deq(out=None) == moe.MOE_ERR_INVALID_ARG
    assert deq(rows=FAKE + 8) == moe.MOE_ERR_INVALID_ARG
    assert deq(out=FAKE + 8) == moe.MOE_ERR_INVALID_ARG
    assert deq(n=MIS) == moe.MOE_ERR_INVALID_ARG


def test_expert_linear_validation(moe):
    lib = moe.lib
    SE = 64 * 8
    # status, counts, band bound; block rows and band prefix; task prefix; band and task counts
    assert moe.moe_expert_linear_workspace_size(64, 8, 327680) == 4 * (4 + 2 * SE + 1 + 64 + 1 + 2 * (SE + 2560))
    assert moe.moe_expert_linear_workspace_size(4, 4, 0) == 4 * (4 + 32 + 1 + 5 + 2 * 16)
    n = ctypes.c_size_t(0)
    assert lib.moe_expert_linear_workspace_size(0, 4, 10, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_linear_workspace_size(128, 64, 10, ctypes.byref(n)) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_expert_linear_workspace_size(4, 4, -1, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    ws = moe.moe_expert_linear_workspace_size(4, 4, 512)

    def lin(recv=FAKE, cnt=FAKE, S=4, El=4, H=256, H_out=256, W=FAKE, rows=512, y=FAKE, w=FAKE, wb=ws):
        return lib.moe_expert_linear(recv, cnt, S, El, H, H_out, W, rows, y, w, wb, None)

    assert lin(S=0) == moe.MOE_ERR_INVALID_ARG
    assert lin(rows=-1) == moe.MOE_ERR_INVALID_ARG
    assert lin(rows=2 ** 31) == moe.MOE_ERR_UNSUPPORTED
    assert lin(H=96) == moe.MOE_ERR_UNSUPPORTED            # H % 64
    assert lin(H_out=192) == moe.MOE_ERR_UNSUPPORTED       # H_out % 128
    assert lin(H_out=0) == moe.MOE_ERR_UNSUPPORTED
    assert lin(cnt=None) == moe.MOE_ERR_INVALID_ARG
    assert lin(recv=None) == moe.MOE_ERR_INVALID_ARG
    assert lin(W=None) == moe.MOE_ERR_INVALID_ARG
    assert lin(y=None) == moe.MOE_ERR_INVALID_ARG
    assert lin(recv=FAKE + 8) == moe.MOE_ERR_INVALID_ARG
    assert lin(W=FAKE + 8) == moe.MOE_ERR_INVALID_ARG
    assert lin(cnt=MIS) == moe.MOE_ERR_INVALID_ARG
    assert lin(w=None) == moe.MOE_ERR_WORKSPACE
    assert lin(wb=ws - 4) == moe.MOE_ERR_WORKSPACE

    def ret(self_rank=0, consumers=8, group=4, r=FAKE, recv=FAKE, H=256):
        return lib.moe_expert_linear_return(recv, FAKE, 4, 4, H, 256, FAKE, 512, self_rank, consumers,
                                            group, FAKE, r, FAKE, ws, None)

    assert ret(H=96) == moe.MOE_ERR_UNSUPPORTED
    assert ret(recv=None) == moe.MOE_ERR_INVALID_ARG
    assert ret(self_rank=-1) == moe.MOE_ERR_INVALID_ARG
    assert ret(self_rank=4) == moe.MOE_ERR_INVALID_ARG
    assert ret(consumers=-1) == moe.MOE_ERR_INVALID_ARG
    assert ret(group=0) == moe.MOE_ERR_INVALID_ARG
    assert ret(r=None) == moe.MOE_ERR_INVALID_ARG
    assert ret(r=FAKE + 8) == moe.MOE_ERR_INVALID_ARG


def test_route_layout_validation(moe):
    lib = moe.lib
    # the ticket word, then the tiled layout's histograms when there are any
    assert moe.moe_route_dispatch_layout_workspace_size(100, 64, 2, 8) == 16
    assert moe.moe_route_dispatch_layout_workspace_size(8192, 64, 8, 8) == 16 + 32768
    n = ctypes.c_size_t(0)
    assert lib.moe_route_dispatch_layout_workspace_size(4, 16, 2, 3, ctypes.byref(n)) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_route_dispatch_layout_workspace_size(4, 16, 2, 4, None) == moe.MOE_ERR_INVALID_ARG

    def call(lg=FAKE, b=None, T=100, E=64, k=2, flags=1, R=8, C=-1, idx=FAKE, w=FAKE, out=FAKE, pos=FAKE,
             ws=FAKE, wsb=16):
        return lib.moe_route_dispatch_layout(lg, b, T, E, k, flags, R, C, idx, w, out, out, out, out, out, pos,
                                             None, ws, wsb, None)

    assert call(T=-1) == moe.MOE_ERR_INVALID_ARG
    assert call(k=0) == moe.MOE_ERR_UNSUPPORTED
    assert call(k=33, E=64) == moe.MOE_ERR_UNSUPPORTED
    assert call(E=2048) == moe.MOE_ERR_UNSUPPORTED
    assert call(R=3) == moe.MOE_ERR_INVALID_ARG
    assert call(flags=2) == moe.MOE_ERR_INVALID_ARG
    assert call(lg=None) == moe.MOE_ERR_INVALID_ARG
    assert call(idx=None) == moe.MOE_ERR_INVALID_ARG
    assert call(w=None) == moe.MOE_ERR_INVALID_ARG
    assert call(pos=None) == moe.MOE_ERR_INVALID_ARG
    assert call(out=None) == moe.MOE_ERR_INVALID_ARG
    assert call(lg=MIS) == moe.MOE_ERR_INVALID_ARG
    assert call(b=MIS) == moe.MOE_ERR_INVALID_ARG
    assert call(ws=None) == moe.MOE_ERR_WORKSPACE
    assert call(ws=FAKE + 8) == moe.MOE_ERR_WORKSPACE
    assert call(wsb=15) == moe.MOE_ERR_WORKSPACE
    assert call(T=8192, k=8, wsb=16 + 32767) == moe.MOE_ERR_WORKSPACE


def test_floor_validation(moe):
    lib = moe.lib

    def floor(src=FAKE, rb=1024, dst=FAKE, wb=1024, flags=1):
        return lib.moe_hbm_floor(src, rb, dst, wb, flags, None)

    assert floor(rb=-16) == moe.MOE_ERR_INVALID_ARG
    assert floor(wb=-16) == moe.MOE_ERR_INVALID_ARG
    assert floor(rb=1000) == moe.MOE_ERR_INVALID_ARG       # not a multiple of 16
    assert floor(wb=24) == moe.MOE_ERR_INVALID_ARG
    assert floor(flags=2) == moe.MOE_ERR_INVALID_ARG
    assert floor(src=None) == moe.MOE_ERR_INVALID_ARG
    assert floor(dst=FAKE + 8) == moe.MOE_ERR_INVALID_ARG
    assert floor(src=None, rb=0, dst=None, wb=0) == moe.MOE_OK


def test_binding_refuses_host_tensors(moe):
    import torch
    with pytest.raises(ValueError):
        moe.moe_route_topk(torch.zeros(4, 8), None, 2, topk_idx=torch.zeros(4, 2, dtype=torch.int32),
                           topk_w=torch.zeros(4, 2), stream=0)


def test_header_is_c_and_readme_example_compiles(tmp_path):
    """include/moe_ep.h is plain C11, and the call sequence shown in the
    README compiles against it (types and argument order)."""
    import shutil
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    readme = open(os.path.join(root, "README.md")).read()
    block = re.search(r"```c\n(.*?)```", readme, re.S).group(1)
    src = tmp_path / "example.c"
    src.write_text(
        '#include "moe_ep.h"\n'
        "void step(int64_t T, int32_t E, int32_t k, int32_t R, int32_t H, int32_t capacity, int64_t send_rows,\n"
        "          const float *logits, const float *bias, const uint16_t *x, const uint16_t *shared,\n"
        "          const uint16_t *residual, int32_t *topk_idx, float *topk_w, int32_t *expert_demand,\n"
        "          int32_t *expert_counts, int32_t *expert_offsets, int32_t *dest_counts,\n"
        "          int32_t *dest_offsets, int32_t *pos, int32_t *send_src, void *ws, uint16_t *send,\n"
        "          const uint16_t *y, void *out, void *stream)\n{\n" + block + "(void)send;\n}\n")
    r = subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-Wno-unused-parameter",
                        "-I", os.path.join(root, "include"), "-c", str(src), "-o", str(tmp_path / "e.o")],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
