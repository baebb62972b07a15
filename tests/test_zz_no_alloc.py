"""GPU check of moe_dispatch_layout_noalloc, the layout entry point that
allocates nothing (its tile histograms live in the library's own device
array): called through the C ABI, its outputs must equal moe_dispatch_layout's
(with a caller workspace) bit for bit, on two calls in a row, the second with
a smaller input, so the array holds the first call's histograms when the
second starts. Both are also checked against the oracle."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("expert_demand", "expert_counts", "expert_offsets", "dest_counts", "dest_offsets", "pos", "send_src")


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import combine_route_topk_amd
    return combine_route_topk_amd


def outputs(T, E, k, R):
    i32 = dict(dtype=torch.int32, device=DEV)
    shapes = {"expert_demand": (E,), "expert_counts": (E,), "expert_offsets": (E + 1,), "dest_counts": (R,),
              "dest_offsets": (R + 1,), "pos": (T, k), "send_src": (T * k,)}
    return {n: torch.full(shapes[n], -7, **i32) for n in NAMES}


def run_both(moe, idx, E, R, capacity):
    T, k = idx.shape
    lib = moe.lib
    sp = torch.cuda.current_stream().cuda_stream
    d_idx = torch.from_numpy(idx).to(DEV)
    a = outputs(T, E, k, R)
    print(f"[case] noalloc layout T={T} E={E} k={k} R={R} C={capacity}", flush=True)
    rc = lib.moe_dispatch_layout_noalloc(d_idx.data_ptr(), T, E, k, R, capacity,
                                         *[a[n].data_ptr() for n in NAMES], ctypes.c_void_p(sp))
    assert rc == moe.MOE_OK, moe.moe_status_string(rc)
    b = outputs(T, E, k, R)
    ws = torch.empty(max(moe.moe_layout_workspace_size(T, E, k, R), 16), dtype=torch.uint8, device=DEV)
    rc = lib.moe_dispatch_layout(d_idx.data_ptr(), T, E, k, R, capacity, *[b[n].data_ptr() for n in NAMES],
                                 ws.data_ptr(), ws.numel(), ctypes.c_void_p(sp))
    assert rc == moe.MOE_OK, moe.moe_status_string(rc)
    torch.cuda.synchronize()
    ref = oracle.dispatch_layout(idx, E, R, capacity)
    N = int(ref["expert_offsets"][-1])
    for n in NAMES:
        got_a, got_b = a[n].cpu().numpy(), b[n].cpu().numpy()
        if n == "send_src":
            got_a, got_b, want = got_a[:N], got_b[:N], ref[n][:N]
            assert np.all(a[n].cpu().numpy()[N:] == -7), "send_src past N written"
        else:
            want = ref[n]
        np.testing.assert_array_equal(got_a, got_b, err_msg=n)
        np.testing.assert_array_equal(got_a, want, err_msg=n)
    return N


def test_noalloc_matches_workspace_entry_point(moe):
    """Two calls in a row through the tiled layout (the path that uses the
    array): the fine-grained workload's routing (327,680 assignments, 128
    tiles of 512 experts), then a smaller capacity-limited batch with fewer
    experts; then a one-block-path call, which needs no array at all."""
    w = synthetic.WORKLOADS[5]
    d = synthetic.make_inputs(w, seed=0, with_activations=False)
    idx, _ = oracle.route_topk(d["logits"], d["bias"], w.k)
    assert moe.moe_layout_workspace_size(w.T, w.E, w.k, w.R) > 0
    run_both(moe, idx, w.E, w.R, -1)
    r = np.random.default_rng(7)
    small = np.argsort(r.random((3000, 64)), axis=1)[:, :4].astype(np.int32)   # distinct ids per row
    assert moe.moe_layout_workspace_size(3000, 64, 4, 8) > 0
    run_both(moe, small, 64, 8, 150)
    tiny = np.argsort(r.random((100, 16)), axis=1)[:, :2].astype(np.int32)
    assert moe.moe_layout_workspace_size(100, 16, 2, 4) == 0
    run_both(moe, tiny, 16, 4, -1)


def test_noalloc_rejects_bad_arguments(moe):
    lib = moe.lib
    FAKE = 0x10000
    args = [FAKE] * 7
    assert lib.moe_dispatch_layout_noalloc(FAKE, -1, 16, 2, 4, -1, *args, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_layout_noalloc(FAKE, 8, 16, 2, 3, -1, *args, None) == moe.MOE_ERR_INVALID_ARG
    assert lib.moe_dispatch_layout_noalloc(FAKE, 8, 2048, 2, 4, -1, *args, None) == moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_dispatch_layout_noalloc(None, 8, 16, 2, 4, -1, *args, None) == moe.MOE_ERR_INVALID_ARG
