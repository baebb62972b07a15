"""GPU check of the synthetic floor (moe_hbm_floor): it really moves the
bytes it is timed for.

The floor is a diagnostic, not part of the path, and its output contents
are not part of its contract; this test pins them anyway so that a change
that lets the compiler drop its loads or stores (which would make the floor
look faster than the memory system) fails: the first min(read, write) bytes
of dst are a copy of src, written bytes past read_bytes hold the constant
pattern, and nothing past write_bytes is touched. Sizes leave ragged tails
inside and past a 4 KiB tile. Every test prints its case before touching
the GPU.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CANARY = 0xA5
PATTERN = np.frombuffer(np.array([0x3F803F80] * 4, dtype="<u4").tobytes(), dtype=np.uint8)


@pytest.fixture(scope="module")
def moe():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import combine_route_topk_amd
    return combine_route_topk_amd


def say(*a):
    print("[case]", *a, flush=True)


N = 3 * 4096 * 256 + 4096 + 48  # three 1 MiB runs of tiles, one tile, a 48-byte tail


@pytest.mark.parametrize("nt", [True, False], ids=["nt", "plain"])
@pytest.mark.parametrize("read_bytes,write_bytes", [
    (N, N), (N, N // 2 // 16 * 16), (N // 2 // 16 * 16, N), (0, N), (N, 0), (16, 16), (4096 + 16, 48),
])
def test_floor_moves_its_bytes(moe, nt, read_bytes, write_bytes):
    say("floor", "nt" if nt else "plain", "read", read_bytes, "write", write_bytes)
    rng = np.random.default_rng(7)
    src_h = rng.integers(0, 256, size=N + 64, dtype=np.uint8)
    src = torch.from_numpy(src_h).to(DEV)
    dst = torch.full((N + 64,), CANARY, dtype=torch.uint8, device=DEV)
    moe.moe_hbm_floor(src, read_bytes, dst, write_bytes, nt_store=nt)
    torch.cuda.synchronize()
    out = dst.cpu().numpy()
    copied = min(read_bytes, write_bytes)
    assert np.array_equal(out[:copied], src_h[:copied])
    if write_bytes > read_bytes:
        tail = out[read_bytes:write_bytes]
        assert np.array_equal(tail, np.resize(PATTERN, tail.size))
    assert (out[max(write_bytes, 0):] == CANARY).all()
