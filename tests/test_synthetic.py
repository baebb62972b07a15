"""The seeded workload generator: shapes, determinism, the capacity reading."""

import numpy as np

import synthetic


def test_workload_shapes_and_capacity():
    w = synthetic.WORKLOADS
    assert [(v.T, v.H, v.E, v.k, v.R) for v in w.values()] == [
        (256, 512, 16, 2, 4), (128, 7168, 256, 8, 32), (16384, 4096, 64, 2, 8),
        (4096, 7168, 384, 8, 64), (32768, 2048, 512, 10, 64)]
    assert w[3].capacity == 615          # ceil(1.2 * 16384 * 2 / 64) = ceil(614.4)
    assert all(v.capacity == -1 for i, v in w.items() if i != 3)
    assert w[4].local_experts == 6 and w[5].shared


def test_generator_is_deterministic():
    w = synthetic.WORKLOADS[1]
    a = synthetic.make_inputs(w, 0)
    b = synthetic.make_inputs(w, 0)
    c = synthetic.make_inputs(w, 1)
    for key in ("logits", "x", "residual"):
        assert np.array_equal(a[key], b[key])
        assert not np.array_equal(a[key], c[key])
    assert a["x"].dtype == np.uint16 and a["x"].shape == (256, 512)
    assert np.all(a["bias"] == 0)
    bias2 = synthetic.make_inputs(synthetic.WORKLOADS[2], 0, with_activations=False)["bias"]
    assert bias2.shape == (256,) and np.abs(bias2).max() <= 0.1


def test_skew_makes_low_ids_popular():
    w = synthetic.WORKLOADS[3]
    logits = synthetic.make_logits(w, 0, T=2048)
    top1 = logits.argmax(axis=1)
    counts = np.bincount(top1, minlength=w.E)
    assert counts[0] == counts.max()


def test_round_robin():
    idx = synthetic.round_robin_idx(5, 4, 3)
    assert idx.tolist() == [[0, 1, 2], [3, 0, 1], [2, 3, 0], [1, 2, 3], [0, 1, 2]]
