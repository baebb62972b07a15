"""Pins for the oracle's stand-in expert computation on the tile-signalled
return path: a grouped linear map over the (source, local expert) blocks
of a source-major receive buffer.

Sources: thecoregrid "Mixture-of-experts acceleration through overlap"
(a producer GEMM whose output tiles each belong to one destination);
aicassindra "gpu_moe_all_to_all", "Overlapping dispatch with expert
compute" (dispatch, compute and combine form a strict chain).

Independent references: numpy's integer matmul on integer-valued inputs
(every sum exact, so the one bf16 rounding is checked through torch), the
identity map, per-expert power-of-two scalings (exact, and they show which
expert each row was given to), and synthetic weights' scale.
"""

import numpy as np
import pytest
import torch

import synthetic


def bf16_bits(a):
    return torch.from_numpy(np.array(a, np.float64)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def labels(cnt):
    S, El = cnt.shape
    return np.concatenate([np.repeat(np.arange(El), cnt[s]) for s in range(S)]).astype(np.int64)


@pytest.mark.parametrize("S,El,H,H_out,seed", [(3, 2, 64, 32, 0), (1, 4, 32, 96, 1), (5, 1, 128, 64, 2), (4, 3, 96, 96, 3)])
def test_integer_inputs_match_numpy(orc, S, El, H, H_out, seed):
    r = np.random.default_rng(seed)
    cnt = r.integers(0, 7, size=(S, El)).astype(np.int32)
    cnt[0, 0] = 0
    N = int(cnt.sum())
    xi = r.integers(-8, 9, size=(N, H))
    wi = r.integers(-8, 9, size=(El, H_out, H))
    x, W = bf16_bits(xi), bf16_bits(wi)
    y = orc.expert_linear(x, cnt, W)
    lab = labels(cnt)
    exact = np.stack([xi[i] @ wi[lab[i]].T for i in range(N)]) if N else np.zeros((0, H_out))
    np.testing.assert_array_equal(y, bf16_bits(exact))


def test_identity_and_power_of_two_maps(orc):
    r = np.random.default_rng(4)
    S, El, H = 6, 3, 64
    cnt = r.integers(0, 9, size=(S, El)).astype(np.int32)
    cnt[2, :] = 0
    N = int(cnt.sum())
    x = synthetic.bf16_bits_from_f32(r.standard_normal((N, H)).astype(np.float32))
    eye = np.broadcast_to(np.eye(H), (El, H, H))
    np.testing.assert_array_equal(orc.expert_linear(x, cnt, bf16_bits(eye)), x)
    scale = np.array([0.5, 2.0, 8.0])
    y = orc.expert_linear(x, cnt, bf16_bits(eye * scale[:, None, None]))
    xv = orc.bf16_to_f64(x)
    np.testing.assert_array_equal(orc.bf16_to_f64(y), xv * scale[labels(cnt)][:, None])


def test_synthetic_weights_keep_unit_scale(orc):
    S, El, H = 2, 2, 512
    cnt = np.array([[40, 30], [20, 10]], np.int32)
    x = synthetic.normal_bf16(0, synthetic.STREAM_X, (100, H))
    W = synthetic.make_expert_weights(El, H, H)
    y = orc.bf16_to_f64(orc.expert_linear(x, cnt, W))
    assert 0.8 < y.std() < 1.2


def test_rejects_negative_counts(orc):
    with pytest.raises(ValueError):
        orc.expert_linear(np.zeros((4, 32), np.uint16), np.array([[2, -1]], np.int32), np.zeros((2, 32, 32), np.uint16))
