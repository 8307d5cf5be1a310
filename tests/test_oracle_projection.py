"""Pins of the oracle's projections with the pack/unpack fused in: identity
weights reduce them to the pack/unpack and the RoPE, per-stream weights are
selected per token, and the products agree with torch's linear layer."""
import numpy as np
import pytest

import oracle
from oracle import projection

torch = pytest.importorskip("torch")

SAMPLES = [(2, 3, 4), (0, 0, 2), (1, 2, 0), (3, 1, 1)]
H, D = 2, 8
HD = H * D


def _streams(seed):
    rng = np.random.default_rng(seed)
    nt = sum(s[2] for s in SAMPLES)
    ni = sum(s[0] * s[1] for s in SAMPLES)
    return rng.standard_normal((nt, HD)), rng.standard_normal((ni, HD))


def test_linear_hand_example_and_torch():
    x = np.array([[1.0, 2.0], [3.0, -1.0]])
    w = np.array([[1.0, 0.0], [0.5, 2.0], [0.0, -1.0]])
    b = np.array([0.0, 1.0, 2.0])
    assert projection.linear(x, w, b).tolist() == [[1.0, 5.5, 0.0], [3.0, 0.5, 3.0]]
    rng = np.random.default_rng(1)
    x, w, b = rng.standard_normal((7, 5)), rng.standard_normal((4, 5)), rng.standard_normal(4)
    ref = torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w),
                                     torch.from_numpy(b)).numpy()
    assert np.abs(projection.linear(x, w, b) - ref).max() < 1e-12


def test_identity_weights_reduce_to_pack_and_rope():
    xt, xi = _streams(2)
    eye3 = np.concatenate([np.eye(HD)] * 3, axis=0)        # [3HD, HD]
    q, k, v = projection.qkv_project_pack(xt, xi, eye3, None, eye3, None, SAMPLES, H, D,
                                          rope=False)
    joint = oracle.pack_joint(xt.reshape(-1, H, D), xi.reshape(-1, H, D), SAMPLES)
    assert np.array_equal(q, joint) and np.array_equal(k, joint) and np.array_equal(v, joint)
    q, k, v = projection.qkv_project_pack(xt, xi, eye3, None, eye3, None, SAMPLES, H, D)
    assert np.abs(q - oracle.rope2d(joint, SAMPLES)).max() < 1e-14
    assert np.array_equal(v, joint)
    yt, yi = projection.out_project_unpack(joint, np.eye(HD), None, np.eye(HD), None, SAMPLES)
    assert np.array_equal(yt, xt) and np.array_equal(yi, xi)


def test_per_stream_weights_and_parts():
    xt, xi = _streams(3)
    w_t = np.concatenate([2 * np.eye(HD), 5 * np.eye(HD), 7 * np.eye(HD)])
    w_i = np.concatenate([3 * np.eye(HD), 11 * np.eye(HD), 13 * np.eye(HD)])
    b = np.arange(3 * HD, dtype=np.float64)
    q, k, v = projection.qkv_project_pack(xt, xi, w_t, b, w_i, b, SAMPLES, H, D, rope=False)
    # sample 0: 4 text rows then 6 image rows
    assert np.allclose(q[0].ravel(), 2 * xt[0] + b[:HD])
    assert np.allclose(k[4].ravel(), 11 * xi[0] + b[HD:2 * HD])
    assert np.allclose(v[4].ravel(), 13 * xi[0] + b[2 * HD:])
    # sample 1 is text only (2 rows), joint rows 10, 11
    assert np.allclose(v[11].ravel(), 7 * xt[5] + b[2 * HD:])
