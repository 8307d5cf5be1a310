"""Pins for the CPU oracle, independent of the oracle's own formulas.

Each test checks the oracle against something other than itself: values the
pages fix (tests/golden/), closed forms, a brute-force twin with an explicit
block-diagonal mask, a library routine (torch's fp64 scaled-dot-product
attention and autograd), central finite differences, and invariants of the
mathematics.  No GPU is involved.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from pvj_inputs import random_small_pack, workload, draw_tensors

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------------------
# offsets and positions
# ----------------------------------------------------------------------------

def test_token_counts_match_pages():
    g = json.load(open(os.path.join(GOLDEN, "token_counts.json")))
    s = g["pixels_per_token_side"]
    for case in g["cases"]:
        hp, wp = case["pixels"]
        sample = (hp // s, wp // s, case["text"])
        assert oracle.sample_lengths([sample])[0] == case["sample_tokens"]
        assert sample[0] * sample[1] == case["image_tokens"]
    cfg = [(1024 // s, 1024 // s, 256), (1024 // s, 1024 // s, 16)]
    assert oracle.cu_seqlens(cfg).tolist() == g["cfg_pack_1024"]["cu_seqlens"]


def test_cu_seqlens_hand_example():
    samples = [(2, 3, 1), (0, 0, 2), (1, 1, 0), (0, 0, 0), (3, 0, 4)]
    assert oracle.sample_lengths(samples).tolist() == [7, 2, 1, 0, 4]
    assert oracle.cu_seqlens(samples).tolist() == [0, 7, 9, 10, 10, 14]
    assert oracle.cu_seqlens([]).tolist() == [0]


def test_positions_hand_example():
    # text first at (0,0), then a 2x3 grid row-major; a second sample restarts at its origin
    pos = oracle.token_positions([(2, 3, 1), (1, 2, 2)])
    want = [(0, 0), (0, 0), (0, 1), (0, 2), (1, 0), (1, 1), (1, 2),
            (0, 0), (0, 0), (0, 0), (0, 1)]
    assert [tuple(p) for p in pos.tolist()] == want


# ----------------------------------------------------------------------------
# 2D RoPE
# ----------------------------------------------------------------------------

def test_rope_worked_values():
    # D = 4: one pair per axis, omega_0 = 1.  Row position 1 rotates the first
    # pair by 1 rad; column position 1 rotates the second pair by 1 rad.
    e0 = np.array([1.0, 0, 0, 0]).reshape(1, 1, 4)
    y = oracle.rope2d_at(e0, np.array([[1, 0]]))
    assert np.allclose(y.ravel(), [math.cos(1), math.sin(1), 0, 0], atol=1e-15)
    e1 = np.array([0, 1.0, 0, 0]).reshape(1, 1, 4)
    y = oracle.rope2d_at(e1, np.array([[1, 0]]))
    assert np.allclose(y.ravel(), [-math.sin(1), math.cos(1), 0, 0], atol=1e-15)
    e2 = np.array([0, 0, 1.0, 0]).reshape(1, 1, 4)
    y = oracle.rope2d_at(e2, np.array([[5, 1]]))
    assert np.allclose(y.ravel(), [0, 0, math.cos(1), math.sin(1)], atol=1e-15)
    # D = 8: two pairs per axis, omega = (1, 10000**-0.5 = 0.01)
    e = np.zeros((1, 1, 8)); e[0, 0, 2] = 1.0
    y = oracle.rope2d_at(e, np.array([[2, 7]]))
    assert np.allclose(y.ravel(), [0, 0, math.cos(0.02), math.sin(0.02), 0, 0, 0, 0], atol=1e-15)
    e = np.zeros((1, 1, 8)); e[0, 0, 7] = 1.0
    y = oracle.rope2d_at(e, np.array([[2, 7]]))
    assert np.allclose(y.ravel(), [0, 0, 0, 0, 0, 0, -math.sin(0.07), math.cos(0.07)], atol=1e-15)


@pytest.mark.parametrize("D", [8, 64, 128])
def test_rope_frequencies_endpoints(D):
    w = oracle.rope_frequencies(D)
    assert len(w) == D // 4 and w[0] == 1.0
    # geometric: ratio is constant, and omega_{D/4} would be 1/theta
    r = w[1:] / w[:-1]
    assert np.allclose(r, r[0], rtol=1e-12)
    assert math.isclose(w[-1] * r[0], 1e-4, rel_tol=1e-12)


def test_rope_complex_multiply_formulation():
    rng = np.random.default_rng(1)
    D, H, N = 16, 3, 20
    x = _rand(rng, N, H, D)
    pos = rng.integers(0, 40, size=(N, 2))
    y = oracle.rope2d_at(x, pos)
    # second formulation: each adjacent pair is a complex number times e^{i p w}
    omega = 1e4 ** (-np.arange(D // 4) / (D // 4))
    for axis in range(2):
        half = x[:, :, axis * D // 2:(axis + 1) * D // 2]
        z = half[..., 0::2] + 1j * half[..., 1::2]
        rot = np.exp(1j * pos[:, axis][:, None, None] * omega[None, None, :])
        zz = z * rot
        got = y[:, :, axis * D // 2:(axis + 1) * D // 2]
        assert np.allclose(got[..., 0::2], zz.real, atol=1e-13)
        assert np.allclose(got[..., 1::2], zz.imag, atol=1e-13)


def test_rope_norm_and_inverse():
    rng = np.random.default_rng(2)
    x = _rand(rng, 30, 2, 32)
    pos = rng.integers(0, 128, size=(30, 2))
    y = oracle.rope2d_at(x, pos)
    assert np.allclose(np.linalg.norm(y, axis=2), np.linalg.norm(x, axis=2), rtol=1e-14)
    pairs_x = (x.reshape(30, 2, 16, 2) ** 2).sum(-1)
    pairs_y = (y.reshape(30, 2, 16, 2) ** 2).sum(-1)
    assert np.allclose(pairs_x, pairs_y, rtol=1e-13)
    back = oracle.rope2d_at(y, pos, inverse=True)
    assert np.allclose(back, x, atol=1e-13)


def test_rope_relative_offset():
    rng = np.random.default_rng(3)
    D = 32
    q = _rand(rng, 1, 1, D)
    k = _rand(rng, 1, 1, D)
    for _ in range(10):
        p = rng.integers(0, 100, size=(1, 2))
        p2 = rng.integers(0, 100, size=(1, 2))
        lhs = (oracle.rope2d_at(q, p) * oracle.rope2d_at(k, p2)).sum()
        rhs = (q * oracle.rope2d_at(k, p2 - p)).sum()
        assert math.isclose(lhs, rhs, rel_tol=1e-11, abs_tol=1e-11)


def test_rope_shift_invariance_of_attention():
    # an image-only sample: shifting every position by (dr, dc) leaves the logits unchanged
    rng = np.random.default_rng(4)
    h, w, D = 3, 5, 16
    q = _rand(rng, h * w, 2, D)
    k = _rand(rng, h * w, 2, D)
    pos = oracle.token_positions([(h, w, 0)])
    s0 = np.einsum("ihd,jhd->hij", oracle.rope2d_at(q, pos), oracle.rope2d_at(k, pos))
    shifted = pos + np.array([[7, 11]])
    s1 = np.einsum("ihd,jhd->hij", oracle.rope2d_at(q, shifted), oracle.rope2d_at(k, shifted))
    assert np.allclose(s0, s1, atol=1e-11)


def test_rope_text_tokens_identity():
    rng = np.random.default_rng(5)
    x = _rand(rng, 9, 2, 16)
    assert np.array_equal(oracle.rope2d(x, [(0, 0, 4), (0, 7, 5)]), x)


# ----------------------------------------------------------------------------
# forward
# ----------------------------------------------------------------------------

def _masked_sdpa(q, k, v, samples, scale):
    """torch fp64 scaled_dot_product_attention over the whole pack with a boolean
    block-diagonal mask (a library routine, independent of the oracle)."""
    T = q.shape[0]
    lens = [s[2] + s[0] * s[1] * (s[3] if len(s) > 3 else 1) for s in samples]
    owner = np.concatenate([[i] * n for i, n in enumerate(lens)] + [[]])
    owner = owner.astype(np.int64)
    mask = torch.from_numpy(owner[:, None] == owner[None, :])
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]
    kt = torch.from_numpy(k).permute(1, 0, 2)[None]
    vt = torch.from_numpy(v).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    logits = (qt @ kt.transpose(-1, -2)) * scale
    logits = logits.masked_fill(~mask, -math.inf)
    lse = torch.logsumexp(logits, dim=-1)[0]
    return o[0].permute(1, 0, 2).numpy(), lse.numpy()


@pytest.mark.parametrize("seed", range(6))
def test_fwd_matches_bruteforce_and_sdpa(seed):
    rng = np.random.default_rng(100 + seed)
    samples = random_small_pack(rng, int(rng.integers(1, 6)), allow_empty=True)
    samples.append((2, 2, 1))  # at least one non-empty sample
    T = int(oracle.sample_lengths(samples).sum())
    H, D = 2, 8
    q, k, v = (_rand(rng, T, H, D) for _ in range(3))
    o, lse = oracle.attn_fwd(q, k, v, samples)
    ob, lseb = oracle.dense_masked_attn_fwd(q, k, v, samples)
    assert np.abs(o - ob).max() <= 1e-12
    assert np.abs(lse - lseb).max() <= 1e-12
    os_, lses = _masked_sdpa(q, k, v, samples, 1 / math.sqrt(D))
    assert np.abs(o - os_).max() <= 1e-12
    assert np.abs(lse - lses).max() <= 1e-12


def test_fwd_default_scale_is_inverse_sqrt_d():
    rng = np.random.default_rng(7)
    samples = [(2, 3, 2)]
    q, k, v = (_rand(rng, 8, 1, 16) for _ in range(3))
    o, _ = oracle.attn_fwd(q, k, v, samples)
    qt, kt, vt = (torch.from_numpy(x).permute(1, 0, 2)[None] for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0].permute(1, 0, 2).numpy()
    assert np.abs(o - ref).max() <= 1e-12


def test_fwd_closed_forms():
    rng = np.random.default_rng(8)
    D = 16
    # L = 1: the only key gets probability 1, so O = V and LSE = scale * q.k
    samples = [(1, 1, 0), (0, 0, 1)]
    q, k, v = (_rand(rng, 2, 3, D) for _ in range(3))
    o, lse = oracle.attn_fwd(q, k, v, samples)
    assert np.allclose(o, v, atol=1e-15)
    assert np.allclose(lse, (q * k).sum(-1).T / 4.0, atol=1e-14)
    # Q = 0: uniform probabilities, O = mean of V, LSE = ln L (for any K, with or without RoPE)
    samples = [(3, 4, 5), (2, 2, 0)]
    T = 21
    q = np.zeros((T, 2, D))
    k, v = _rand(rng, T, 2, D), _rand(rng, T, 2, D)
    for rope in (False, True):
        o, lse = oracle.attn_fwd(q, k, v, samples, rope=rope)
        assert np.allclose(o[:17], v[:17].mean(0, keepdims=True), atol=1e-14)
        assert np.allclose(o[17:], v[17:].mean(0, keepdims=True), atol=1e-14)
        assert np.allclose(lse[:, :17], math.log(17), atol=1e-14)
        assert np.allclose(lse[:, 17:], math.log(4), atol=1e-14)


def test_fwd_rope_matches_explicit_rotation():
    # rope=True equals rotating Q and K by the per-sample positions, then plain attention
    rng = np.random.default_rng(9)
    samples = [(2, 3, 2), (3, 1, 1)]
    q, k, v = (_rand(rng, 12, 2, 8) for _ in range(3))
    pos = np.array([(0, 0), (0, 0), (0, 0), (0, 1), (0, 2), (1, 0), (1, 1), (1, 2),
                    (0, 0), (0, 0), (1, 0), (2, 0)])
    o1, l1 = oracle.attn_fwd(q, k, v, samples, rope=True)
    o2, l2 = oracle.dense_masked_attn_fwd(oracle.rope2d_at(q, pos), oracle.rope2d_at(k, pos), v,
                                          samples)
    assert np.abs(o1 - o2).max() <= 1e-12 and np.abs(l1 - l2).max() <= 1e-12


def test_fwd_rows_helper():
    rng = np.random.default_rng(10)
    samples = [(2, 3, 2), (3, 3, 1)]
    q, k, v = (_rand(rng, 18, 2, 8) for _ in range(3))
    o, lse = oracle.attn_fwd(q, k, v, samples, rope=True)
    rows = [0, 4, 9]
    o1, l1 = oracle.attn_fwd_rows(q, k, v, samples, 1, 1, rows, rope=True)
    assert np.abs(o1 - o[8 + np.array(rows), 1]).max() <= 1e-13
    assert np.abs(l1 - lse[1, 8 + np.array(rows)]).max() <= 1e-13


def test_pack_invariants():
    # single-sample pack == unpacked; permuting samples permutes outputs
    rng = np.random.default_rng(11)
    samples = [(2, 3, 2), (1, 4, 3), (3, 2, 0)]
    lens = oracle.sample_lengths(samples)
    T = int(lens.sum())
    q, k, v = (_rand(rng, T, 2, 8) for _ in range(3))
    o, lse = oracle.attn_fwd(q, k, v, samples, rope=True)
    cu = oracle.cu_seqlens(samples)
    for i, s in enumerate(samples):
        a, b = cu[i], cu[i + 1]
        oi, li = oracle.attn_fwd(q[a:b], k[a:b], v[a:b], [s], rope=True)
        assert np.array_equal(oi, o[a:b]) and np.array_equal(li, lse[:, a:b])
    perm = [2, 0, 1]
    idx = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in perm])
    op, lp = oracle.attn_fwd(q[idx], k[idx], v[idx], [samples[i] for i in perm], rope=True)
    assert np.array_equal(op, o[idx]) and np.array_equal(lp, lse[:, idx])


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------

def _loss(q, k, v, do, samples, rope):
    o, _ = oracle.attn_fwd(q, k, v, samples, rope=rope)
    return float((o * do).sum())


@pytest.mark.parametrize("rope", [False, True])
def test_bwd_finite_differences(rope):
    rng = np.random.default_rng(12 + rope)
    samples = [(2, 2, 1), (1, 3, 2), (0, 0, 1)]
    T, H, D = 11, 2, 8
    q, k, v, do = (_rand(rng, T, H, D) for _ in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, samples, rope=rope)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            i, h, d = rng.integers(0, T), rng.integers(0, H), rng.integers(0, D)
            xp = x.copy(); xp[i, h, d] += eps
            xm = x.copy(); xm[i, h, d] -= eps
            args_p = {"q": q, "k": k, "v": v}; args_p[name] = xp
            args_m = {"q": q, "k": k, "v": v}; args_m[name] = xm
            fd = (_loss(args_p["q"], args_p["k"], args_p["v"], do, samples, rope)
                  - _loss(args_m["q"], args_m["k"], args_m["v"], do, samples, rope)) / (2 * eps)
            assert abs(fd - g[i, h, d]) <= 1e-6 * max(1.0, abs(fd)), (name, i, h, d, fd, g[i, h, d])


def test_bwd_matches_torch_autograd():
    rng = np.random.default_rng(14)
    samples = [(3, 3, 2), (2, 4, 1), (1, 1, 0)]
    T, H, D = 21, 3, 16
    q, k, v, do = (_rand(rng, T, H, D) for _ in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, samples)
    tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
    owner = np.concatenate([[i] * (t + h * w) for i, (h, w, t) in enumerate(samples)])
    mask = torch.from_numpy(owner[:, None] == owner[None, :])
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.permute(1, 0, 2), tk.permute(1, 0, 2), tv.permute(1, 0, 2), attn_mask=mask)
    (o.permute(1, 0, 2) * torch.from_numpy(do)).sum().backward()
    assert np.abs(dq - tq.grad.numpy()).max() <= 1e-12
    assert np.abs(dk - tk.grad.numpy()).max() <= 1e-12
    assert np.abs(dv - tv.grad.numpy()).max() <= 1e-12


def test_bwd_invariants():
    # softmax shift invariance: per sample and head, the key gradients sum to zero;
    # the value gradients sum to the output gradients (columns of P sum over rows to 1 per row)
    rng = np.random.default_rng(15)
    samples = [(3, 2, 2), (2, 2, 3)]
    T, H, D = 15, 2, 8
    q, k, v, do = (_rand(rng, T, H, D) for _ in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, samples)
    cu = oracle.cu_seqlens(samples)
    for i in range(len(samples)):
        a, b = cu[i], cu[i + 1]
        assert np.abs(dk[a:b].sum(0)).max() <= 1e-12
        assert np.abs(dv[a:b].sum(0) - do[a:b].sum(0)).max() <= 1e-12
    # with RoPE the invariant holds for the rotated-key gradient R dK
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, samples, rope=True)
    dkr = oracle.rope2d(dk, samples)
    for i in range(len(samples)):
        a, b = cu[i], cu[i + 1]
        assert np.abs(dkr[a:b].sum(0)).max() <= 1e-12


def test_delta_closed_form():
    rng = np.random.default_rng(16)
    o, do = _rand(rng, 5, 3, 4), _rand(rng, 5, 3, 4)
    d = oracle.attn_bwd_delta(o, do)
    for t in range(5):
        for h in range(3):
            assert math.isclose(d[h, t], sum(o[t, h, j] * do[t, h, j] for j in range(4)),
                                rel_tol=1e-14, abs_tol=1e-14)


# ----------------------------------------------------------------------------
# the two modality streams
# ----------------------------------------------------------------------------

def test_pack_unpack_hand_example():
    samples = [(1, 2, 1), (0, 0, 2), (2, 1, 0)]
    text = np.arange(3).reshape(3, 1, 1) + 100.0       # t = 1 + 2 + 0
    image = np.arange(4).reshape(4, 1, 1) + 200.0      # hw = 2 + 0 + 2
    joint = oracle.pack_joint(text, image, samples)
    assert joint.ravel().tolist() == [100, 200, 201, 101, 102, 202, 203]
    t2, i2 = oracle.unpack_joint(joint, samples)
    assert np.array_equal(t2, text) and np.array_equal(i2, image)


# ----------------------------------------------------------------------------
# the synthetic workloads (generator checks, not oracle pins)
# ----------------------------------------------------------------------------

def test_workload_shapes():
    assert workload("single_1024").n_tokens == 4352
    assert workload("cfg_1024").n_tokens == 8464
    assert workload("tiny_f32").n_tokens == 560
    tr = workload("train_64k", 0)
    assert tr.samples[:3] == [(116, 92, 277), (56, 60, 51), (36, 32, 116)]
    assert len(tr.samples) == 7 and tr.n_tokens == 55151
    for s in range(20):
        w = workload("train_64k", s)
        assert w.n_tokens <= 65536
        for (h, ww, t) in w.samples:
            assert 32 <= h <= 128 and 32 <= ww <= 128 and 32 <= t <= 512
            assert max(h, ww) <= 4 * min(h, ww)
    ex = workload("extreme", 0)
    assert [t for (_, _, t) in ex.samples] == [438, 332, 270, 150, 168, 36, 53]
    assert ex.n_tokens == 30119


def test_cfg_tensors_share_image_rows():
    wl = workload("cfg_1024")
    q, = draw_tensors(wl.n_tokens, 2, 8, "bf16", 0, n=1, samples=wl.samples,
                      shared_image=wl.shared_image)
    assert np.array_equal(q[256:4352], q[4352 + 16:])
    assert not np.array_equal(q[:16], q[4352:4352 + 16])


# ----------------------------------------------------------------------------
# editing mode: 3-axis (row, col, frame) RoPE
# ----------------------------------------------------------------------------

def test_positions3_hand_example():
    pos = oracle.token_positions3([(2, 2, 1, 2), (1, 2, 0)])
    want = [(0, 0, 0),
            (0, 0, 0), (0, 1, 0), (1, 0, 0), (1, 1, 0),
            (0, 0, 1), (0, 1, 1), (1, 0, 1), (1, 1, 1),
            (0, 0, 0), (0, 1, 0)]
    assert [tuple(p) for p in pos.tolist()] == want
    assert oracle.sample_lengths([(2, 2, 1, 2), (1, 2, 0)]).tolist() == [9, 2]
    assert oracle.rope_axis_dims(128, 3) == (56, 56, 16)
    assert oracle.rope_axis_dims(64, 3) == (24, 24, 16)


def test_rope3_worked_values():
    # D = 32 -> parts (8, 8, 16): row dims 0..7, col dims 8..15, frame dims 16..31
    def unit(i):
        e = np.zeros((1, 1, 32)); e[0, 0, i] = 1.0
        return e
    dims = oracle.rope_axis_dims(32, 3)
    y = oracle.rope_nd_at(unit(16), np.array([[5, 3, 1]]), dims)      # frame pair 0 by f = 1
    assert np.allclose(y[0, 0, 16:18], [math.cos(1), math.sin(1)], atol=1e-15)
    assert np.allclose(np.delete(y.ravel(), [16, 17]), 0, atol=1e-15)
    y = oracle.rope_nd_at(unit(8), np.array([[5, 3, 1]]), dims)       # col pair 0 by c = 3
    assert np.allclose(y[0, 0, 8:10], [math.cos(3), math.sin(3)], atol=1e-15)
    y = oracle.rope_nd_at(unit(2), np.array([[5, 3, 1]]), dims)       # row pair 1, omega = 1e4**-0.25
    w = 1e4 ** -0.25
    assert np.allclose(y[0, 0, 2:4], [math.cos(5 * w), math.sin(5 * w)], atol=1e-15)
    y = oracle.rope_nd_at(unit(18), np.array([[5, 3, 2]]), dims)      # frame pair 1, omega = 1e4**-1/8
    w = 1e4 ** (-1 / 8)
    assert np.allclose(y[0, 0, 18:20], [math.cos(2 * w), math.sin(2 * w)], atol=1e-15)


def test_rope_nd_two_axes_equals_2d():
    rng = np.random.default_rng(30)
    x = _rand(rng, 12, 2, 64)
    pos = rng.integers(0, 50, size=(12, 2))
    assert np.allclose(oracle.rope_nd_at(x, pos, (32, 32)), oracle.rope2d_at(x, pos), atol=1e-14)


def test_rope3_norm_inverse_and_shift_invariance():
    rng = np.random.default_rng(31)
    samples = [(3, 4, 2, 2)]
    T, D = 26, 64
    q, k = _rand(rng, T, 2, D), _rand(rng, T, 2, D)
    qr = oracle.rope3d(q, samples)
    assert np.allclose(np.linalg.norm(qr, axis=2), np.linalg.norm(q, axis=2), rtol=1e-14)
    assert np.allclose(oracle.rope3d(qr, samples, inverse=True), q, atol=1e-13)
    pos = oracle.token_positions3(samples)[2:]          # image tokens only
    dims = oracle.rope_axis_dims(D, 3)
    s0 = np.einsum("ihd,jhd->hij", oracle.rope_nd_at(q[2:], pos, dims),
                   oracle.rope_nd_at(k[2:], pos, dims))
    sh = pos + np.array([[4, 9, 3]])
    s1 = np.einsum("ihd,jhd->hij", oracle.rope_nd_at(q[2:], sh, dims),
                   oracle.rope_nd_at(k[2:], sh, dims))
    assert np.allclose(s0, s1, atol=1e-11)


def test_frame_axis_separates_source_and_target():
    # identical source and target grids: the 2-axis RoPE cannot tell them apart
    # (equal outputs), the frame axis can (the pages' reason for adding it)
    rng = np.random.default_rng(32)
    h, w, t = 2, 3, 2
    n = h * w
    q, k, v = (_rand(rng, t + 2 * n, 1, 32) for _ in range(3))
    for x in (q, k, v):
        x[t + n:] = x[t:t + n]
    o2, _ = oracle.attn_fwd(q, k, v, [(h, w, t, 2)], rope=True, axes=2)
    o3, _ = oracle.attn_fwd(q, k, v, [(h, w, t, 2)], rope=True, axes=3)
    assert np.allclose(o2[t:t + n], o2[t + n:], atol=1e-13)
    assert np.abs(o3[t:t + n] - o3[t + n:]).max() > 1e-3


def test_fwd3_matches_bruteforce_and_sdpa():
    rng = np.random.default_rng(33)
    samples = [(2, 3, 2, 2), (3, 1, 1, 1), (0, 0, 3, 1), (2, 2, 0, 3)]
    T = int(oracle.sample_lengths(samples).sum())
    q, k, v = (_rand(rng, T, 2, 32) for _ in range(3))
    o, lse = oracle.attn_fwd(q, k, v, samples, rope=True, axes=3)
    pos = oracle.token_positions3(samples)
    dims = oracle.rope_axis_dims(32, 3)
    qr, kr = oracle.rope_nd_at(q, pos, dims), oracle.rope_nd_at(k, pos, dims)
    ob, lb = oracle.dense_masked_attn_fwd(qr, kr, v, samples)
    assert np.abs(o - ob).max() <= 1e-12 and np.abs(lse - lb).max() <= 1e-12
    os_, ls_ = _masked_sdpa(qr, kr, v, samples, 1 / math.sqrt(32))
    assert np.abs(o - os_).max() <= 1e-12 and np.abs(lse - ls_).max() <= 1e-12


def test_bwd3_finite_differences():
    rng = np.random.default_rng(34)
    samples = [(2, 2, 1, 2), (1, 2, 1, 1)]
    T, H, D = 12, 1, 32
    q, k, v, do = (_rand(rng, T, H, D) for _ in range(4))
    dq, dk, dv = oracle.attn_bwd(q, k, v, do, samples, rope=True, axes=3)

    def loss(qq, kk, vv):
        o, _ = oracle.attn_fwd(qq, kk, vv, samples, rope=True, axes=3)
        return float((o * do).sum())
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(8):
            i, d = rng.integers(0, T), rng.integers(0, D)
            xp = x.copy(); xp[i, 0, d] += eps
            xm = x.copy(); xm[i, 0, d] -= eps
            args = {"q": q, "k": k, "v": v}
            ap = dict(args); ap[name] = xp
            am = dict(args); am[name] = xm
            fd = (loss(ap["q"], ap["k"], ap["v"]) - loss(am["q"], am["k"], am["v"])) / (2 * eps)
            assert abs(fd - g[i, 0, d]) <= 1e-6 * max(1.0, abs(fd)), (name, i, d)


def test_pack3_hand_example():
    samples = [(1, 2, 1, 2), (0, 0, 1, 1)]
    text = np.array([100.0, 101.0]).reshape(2, 1, 1)
    image = np.arange(4).reshape(4, 1, 1) + 200.0
    joint = oracle.pack_joint(text, image, samples)
    assert joint.ravel().tolist() == [100, 200, 201, 202, 203, 101]
    t2, i2 = oracle.unpack_joint(joint, samples)
    assert np.array_equal(t2, text) and np.array_equal(i2, image)
