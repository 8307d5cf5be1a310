"""GPU parity of editing packs (a frame axis on top of the 2D latent grid, so
every RoPE in the plan is the 3-axis row/col/frame one) against the oracle,
through the C ABI: the standalone RoPE, pack/unpack, the forward with RoPE on
load and the backward with its inverse rotation.

Small ragged packs are compared in full (frames 0..3, empty, text-only and
one-token samples); the full editing workload (two 1024-class source/target
pairs, 24 heads, D=128) on whole (sample, head) slices.
"""
import numpy as np
import pytest

import oracle
from pvj_inputs import draw_tensors, random_small_pack, workload, workload_tensors

from helpers import Guarded, GuardedLse, assert_close, assert_lse, say, to_dev, to_np

torch = pytest.importorskip("torch")
pvj = pytest.importorskip("packed_varlen_joint_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pvj.load_library()


def _plan(samples, H, D, dt):
    p = pvj.Plan(samples, H, D, dt).upload()
    assert p.rope_axes()[0] == 3
    return p


EDIT_RAGGED = [(0, 0, 0, 0), (3, 5, 7, 2), (1, 1, 0, 3), (0, 0, 1, 1), (9, 17, 33, 2),
               (4, 4, 130, 0), (2, 40, 3, 3), (12, 12, 0, 1), (5, 0, 4, 2)]


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_rope3_apply(dt, D):
    say("rope (3 axes) dt=%s D=%d ragged editing pack" % (dt, D))
    H = 3
    plan = _plan(EDIT_RAGGED, H, D, dt)
    T = plan.n_tokens
    x, = draw_tensors(T, H, D, dt, 8, n=1)
    xd = to_dev(x, dt)
    for inverse in (False, True):
        ref = oracle.rope_apply(x, EDIT_RAGGED, inverse=inverse, axes=3)
        y = Guarded(T, H, D, dt)
        pvj.rope2d_apply(plan, xd, y.t, inverse=inverse)
        torch.cuda.synchronize()
        y.check("rope3")
        err = np.abs(to_np(y.t) - ref)
        bound = (2.0 ** -8 * np.abs(ref) + 1e-5) if dt == "bf16" else 1e-5
        say("   inverse=%d max_abs=%.3e" % (inverse, err.max()))
        assert np.all(err <= bound)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_pack_unpack_frames_bit_exact(dt):
    say("pack/unpack editing pack dt=%s" % dt)
    H, D = 2, 64
    plan = _plan(EDIT_RAGGED, H, D, dt)
    text = draw_tensors(plan.n_text, H, D, dt, 3, n=1)[0]
    image = draw_tensors(plan.n_image, H, D, dt, 4, n=1)[0]
    ref = oracle.pack_joint(text, image, EDIT_RAGGED)
    j = Guarded(plan.n_tokens, H, D, dt)
    pvj.pack(plan, to_dev(text, dt), to_dev(image, dt), j.t)
    torch.cuda.synchronize()
    j.check("pack")
    assert np.array_equal(to_np(j.t), ref)
    t2, i2 = pvj.unpack(plan, j.t)
    assert np.array_equal(to_np(t2), text) and np.array_equal(to_np(i2), image)


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_fwd_bwd_frames_ragged(dt, D):
    say("fwd+bwd editing pack dt=%s D=%d" % (dt, D))
    H = 2
    plan = _plan(EDIT_RAGGED, H, D, dt)
    T = plan.n_tokens
    q, k, v, do = draw_tensors(T, H, D, dt, 21, n=4)
    qd, kd, vd, dod = (to_dev(x, dt) for x in (q, k, v, do))
    o = Guarded(T, H, D, dt)
    lse = GuardedLse(H, T)
    pvj.varlen_attn_fwd(plan, qd, kd, vd, rope_fused=True, out=o.t, lse=lse.t)
    torch.cuda.synchronize()
    o.check("o")
    lse.check()
    ro, rl = oracle.attn_fwd(q, k, v, EDIT_RAGGED, rope=True, axes=3)
    assert_close("o", to_np(o.t), ro, dt)
    assert_lse(to_np(lse.t), rl, dt)
    g = [Guarded(T, H, D, dt) for _ in range(3)]
    pvj.varlen_attn_bwd(plan, qd, kd, vd, o.t, lse.t, dod, rope_fused=True, dq=g[0].t,
                        dk=g[1].t, dv=g[2].t)
    torch.cuda.synchronize()
    for name, x in zip(("dq", "dk", "dv"), g):
        x.check(name)
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, EDIT_RAGGED, rope=True, axes=3)
    assert_close("dq", to_np(g[0].t), rq, dt)
    assert_close("dk", to_np(g[1].t), rk, dt)
    assert_close("dv", to_np(g[2].t), rv, dt)


@pytest.mark.parametrize("seed", range(2))
def test_fwd_bwd_frames_random(seed):
    rng = np.random.default_rng(900 + seed)
    samples = random_small_pack(rng, int(rng.integers(1, 6)), max_side=16, max_text=200,
                                max_frames=3)
    dt, H, D = "bf16", 2, 128
    say("fwd+bwd random editing pack seed=%d samples=%s" % (seed, samples))
    plan = _plan(samples, H, D, dt)
    if plan.n_tokens == 0:
        return
    q, k, v, do = draw_tensors(plan.n_tokens, H, D, dt, 950 + seed, n=4)
    qd, kd, vd, dod = (to_dev(x, dt) for x in (q, k, v, do))
    o, lse = pvj.varlen_attn_fwd(plan, qd, kd, vd, rope_fused=True)
    dq, dk, dv = pvj.varlen_attn_bwd(plan, qd, kd, vd, o, lse, dod, rope_fused=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd(q, k, v, samples, rope=True, axes=3)
    assert_close("o", to_np(o), ro, dt)
    assert_lse(to_np(lse), rl, dt)
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, samples, rope=True, axes=3)
    assert_close("dq", to_np(dq), rq, dt)
    assert_close("dk", to_np(dk), rk, dt)
    assert_close("dv", to_np(dv), rv, dt)


def test_fused_rope_equals_standalone_then_plain():
    # RoPE on load must equal the standalone 3-axis RoPE followed by attention
    # without RoPE (same rounding of the rotated operands in fp32)
    samples = [(6, 7, 20, 2), (3, 9, 5, 3)]
    dt, H, D = "f32", 2, 64
    plan = _plan(samples, H, D, dt)
    q, k, v = (to_dev(x, dt) for x in draw_tensors(plan.n_tokens, H, D, dt, 31, n=3))
    o1, l1 = pvj.varlen_attn_fwd(plan, q, k, v, rope_fused=True)
    qr, kr = pvj.rope2d_apply(plan, q), pvj.rope2d_apply(plan, k)
    o2, l2 = pvj.varlen_attn_fwd(plan, qr, kr, v, rope_fused=False)
    torch.cuda.synchronize()
    assert (o1 - o2).abs().max().item() <= 1e-5
    assert (l1 - l2).abs().max().item() <= 1e-5


def test_pack_rope_frames_chain():
    # 3-axis: pack + RoPE in one pass == pack then RoPE (bitwise); the
    # PREROTATED backward on it == the fused-RoPE backward (bitwise)
    samples = EDIT_RAGGED
    dt, H, D = "bf16", 2, 128
    plan = _plan(samples, H, D, dt)
    say("pack_rope + PREROTATED bwd on an editing pack")
    tq, iq, tk, ik = (to_dev(draw_tensors(n, H, D, dt, 70 + s, n=1)[0], dt)
                      for s, n in enumerate([plan.n_text, plan.n_image] * 2))
    qr = pvj.pack(plan, tq, iq, rope=True)
    q = pvj.pack(plan, tq, iq)
    k = pvj.pack(plan, tk, ik)
    kr = pvj.pack(plan, tk, ik, rope=True)
    assert torch.equal(qr, pvj.rope2d_apply(plan, q))
    v, do = (to_dev(x, dt) for x in draw_tensors(plan.n_tokens, H, D, dt, 75, n=2))
    o1, l1 = pvj.varlen_attn_fwd(plan, q, k, v, rope_fused=True)
    o2, l2 = pvj.varlen_attn_fwd(plan, qr, kr, v)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = pvj.varlen_attn_bwd(plan, q, k, v, o1, l1, do, rope_fused=True)
    g2 = pvj.varlen_attn_bwd(plan, qr, kr, v, o2, l2, do, rope_prerotated=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_edit_workload_sampled():
    wl = workload("edit_1024")
    say("fwd+bwd edit_1024 T=%d" % wl.n_tokens)
    plan = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    q, k, v, do = workload_tensors(wl, 4)
    qd, kd, vd, dod = (to_dev(x, "bf16") for x in (q, k, v, do))
    o, lse = pvj.varlen_attn_fwd(plan, qd, kd, vd, rope_fused=True)
    dq, dk, dv = pvj.varlen_attn_bwd(plan, qd, kd, vd, o, lse, dod, rope_fused=True)
    torch.cuda.synchronize()
    cu = oracle.cu_seqlens(wl.samples)
    rng = np.random.default_rng(4)
    for i in range(len(wl.samples)):
        h = int(rng.integers(0, wl.n_heads))
        a, b = int(cu[i]), int(cu[i + 1])
        say("  sample %d (L=%d) head %d" % (i, b - a, h))
        sl = lambda x: x[a:b, h:h + 1]
        ro, rl = oracle.attn_fwd(sl(q), sl(k), sl(v), [wl.samples[i]], rope=True, axes=3)
        assert_close("o", to_np(o[a:b, h:h + 1]), ro, "bf16")
        assert_lse(to_np(lse[h:h + 1, a:b]), rl, "bf16")
        rq, rk, rv = oracle.attn_bwd(sl(q), sl(k), sl(v), sl(do), [wl.samples[i]], rope=True,
                                     axes=3)
        assert_close("dq", to_np(dq[a:b, h:h + 1]), rq, "bf16")
        assert_close("dk", to_np(dk[a:b, h:h + 1]), rk, "bf16")
        assert_close("dv", to_np(dv[a:b, h:h + 1]), rv, "bf16")
