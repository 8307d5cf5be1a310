"""GPU parity of the attention backward (through the C ABI) against the oracle.

Full comparison of dQ, dK, dV on small ragged packs (every dtype, head dim,
with and without RoPE on load); at the full training and extreme-shape packs,
whole (sample, head) slices against the oracle, plus properties that hold at
any size: dK and dV are bitwise deterministic, a one-sample pack equals the
unpacked call, and the softmax shift invariants hold.
"""
import numpy as np
import pytest

import oracle
from pvj_inputs import draw_tensors, random_small_pack, workload, workload_tensors

from helpers import Guarded, assert_close, say, to_dev, to_np

torch = pytest.importorskip("torch")
pvj = pytest.importorskip("packed_varlen_joint_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pvj.load_library()


def _plan(samples, H, D, dt):
    return pvj.Plan(samples, H, D, dt).upload()


RAGGED = [(0, 0, 0), (3, 5, 7), (1, 1, 0), (0, 0, 1), (9, 17, 33), (0, 0, 130), (2, 64, 3),
          (12, 12, 0), (5, 0, 4)]


def _fwd_bwd(plan, q, k, v, do, rope, dt):
    o, lse = pvj.varlen_attn_fwd(plan, q, k, v, rope_fused=rope)
    T, H, D = plan.n_tokens, plan.n_heads, plan.head_dim
    g = [Guarded(T, H, D, dt) for _ in range(3)]
    pvj.varlen_attn_bwd(plan, q, k, v, o, lse, do, rope_fused=rope, dq=g[0].t, dk=g[1].t,
                        dv=g[2].t)
    torch.cuda.synchronize()
    for name, x in zip(("dq", "dk", "dv"), g):
        x.check(name)
    return o, lse, g[0].t, g[1].t, g[2].t


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("rope", [False, True])
def test_bwd_ragged_pack(dt, D, rope):
    say("bwd ragged pack dt=%s D=%d rope=%d" % (dt, D, rope))
    H = 3
    plan = _plan(RAGGED, H, D, dt)
    q, k, v, do = draw_tensors(plan.n_tokens, H, D, dt, 41, n=4)
    _, _, dq, dk, dv = _fwd_bwd(plan, *(to_dev(x, dt) for x in (q, k, v, do)), rope, dt)
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, RAGGED, rope=rope)
    assert_close("dq", to_np(dq), rq, dt)
    assert_close("dk", to_np(dk), rk, dt)
    assert_close("dv", to_np(dv), rv, dt)


@pytest.mark.parametrize("seed", range(3))
def test_bwd_random_packs(seed):
    rng = np.random.default_rng(500 + seed)
    samples = random_small_pack(rng, int(rng.integers(1, 8)), max_side=20, max_text=260)
    dt, H, D = "bf16", 2, 128
    say("bwd random pack seed=%d samples=%s" % (seed, samples))
    plan = _plan(samples, H, D, dt)
    if plan.n_tokens == 0:
        return
    q, k, v, do = draw_tensors(plan.n_tokens, H, D, dt, 600 + seed, n=4)
    _, _, dq, dk, dv = _fwd_bwd(plan, *(to_dev(x, dt) for x in (q, k, v, do)), True, dt)
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, samples, rope=True)
    assert_close("dq", to_np(dq), rq, dt)
    assert_close("dk", to_np(dk), rk, dt)
    assert_close("dv", to_np(dv), rv, dt)


def test_bwd_tiny_f32_workload():
    wl = workload("tiny_f32")
    say("bwd tiny_f32 (fp32 backward on the tiny pack)")
    plan = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    q, k, v, do = workload_tensors(wl, 4)
    _, _, dq, dk, dv = _fwd_bwd(plan, *(to_dev(x, "f32") for x in (q, k, v, do)), True, "f32")
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, wl.samples, rope=True)
    assert_close("dq", to_np(dq), rq, "f32")
    assert_close("dk", to_np(dk), rk, "f32")
    assert_close("dv", to_np(dv), rv, "f32")


def test_bwd_bitwise_and_invariants():
    samples = [(9, 17, 33), (12, 12, 0), (3, 5, 7), (0, 0, 130)]
    H, D, dt = 2, 128, "bf16"
    plan = _plan(samples, H, D, dt)
    q, k, v, do = (to_dev(x, dt) for x in draw_tensors(plan.n_tokens, H, D, dt, 77, n=4))
    say("bwd bitwise: determinism of dQ/dK/dV, single == unpacked")
    o, lse = pvj.varlen_attn_fwd(plan, q, k, v, rope_fused=False)
    g1 = pvj.varlen_attn_bwd(plan, q, k, v, o, lse, do)
    g2 = pvj.varlen_attn_bwd(plan, q, k, v, o, lse, do)
    torch.cuda.synchronize()
    assert torch.equal(g1[0], g2[0]) and torch.equal(g1[1], g2[1]) and torch.equal(g1[2], g2[2])
    cu = plan.cu_seqlens
    for i, s in enumerate(samples):
        a, b = cu[i], cu[i + 1]
        p1 = _plan([s], H, D, dt)
        sl = lambda t: t[a:b].contiguous()
        oi, li = pvj.varlen_attn_fwd(p1, sl(q), sl(k), sl(v))
        gi = pvj.varlen_attn_bwd(p1, sl(q), sl(k), sl(v), oi, li, sl(do))
        assert torch.equal(gi[0], g1[0][a:b])
        assert torch.equal(gi[1], g1[1][a:b]) and torch.equal(gi[2], g1[2][a:b])
        # shift invariance: key gradients sum to ~0, value gradients sum to dO's sum
        dks = g1[1][a:b].double().sum(0)
        assert dks.abs().max().item() <= 0.05
        dvs = g1[2][a:b].double().sum(0) - do[a:b].double().sum(0)
        assert dvs.abs().max().item() <= 0.05


def test_bwd_permutation_equivariance():
    # permuting the samples of a pack permutes dQ, dK and dV (bitwise): the
    # offsets confine every gradient to its own sample
    samples = [(9, 17, 33), (12, 12, 0), (3, 5, 7), (0, 0, 130), (2, 64, 3)]
    H, D, dt = 2, 128, "bf16"
    plan = _plan(samples, H, D, dt)
    q, k, v, do = (to_dev(x, dt) for x in draw_tensors(plan.n_tokens, H, D, dt, 78, n=4))
    say("bwd bitwise: permutation equivariance of dQ, dK, dV")
    o, lse = pvj.varlen_attn_fwd(plan, q, k, v, rope_fused=True)
    g = pvj.varlen_attn_bwd(plan, q, k, v, o, lse, do, rope_fused=True)
    cu = plan.cu_seqlens
    for perm in ([4, 2, 0, 3, 1], [1, 0, 2, 4, 3]):
        idx = torch.cat([torch.arange(cu[i], cu[i + 1]) for i in perm]).cuda()
        pp = _plan([samples[i] for i in perm], H, D, dt)
        pq, pk, pv, pdo = (x[idx].contiguous() for x in (q, k, v, do))
        op, lp = pvj.varlen_attn_fwd(pp, pq, pk, pv, rope_fused=True)
        gp = pvj.varlen_attn_bwd(pp, pq, pk, pv, op, lp, pdo, rope_fused=True)
        torch.cuda.synchronize()
        assert torch.equal(op, o[idx]) and torch.equal(lp, lse[:, idx])
        for a, b in zip(gp, g):
            assert torch.equal(a, b[idx])


def _nan_margin(rows, H, D, margin=128):
    # a [rows, H, D] bf16 view whose buffer continues with `margin` NaN rows
    full = torch.full((rows + margin, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    return full[:rows]


@pytest.mark.parametrize("rope", [False, True])
def test_nan_outside_a_sample_does_not_leak(rope):
    # The last, partial tiles of a sample must not read the next sample's rows
    # (or rows past the end of the tensor): the middle sample and 128 rows
    # after the pack are NaN, and the other samples' outputs must be finite
    # and bitwise equal to calls on those samples alone (whose tensors are
    # followed by NaN rows too).  Lengths 186, 95 and 2110 leave partial 32-,
    # 64-, 128- and 256-row tiles; the last one's last forward query tile is
    # split into two key ranges.
    samples = [(9, 17, 33), (0, 0, 100), (5, 7, 60), (40, 52, 30)]
    H, D, dt = 2, 128, "bf16"
    plan = _plan(samples, H, D, dt)
    cu = plan.cu_seqlens
    T = plan.n_tokens
    say("NaN isolation rope=%d T=%d" % (rope, T))
    src = [to_dev(x, dt) for x in draw_tensors(T, H, D, dt, 131, n=4)]
    q, k, v, do = (_nan_margin(T, H, D) for _ in range(4))
    for dst, x in zip((q, k, v, do), src):
        dst.copy_(x)
        dst[cu[1]:cu[2]] = float("nan")
    o, lse = pvj.varlen_attn_fwd(plan, q, k, v, rope_fused=rope)
    o_m = _nan_margin(T, H, D)
    o_m.copy_(o)
    g = pvj.varlen_attn_bwd(plan, q, k, v, o_m, lse, do, rope_fused=rope)
    torch.cuda.synchronize()
    for i in (0, 2, 3):
        a, b = cu[i], cu[i + 1]
        p1 = _plan([samples[i]], H, D, dt)
        one = []
        for x in (q, k, v, do):
            y = _nan_margin(b - a, H, D)
            y.copy_(x[a:b])
            one.append(y)
        oi, li = pvj.varlen_attn_fwd(p1, one[0], one[1], one[2], rope_fused=rope)
        oi_m = _nan_margin(b - a, H, D)
        oi_m.copy_(oi)
        gi = pvj.varlen_attn_bwd(p1, one[0], one[1], one[2], oi_m, li, one[3], rope_fused=rope)
        torch.cuda.synchronize()
        say("  sample %d rows %d..%d" % (i, a, b))
        assert bool(torch.isfinite(o[a:b].float()).all()) and bool(torch.isfinite(lse[:, a:b]).all())
        assert torch.equal(oi, o[a:b]) and torch.equal(li, lse[:, a:b])
        for name, x, y in zip(("dq", "dk", "dv"), gi, g):
            assert bool(torch.isfinite(y[a:b].float()).all()), name + " not finite"
            assert torch.equal(x, y[a:b]), name + " differs from the sample alone"


@pytest.mark.parametrize("name,seed", [("train_64k", 0), ("train_64k", 1), ("extreme", 0)])
def test_bwd_large_workloads_sampled(name, seed):
    wl = workload(name, seed)
    say("bwd %s T=%d samples=%d" % (name, wl.n_tokens, len(wl.samples)))
    plan = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    q, k, v, do = workload_tensors(wl, 4)
    _, _, dq, dk, dv = _fwd_bwd(plan, *(to_dev(x, "bf16") for x in (q, k, v, do)), True, "bf16")
    cu = oracle.cu_seqlens(wl.samples)
    lens = oracle.sample_lengths(wl.samples)
    rng = np.random.default_rng(2)
    # the shortest and the longest sample, then one at random
    picks = [int(np.argmin(lens)), int(np.argmax(lens)), int(rng.integers(0, len(wl.samples)))]
    for i in picks:
        h = int(rng.integers(0, wl.n_heads))
        a, b = int(cu[i]), int(cu[i + 1])
        say("  sample %d (L=%d) head %d" % (i, b - a, h))
        sl = lambda x: x[a:b, h:h + 1]
        rq, rk, rv = oracle.attn_bwd(sl(q), sl(k), sl(v), sl(do), [wl.samples[i]], rope=True)
        assert_close("dq", to_np(dq[a:b, h:h + 1]), rq, "bf16")
        assert_close("dk", to_np(dk[a:b, h:h + 1]), rk, "bf16")
        assert_close("dv", to_np(dv[a:b, h:h + 1]), rv, "bf16")


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f32", 64)])
def test_bwd_prerotated_equals_fused(dt, D):
    # Q', K' from the standalone RoPE + PREROTATED give the bits of ROPE_FUSED
    # (the preprocess rotates and rounds exactly as the standalone RoPE does)
    say("bwd PREROTATED == ROPE_FUSED dt=%s D=%d" % (dt, D))
    H = 2
    plan = _plan(RAGGED, H, D, dt)
    q, k, v, do = (to_dev(x, dt) for x in draw_tensors(plan.n_tokens, H, D, dt, 88, n=4))
    o, lse = pvj.varlen_attn_fwd(plan, q, k, v, rope_fused=True)
    g1 = pvj.varlen_attn_bwd(plan, q, k, v, o, lse, do, rope_fused=True)
    qr, kr = pvj.rope2d_apply(plan, q), pvj.rope2d_apply(plan, k)
    g2 = pvj.varlen_attn_bwd(plan, qr, kr, v, o, lse, do, rope_prerotated=True)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    with pytest.raises(pvj.PvjError):
        pvj.varlen_attn_bwd(plan, q, k, v, o, lse, do, rope_fused=True, rope_prerotated=True)


def test_bwd_fused_chain_step_vs_oracle():
    # the training step composition: pack_rope(Q), pack_rope(K), pack(V) ->
    # forward without flags -> backward PREROTATED -> unpack; against the
    # oracle's gradients with respect to the un-rotated Q, K
    H, D, dt = 2, 128, "bf16"
    plan = _plan(RAGGED, H, D, dt)
    say("fused-chain step vs oracle")
    q, k, v, do = draw_tensors(plan.n_tokens, H, D, dt, 91, n=4)
    streams = [oracle.unpack_joint(x, RAGGED) for x in (q, k, v, do)]
    dev = [(to_dev(t, dt), to_dev(i, dt)) for (t, i) in streams]
    qr = pvj.pack(plan, *dev[0], rope=True)
    kr = pvj.pack(plan, *dev[1], rope=True)
    vj = pvj.pack(plan, *dev[2])
    dj = pvj.pack(plan, *dev[3])
    o, lse = pvj.varlen_attn_fwd(plan, qr, kr, vj)
    dq, dk, dv = pvj.varlen_attn_bwd(plan, qr, kr, vj, o, lse, dj, rope_prerotated=True)
    torch.cuda.synchronize()
    ro, _ = oracle.attn_fwd(q, k, v, RAGGED, rope=True)
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, RAGGED, rope=True)
    assert_close("o", to_np(o), ro, dt)
    assert_close("dq", to_np(dq), rq, dt)
    assert_close("dk", to_np(dk), rk, dt)
    assert_close("dv", to_np(dv), rv, dt)


@pytest.mark.parametrize("D", [128, 64])
def test_fwd_bwd_tile_boundaries(D):
    # sample lengths on either side of the work-item tiles (bf16: 256 queries
    # per forward / dQ workgroup, 128 keys per dK/dV workgroup, 64-key and
    # 32-query streamed tiles), text-only and image samples mixed
    samples = [(0, 0, 255), (0, 0, 256), (0, 0, 257), (16, 16, 0), (16, 16, 1), (0, 0, 127),
               (0, 0, 129), (8, 8, 447), (0, 0, 31), (0, 0, 33), (16, 32, 0)]
    H, dt = 2, "bf16"
    plan = _plan(samples, H, D, dt)
    say("fwd+bwd tile boundaries D=%d T=%d" % (D, plan.n_tokens))
    q, k, v, do = draw_tensors(plan.n_tokens, H, D, dt, 97, n=4)
    o, _, dq, dk, dv = _fwd_bwd(plan, *(to_dev(x, dt) for x in (q, k, v, do)), True, dt)
    ro, _ = oracle.attn_fwd(q, k, v, samples, rope=True)
    assert_close("o", to_np(o), ro, dt)
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, samples, rope=True)
    assert_close("dq", to_np(dq), rq, dt)
    assert_close("dk", to_np(dk), rk, dt)
    assert_close("dv", to_np(dv), rv, dt)
