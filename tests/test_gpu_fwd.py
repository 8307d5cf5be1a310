"""GPU parity of the forward path (pack/unpack, standalone 2D RoPE, varlen
attention forward) against the CPU oracle, through the C ABI.

Full-tensor comparison at sizes the oracle finishes in seconds (several tiles,
ragged tails, empty and one-token samples); at the full workload sizes,
sampled (sample, head, rows) outputs the oracle computes one by one, plus
bitwise properties that hold at any size (determinism, single sample ==
unpacked, permutation equivariance, the CFG pack == two separate calls).
"""
import numpy as np
import pytest

import oracle
from pvj_inputs import draw_tensors, random_small_pack, workload, workload_tensors

from helpers import (Guarded, GuardedLse, assert_close, assert_lse, say, to_dev, to_np)

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


# ----------------------------------------------------------------------------
# standalone RoPE and pack/unpack
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dt,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_rope2d_apply(dt, D):
    say("rope2d_apply dt=%s D=%d ragged pack" % (dt, D))
    H = 3
    plan = _plan(RAGGED, H, D, dt)
    T = plan.n_tokens
    x, = draw_tensors(T, H, D, dt, 5, n=1)
    xd = to_dev(x, dt)
    ref = oracle.rope2d(x, RAGGED)
    for inverse in (False, True):
        ref = oracle.rope2d(x, RAGGED, inverse=inverse)
        y = Guarded(T, H, D, dt)
        pvj.rope2d_apply(plan, xd, y.t, inverse=inverse)
        torch.cuda.synchronize()
        y.check("rope2d")
        got = to_np(y.t)
        bound = (2.0 ** -8 * np.abs(ref) + 1e-5) if dt == "bf16" else 1e-5
        err = np.abs(got - ref)
        say("   inverse=%d max_abs=%.3e" % (inverse, err.max()))
        assert np.all(err <= bound)
    # in place, then inverse in place returns to x within rounding
    z = xd.clone()
    pvj.rope2d_apply(plan, z, z)
    pvj.rope2d_apply(plan, z, z, inverse=True)
    back = to_np(z)
    assert np.abs(back - x).max() <= (0.03 * np.abs(x).max() if dt == "bf16" else 1e-5)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_pack_unpack_bit_exact(dt):
    say("pack/unpack dt=%s" % dt)
    H, D = 3, 64
    plan = _plan(RAGGED, H, D, dt)
    text, image = draw_tensors(plan.n_text, H, D, dt, 1, n=1)[0], \
        draw_tensors(plan.n_image, H, D, dt, 2, n=1)[0]
    ref = oracle.pack_joint(text, image, RAGGED)
    j = Guarded(plan.n_tokens, H, D, dt)
    pvj.pack(plan, to_dev(text, dt), to_dev(image, dt), j.t)
    torch.cuda.synchronize()
    j.check("pack")
    assert np.array_equal(to_np(j.t), ref)
    t2, i2 = pvj.unpack(plan, j.t)
    assert np.array_equal(to_np(t2), text) and np.array_equal(to_np(i2), image)


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f32", 64)])
def test_pack_rope_fused_chain(dt, D):
    # pack + RoPE in one pass == pack, then the standalone RoPE (bitwise), and
    # matches the oracle's rotation of the packed tensor; unpack_rope likewise
    say("pack_rope / unpack_rope dt=%s D=%d" % (dt, D))
    H = 3
    plan = _plan(RAGGED, H, D, dt)
    text = to_dev(draw_tensors(plan.n_text, H, D, dt, 6, n=1)[0], dt)
    image = to_dev(draw_tensors(plan.n_image, H, D, dt, 7, n=1)[0], dt)
    for inverse in (False, True):
        j = Guarded(plan.n_tokens, H, D, dt)
        pvj.pack(plan, text, image, j.t, rope=True, inverse=inverse)
        two = pvj.rope2d_apply(plan, pvj.pack(plan, text, image), inverse=inverse)
        torch.cuda.synchronize()
        j.check("pack_rope")
        assert torch.equal(j.t, two)
        ref = oracle.rope2d(oracle.pack_joint(to_np(text), to_np(image), RAGGED),
                            RAGGED, inverse=inverse)
        bound = (2.0 ** -8 * np.abs(ref) + 1e-5) if dt == "bf16" else 1e-5
        assert np.all(np.abs(to_np(j.t) - ref) <= bound)
        t2, i2 = pvj.unpack(plan, j.t, rope=True, inverse=not inverse)
        t3, i3 = pvj.unpack(plan, pvj.rope2d_apply(plan, j.t, inverse=not inverse))
        assert torch.equal(t2, t3) and torch.equal(i2, i3)


def test_fwd_on_prerotated_pack_equals_fused():
    # the forward on pack_rope's output (no flags) gives the bits of the
    # forward with RoPE on load: both round R x to bf16 the same way
    H, D, dt = 2, 128, "bf16"
    plan = _plan(RAGGED, H, D, dt)
    say("fwd on pack_rope output == fused RoPE fwd")
    tq, iq, tk, ik, tv, iv = (to_dev(draw_tensors(n, H, D, dt, 60 + s, n=1)[0], dt)
                              for s, n in enumerate([plan.n_text, plan.n_image] * 3))
    q, k, v = pvj.pack(plan, tq, iq), pvj.pack(plan, tk, ik), pvj.pack(plan, tv, iv)
    o1, l1 = pvj.varlen_attn_fwd(plan, q, k, v, rope_fused=True)
    qr, kr = pvj.pack(plan, tq, iq, rope=True), pvj.pack(plan, tk, ik, rope=True)
    o2, l2 = pvj.varlen_attn_fwd(plan, qr, kr, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_pack_large_bit_exact():
    wl = workload("train_64k", 1)
    say("pack/unpack train_64k seed 1, T=%d" % wl.n_tokens)
    plan = _plan(wl.samples, wl.n_heads, wl.head_dim, "bf16")
    g = torch.Generator(device="cuda").manual_seed(0)
    text = torch.randn(plan.n_text, 24, 128, device="cuda", generator=g).to(torch.bfloat16)
    image = torch.randn(plan.n_image, 24, 128, device="cuda", generator=g).to(torch.bfloat16)
    joint = pvj.pack(plan, text, image)
    # reference by slicing (torch ops on the device, not the oracle)
    parts, ta, ia = [], 0, 0
    for (h, w, t) in wl.samples:
        parts += [text[ta:ta + t], image[ia:ia + h * w]]
        ta += t
        ia += h * w
    assert torch.equal(joint, torch.cat(parts))
    t2, i2 = pvj.unpack(plan, joint)
    assert torch.equal(t2, text) and torch.equal(i2, image)
    # with RoPE at full size (most blocks lie inside one sample): the one-pass
    # kernels equal pack then the standalone rotation, bit for bit, and the
    # standalone rotation matches the oracle on sampled rows
    say("pack/unpack with RoPE train_64k seed 1")
    jr = pvj.rope2d_apply(plan, joint)
    assert torch.equal(pvj.pack(plan, text, image, rope=True), jr)
    t3, i3 = pvj.unpack(plan, jr, rope=True, inverse=True)
    t4, i4 = pvj.unpack(plan, pvj.rope2d_apply(plan, jr, inverse=True))
    assert torch.equal(t3, t4) and torch.equal(i3, i4)
    rows = np.random.default_rng(3).choice(plan.n_tokens, 512, replace=False)
    rows.sort()
    pos = oracle.token_positions(wl.samples)[rows]
    ref = oracle.rope2d_at(to_np(joint[torch.as_tensor(rows, device="cuda")]), pos)
    got = to_np(jr[torch.as_tensor(rows, device="cuda")])
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-5)


# ----------------------------------------------------------------------------
# forward, full comparison on small packs
# ----------------------------------------------------------------------------

def _fwd(plan, q, k, v, rope, dt):
    o = Guarded(plan.n_tokens, plan.n_heads, plan.head_dim, dt)
    lse = GuardedLse(plan.n_heads, plan.n_tokens)
    pvj.varlen_attn_fwd(plan, q, k, v, rope_fused=rope, out=o.t, lse=lse.t)
    torch.cuda.synchronize()
    o.check("o")
    lse.check()
    return o.t, lse.t


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("rope", [False, True])
def test_fwd_ragged_pack(dt, D, rope):
    say("fwd ragged pack dt=%s D=%d rope=%d" % (dt, D, rope))
    H = 3
    plan = _plan(RAGGED, H, D, dt)
    q, k, v = draw_tensors(plan.n_tokens, H, D, dt, 11, n=3)
    o, lse = _fwd(plan, to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), rope, dt)
    ro, rl = oracle.attn_fwd(q, k, v, RAGGED, rope=rope)
    assert_close("o", to_np(o), ro, dt)
    assert_lse(to_np(lse), rl, dt)


@pytest.mark.parametrize("seed", range(4))
def test_fwd_random_packs(seed):
    rng = np.random.default_rng(300 + seed)
    samples = random_small_pack(rng, int(rng.integers(1, 9)), max_side=24, max_text=200)
    dt = "bf16"
    D = 128
    H = 2
    say("fwd random pack seed=%d samples=%s" % (seed, samples))
    plan = _plan(samples, H, D, dt)
    q, k, v = draw_tensors(plan.n_tokens, H, D, dt, seed, n=3)
    if plan.n_tokens == 0:
        return
    o, lse = _fwd(plan, to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), True, dt)
    ro, rl = oracle.attn_fwd(q, k, v, samples, rope=True)
    assert_close("o", to_np(o), ro, dt)
    assert_lse(to_np(lse), rl, dt)


@pytest.mark.parametrize("rope", [False, True])
def test_fwd_tiny_f32_workload(rope):
    wl = workload("tiny_f32")
    say("fwd tiny_f32 rope=%d" % rope)
    plan = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    q, k, v = workload_tensors(wl, 3)
    dq, dk, dv = (to_dev(x, "f32") for x in (q, k, v))
    if rope:
        o, lse = _fwd(plan, dq, dk, dv, True, "f32")
    else:
        # standalone RoPE, then attention on the rotated Q, K
        qr, kr = pvj.rope2d_apply(plan, dq), pvj.rope2d_apply(plan, dk)
        o, lse = _fwd(plan, qr, kr, dv, False, "f32")
    ro, rl = oracle.attn_fwd(q, k, v, wl.samples, rope=True)
    assert_close("o", to_np(o), ro, "f32")
    assert_lse(to_np(lse), rl, "f32")


def test_fwd_edge_values():
    # Q = 0: uniform attention, O = mean of V per sample, LSE = ln L
    samples = [(3, 7, 5), (1, 1, 0), (0, 0, 3)]
    H, D = 2, 128
    plan = _plan(samples, H, D, "bf16")
    T = plan.n_tokens
    _, k, v = draw_tensors(T, H, D, "bf16", 3, n=3)
    q = np.zeros_like(k)
    say("fwd edge values Q=0")
    o, lse = _fwd(plan, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), True, "bf16")
    ro, rl = oracle.attn_fwd(q, k, v, samples, rope=True)
    assert_close("o", to_np(o), ro, "bf16")
    assert_lse(to_np(lse), rl, "bf16")
    # large logits: scores of magnitude ~100 must not overflow the online softmax
    q, k, v = draw_tensors(T, H, D, "bf16", 4, n=3)
    q = (q * 8).astype(np.float32)
    from pvj_inputs import round_bf16
    q = round_bf16(q)
    o, lse = _fwd(plan, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), False, "bf16")
    ro, rl = oracle.attn_fwd(q, k, v, samples)
    assert_close("o", to_np(o), ro, "bf16")
    assert_lse(to_np(lse), rl, "bf16")


# Samples long enough that the last query tile of each (sample, head) is cut
# into key ranges whose partial states are merged: 2110 (2 parts, last query
# tile 62 rows), 1100 (not split), 4365 (4 parts, last query tile 13 rows,
# last key tile 13 keys), 2061 (2 parts).
SPLIT = [(40, 52, 30), (0, 0, 1100), (66, 66, 9), (31, 64, 77)]


@pytest.mark.parametrize("D", [128, 64])
def test_fwd_split_tiles(D):
    H, dt = 2, "bf16"
    plan = _plan(SPLIT, H, D, dt)
    assert len(plan.work_items(3)[0]) == 3 * H
    say("fwd split tiles D=%d T=%d" % (D, plan.n_tokens))
    q, k, v = draw_tensors(plan.n_tokens, H, D, dt, 17, n=3)
    qd, kd, vd = (to_dev(x, dt) for x in (q, k, v))
    # RoPE on load (one-group kernel) and on pre-rotated Q/K (phase-shifted
    # kernel): same key ranges, same partial states, same bits
    o1, l1 = _fwd(plan, qd, kd, vd, True, dt)
    o2, l2 = _fwd(plan, pvj.rope2d_apply(plan, qd), pvj.rope2d_apply(plan, kd), vd, False, dt)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ro, rl = oracle.attn_fwd(q, k, v, SPLIT, rope=True)
    assert_close("o", to_np(o1), ro, dt)
    assert_lse(to_np(l1), rl, dt)
    # a split sample alone: same bits; without an LSE output: same O
    cu = plan.cu_seqlens
    a, b = cu[2], cu[3]
    p1 = _plan([SPLIT[2]], H, D, dt)
    oi, li = pvj.varlen_attn_fwd(p1, qd[a:b].contiguous(), kd[a:b].contiguous(),
                                 vd[a:b].contiguous(), rope_fused=True)
    assert torch.equal(oi, o1[a:b]) and torch.equal(li, l1[:, a:b])
    o3 = torch.empty_like(o1)
    lib = pvj.load_library()
    st = lib.pvj_varlen_attn_fwd(plan.handle, qd.data_ptr(), kd.data_ptr(), vd.data_ptr(),
                                 o3.data_ptr(), None, 0.0, 1,
                                 torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0 and torch.equal(o3, o1)


# ----------------------------------------------------------------------------
# bitwise properties
# ----------------------------------------------------------------------------

def test_fwd_bitwise_properties():
    samples = [(9, 17, 33), (12, 12, 0), (3, 5, 7), (0, 0, 130)]
    H, D, dt = 2, 128, "bf16"
    plan = _plan(samples, H, D, dt)
    q, k, v = (to_dev(x, dt) for x in draw_tensors(plan.n_tokens, H, D, dt, 21, n=3))
    say("fwd bitwise: determinism, single == unpacked, permutation")
    o1, l1 = pvj.varlen_attn_fwd(plan, q, k, v, rope_fused=True)
    o2, l2 = pvj.varlen_attn_fwd(plan, q, k, v, rope_fused=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    cu = plan.cu_seqlens
    for i, s in enumerate(samples):
        a, b = cu[i], cu[i + 1]
        p1 = _plan([s], H, D, dt)
        oi, li = pvj.varlen_attn_fwd(p1, q[a:b].contiguous(), k[a:b].contiguous(),
                                     v[a:b].contiguous(), rope_fused=True)
        assert torch.equal(oi, o1[a:b]) and torch.equal(li, l1[:, a:b])
    perm = [2, 0, 3, 1]
    idx = torch.cat([torch.arange(cu[i], cu[i + 1]) for i in perm]).cuda()
    pp = _plan([samples[i] for i in perm], H, D, dt)
    op, lp = pvj.varlen_attn_fwd(pp, q[idx].contiguous(), k[idx].contiguous(),
                                 v[idx].contiguous(), rope_fused=True)
    assert torch.equal(op, o1[idx]) and torch.equal(lp, l1[:, idx])


# ----------------------------------------------------------------------------
# full-size workloads (the bench launch configuration), sampled outputs
# ----------------------------------------------------------------------------

def _sampled_rows(wl, q, k, v, o, lse, rng, n_pairs, n_rows, rope=True):
    cu = oracle.cu_seqlens(wl.samples)
    nz = [i for i in range(len(wl.samples)) if cu[i + 1] > cu[i]]
    on, ln_ = to_np(o), to_np(lse)
    for _ in range(n_pairs):
        i = int(rng.choice(nz))
        h = int(rng.integers(0, wl.n_heads))
        L = int(cu[i + 1] - cu[i])
        rows = np.unique(np.concatenate([[0, L - 1], rng.integers(0, L, size=n_rows)]))
        ro, rl = oracle.attn_fwd_rows(q, k, v, wl.samples, i, h, rows, rope=rope)
        say("  sample %d (L=%d) head %d rows %d" % (i, L, h, len(rows)))
        assert_close("o", on[cu[i] + rows, h], ro, wl.dtype)
        assert_lse(ln_[h, cu[i] + rows], rl, wl.dtype)


def test_fwd_single_1024_full_heads():
    wl = workload("single_1024")
    say("fwd single_1024 T=%d" % wl.n_tokens)
    plan = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    q, k, v = workload_tensors(wl, 3)
    o, lse = _fwd(plan, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), True, "bf16")
    # three full heads against the oracle
    for h in (0, 11, 23):
        sl = slice(h, h + 1)
        ro, rl = oracle.attn_fwd(q[:, sl], k[:, sl], v[:, sl], wl.samples, rope=True)
        say("  head %d" % h)
        assert_close("o", to_np(o[:, sl]), ro, "bf16")
        assert_lse(to_np(lse[sl]), rl, "bf16")


def test_fwd_cfg_pack_equals_two_calls():
    wl = workload("cfg_1024")
    say("fwd cfg_1024 T=%d" % wl.n_tokens)
    plan = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    q, k, v = workload_tensors(wl, 3)
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    o, lse = _fwd(plan, qd, kd, vd, True, "bf16")
    cu = plan.cu_seqlens
    for i, s in enumerate(wl.samples):
        a, b = cu[i], cu[i + 1]
        p1 = _plan([s], wl.n_heads, wl.head_dim, "bf16")
        oi, li = pvj.varlen_attn_fwd(p1, qd[a:b].contiguous(), kd[a:b].contiguous(),
                                     vd[a:b].contiguous(), rope_fused=True)
        assert torch.equal(oi, o[a:b]) and torch.equal(li, lse[:, a:b])
    _sampled_rows(wl, q, k, v, o, lse, np.random.default_rng(0), 4, 96)


@pytest.mark.parametrize("name,seed", [("train_64k", 0), ("train_64k", 1), ("extreme", 0)])
def test_fwd_large_workloads_sampled(name, seed):
    wl = workload(name, seed)
    say("fwd %s T=%d samples=%d" % (name, wl.n_tokens, len(wl.samples)))
    plan = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    q, k, v = workload_tensors(wl, 3)
    o, lse = _fwd(plan, to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), True, "bf16")
    _sampled_rows(wl, q, k, v, o, lse, np.random.default_rng(1), 6, 64)


def test_fwd_multi_prompt_cfg_pack():
    # several prompts, each a cond/uncond pair sharing its image rows, in one
    # inference pack: every pair's rows equal a call on that pair alone
    # (bitwise), the uncond image rows see the same queries as the cond ones,
    # and sampled rows match the oracle
    wl = workload("infer_multi")
    say("fwd infer_multi T=%d prompts=%d" % (wl.n_tokens, len(wl.shared_image)))
    plan = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    q, k, v = workload_tensors(wl, 3)
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    o, lse = _fwd(plan, qd, kd, vd, True, "bf16")
    cu = plan.cu_seqlens
    for (c, u) in wl.shared_image[:3]:
        a, b = cu[c], cu[u + 1]
        p2 = _plan(wl.samples[c:u + 1], wl.n_heads, wl.head_dim, "bf16")
        o2, l2 = pvj.varlen_attn_fwd(p2, qd[a:b].contiguous(), kd[a:b].contiguous(),
                                     vd[a:b].contiguous(), rope_fused=True)
        torch.cuda.synchronize()
        assert torch.equal(o2, o[a:b]) and torch.equal(l2, lse[:, a:b])
    _sampled_rows(wl, q, k, v, o, lse, np.random.default_rng(5), 6, 48)


def test_diag_mfma_peak_runs():
    # the matrix-core ceiling probe runs and reports a plausible rate
    # (well above what the attention kernels reach, at most the chip's peak)
    tf = pvj.diag_mfma_peak(rounds=1, iters=2000, reps=1)
    say("measured matrix-core ceiling (small run): %.0f TFLOP/s" % tf)
    assert 500.0 < tf < 2600.0
    lib = pvj.load_library()
    import ctypes
    f = ctypes.c_double()
    assert lib.pvj_diag_mfma_peak(0, 10, 16, 1 << 20, ctypes.byref(f), None) == 1
