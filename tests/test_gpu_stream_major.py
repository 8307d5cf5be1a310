"""GPU checks of the stream-major layout (all samples' text rows, then all
their image rows) through the C ABI.

In this layout the attention kernels run the same products and sums in the
same order as in the joint layout; only the row addresses differ.  So every
output must equal, bit for bit, the joint-layout output of the same rows, and
the joint layout is held to the oracle by the other GPU tests.  Covered here:
ragged packs with text-only and image-only samples, tiles that straddle the
text/image boundary at every offset, forward tiles split over key ranges, both
head dims, the standalone RoPE, the pre-rotated backward, the allocation-free
backward, the full training pack, NaN rows of one sample that must not reach
the others, and a small pack checked against the oracle directly.
"""
import numpy as np
import pytest

import oracle
from pvj_inputs import draw_tensors, workload, workload_tensors

from helpers import Guarded, assert_close, assert_lse, say, to_dev, to_np

torch = pytest.importorskip("torch")
pvj = pytest.importorskip("packed_varlen_joint_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pvj.load_library()


def _plan(samples, H, D, dt="bf16"):
    return pvj.Plan(samples, H, D, dt).upload()


# text-only, image-only and empty samples; text lengths that put the
# text/image boundary at many offsets inside 32-, 64- and 256-row tiles
RAGGED = [(0, 0, 0), (3, 5, 7), (1, 1, 0), (0, 0, 1), (9, 17, 33), (0, 0, 130), (2, 64, 3),
          (12, 12, 0), (5, 0, 4), (7, 9, 61), (4, 4, 255), (6, 11, 17)]
# lengths 2,110, 1,100, 4,365 and 2,061: forward tiles split into 2 to 4 key ranges
SPLIT = [(40, 52, 30), (0, 0, 1100), (66, 66, 9), (31, 64, 77)]


def _to_sm(x, perm):
    y = torch.empty_like(x)
    y[perm] = x
    return y


def _run(plan, q, k, v, do, sm, prerot):
    o, lse = pvj.varlen_attn_fwd(plan, q, k, v, stream_major=sm)
    T, H, D = plan.n_tokens, plan.n_heads, plan.head_dim
    g = [Guarded(T, H, D, "bf16") for _ in range(3)]
    pvj.varlen_attn_bwd(plan, q, k, v, o, lse, do, dq=g[0].t, dk=g[1].t, dv=g[2].t,
                        rope_prerotated=prerot, stream_major=sm)
    torch.cuda.synchronize()
    for name, x in zip(("dq", "dk", "dv"), g):
        x.check(name)
    return o, lse, g[0].t, g[1].t, g[2].t


# packs with an empty image stream or an empty text stream
TEXT_ONLY = [(0, 0, 37), (0, 0, 300), (0, 0, 1)]
IMAGE_ONLY = [(7, 9, 0), (16, 20, 0), (1, 1, 0)]
PACKS = {"ragged": RAGGED, "split": SPLIT, "text_only": TEXT_ONLY, "image_only": IMAGE_ONLY}


@pytest.mark.parametrize("D,pack", [(128, "ragged"), (64, "ragged"), (128, "split"),
                                    (64, "split"), (128, "text_only"), (128, "image_only")])
def test_sm_bitwise_equals_joint(D, pack):
    samples = PACKS[pack]
    H = 2 if pack == "split" else 3
    plan = _plan(samples, H, D)
    T = plan.n_tokens
    say("stream-major vs joint %s D=%d T=%d" % (pack, D, T))
    perm = pvj.stream_major_rows(plan).cuda()
    q, k, v, do = (to_dev(x, "bf16") for x in draw_tensors(T, H, D, "bf16", 77 + D, n=4))
    for prerot in (False, True):
        ref = _run(plan, q, k, v, do, False, prerot)
        sm = _run(plan, *(_to_sm(x, perm) for x in (q, k, v, do)), True, prerot)
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), ref, sm):
            got = b[:, perm] if name == "lse" else b[perm]
            say("   prerotated=%d %s" % (prerot, name))
            assert torch.equal(got, a), name + " differs from the joint layout"
    # the allocation-free backward in the stream-major layout: same bits
    qs, ks, vs, dos = (_to_sm(x, perm) for x in (q, k, v, do))
    o, lse = pvj.varlen_attn_fwd(plan, qs, ks, vs, stream_major=True)
    want = pvj.varlen_attn_bwd(plan, qs, ks, vs, o, lse, dos, stream_major=True)
    got = [torch.empty_like(q) for _ in range(3)]
    pvj.varlen_attn_bwd_noalloc(plan, qs, ks, vs, o, lse, dos, *got, stream_major=True)
    torch.cuda.synchronize()
    for a, b in zip(want, got):
        assert torch.equal(a, b)


# an editing pack: samples of several frames (3-axis RoPE: row, column, frame)
FRAMES = [(3, 4, 5, 2), (0, 0, 7, 1), (2, 6, 0, 3), (5, 5, 33, 2), (1, 1, 1, 1)]


@pytest.mark.parametrize("dt,D,pack", [("bf16", 128, "ragged"), ("bf16", 64, "ragged"),
                                       ("f32", 64, "ragged"), ("bf16", 128, "frames"),
                                       ("bf16", 128, "text_only"), ("bf16", 128, "image_only")])
def test_sm_rope_bitwise_equals_joint(dt, D, pack):
    H = 3
    samples = FRAMES if pack == "frames" else PACKS[pack]
    plan = _plan(samples, H, D, dt)
    say("stream-major rope dt=%s D=%d pack=%s" % (dt, D, pack))
    perm = pvj.stream_major_rows(plan).cuda()
    x, = draw_tensors(plan.n_tokens, H, D, dt, 5, n=1)
    xd = to_dev(x, dt)
    xs = _to_sm(xd, perm)
    for inverse in (False, True):
        ref = pvj.rope2d_apply(plan, xd, inverse=inverse)
        y = Guarded(plan.n_tokens, H, D, dt)
        pvj.rope2d_apply(plan, xs, y.t, inverse=inverse, stream_major=True)
        torch.cuda.synchronize()
        y.check("rope2d stream-major")
        assert torch.equal(y.t[perm], ref)
    z = xs.clone()
    pvj.rope2d_apply(plan, z, z, stream_major=True)     # in place
    assert torch.equal(z[perm], pvj.rope2d_apply(plan, xd))


def test_sm_vs_oracle_rope_step():
    # standalone RoPE on the stream-major Q, K, attention forward, and the
    # pre-rotated backward, against the oracle's fused-RoPE attention
    samples = [(3, 5, 7), (0, 0, 20), (9, 17, 33), (6, 6, 0), (2, 30, 45)]
    H, D, dt = 3, 128, "bf16"
    plan = _plan(samples, H, D, dt)
    T = plan.n_tokens
    say("stream-major rope step vs oracle T=%d" % T)
    perm = pvj.stream_major_rows(plan).cuda()
    q, k, v, do = draw_tensors(T, H, D, dt, 913, n=4)
    qs, ks, vs, dos = (_to_sm(to_dev(x, dt), perm) for x in (q, k, v, do))
    qr = pvj.rope2d_apply(plan, qs, stream_major=True)
    kr = pvj.rope2d_apply(plan, ks, stream_major=True)
    o, lse = pvj.varlen_attn_fwd(plan, qr, kr, vs, stream_major=True)
    dq, dk, dv = pvj.varlen_attn_bwd(plan, qr, kr, vs, o, lse, dos, rope_prerotated=True,
                                     stream_major=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attn_fwd(q, k, v, samples, rope=True)
    rq, rk, rv = oracle.attn_bwd(q, k, v, do, samples, rope=True)
    assert_close("o", to_np(o[perm]), ro, dt)
    assert_lse(to_np(lse[:, perm]), rl, dt)
    assert_close("dq", to_np(dq[perm]), rq, dt)
    assert_close("dk", to_np(dk[perm]), rk, dt)
    assert_close("dv", to_np(dv[perm]), rv, dt)


def _nan_margin(rows, H, D, margin=256):
    full = torch.full((rows + margin, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    return full[:rows]


def test_sm_nan_rows_stay_in_their_sample():
    # Sample 1's text and image rows are NaN; in the stream-major layout they
    # follow sample 0's text rows and sample 0's image rows, so a tile of
    # sample 0 that read past its text run or its image run would pick them
    # up; NaN rows also follow the tensor.  The other samples' outputs must be
    # finite and bitwise those of the same call with sample 1 finite.
    samples = [(9, 17, 33), (3, 4, 50), (0, 0, 70), (5, 7, 60), (40, 52, 30), (2, 3, 0)]
    H, D = 2, 128
    plan = _plan(samples, H, D)
    T = plan.n_tokens
    cu = plan.cu_seqlens
    say("stream-major NaN isolation T=%d" % T)
    perm = pvj.stream_major_rows(plan).cuda()
    src = [_to_sm(to_dev(x, "bf16"), perm) for x in draw_tensors(T, H, D, "bf16", 171, n=4)]
    bad_rows = perm[cu[1]:cu[2]]

    def run(poison):
        t = [_nan_margin(T, H, D) for _ in range(4)]
        for dst, x in zip(t, src):
            dst.copy_(x)
            if poison:
                dst[bad_rows] = float("nan")
        o, lse = pvj.varlen_attn_fwd(plan, t[0], t[1], t[2], stream_major=True)
        o_m = _nan_margin(T, H, D)
        o_m.copy_(o)
        g = pvj.varlen_attn_bwd(plan, t[0], t[1], t[2], o_m, lse, t[3], stream_major=True)
        torch.cuda.synchronize()
        return (o, lse) + tuple(g)

    clean, bad = run(False), run(True)
    for i in (0, 2, 3, 4, 5):
        rows = perm[cu[i]:cu[i + 1]]
        say("  sample %d (%d rows)" % (i, len(rows)))
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), clean, bad):
            x = b[:, rows] if name == "lse" else b[rows]
            y = a[:, rows] if name == "lse" else a[rows]
            assert bool(torch.isfinite(x.float()).all()), name + " not finite"
            assert torch.equal(x, y), name + " depends on another sample's rows"


def test_sm_bitwise_train_pack():
    # the training pack at full size (about 65K tokens, 24 heads of 128)
    wl = workload("train_64k", 0)
    plan = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    say("stream-major vs joint train_64k T=%d samples=%d" % (wl.n_tokens, len(wl.samples)))
    perm = pvj.stream_major_rows(plan).cuda()
    q, k, v, do = (to_dev(x, "bf16") for x in workload_tensors(wl, 4))
    ref = _run(plan, q, k, v, do, False, True)
    sm = _run(plan, *(_to_sm(x, perm) for x in (q, k, v, do)), True, True)
    for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), ref, sm):
        got = b[:, perm] if name == "lse" else b[perm]
        say("   %s" % name)
        assert torch.equal(got, a), name + " differs from the joint layout"


def test_sm_bitwise_inference_pack():
    # the multi-prompt CFG inference pack (12 samples, ~87K tokens), forward
    wl = workload("infer_multi", 0)
    plan = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    say("stream-major vs joint infer_multi T=%d samples=%d" % (wl.n_tokens, len(wl.samples)))
    perm = pvj.stream_major_rows(plan).cuda()
    q, k, v = (to_dev(x, "bf16") for x in workload_tensors(wl, 3))
    o, lse = pvj.varlen_attn_fwd(plan, q, k, v)
    o_s, lse_s = pvj.varlen_attn_fwd(plan, *(_to_sm(x, perm) for x in (q, k, v)),
                                     stream_major=True)
    torch.cuda.synchronize()
    assert torch.equal(o_s[perm], o)
    assert torch.equal(lse_s[:, perm], lse)
