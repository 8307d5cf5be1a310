"""GPU parity of the projections with the modality pack / unpack fused in
(QKV projection writing joint Q, K, V rows with RoPE; output projection
reading the stream's rows of the joint O) against the oracle, through the C ABI.

Identity weights reduce them exactly to pack + RoPE and unpack, so those cases
are compared bitwise with the library's own pack kernels; random weights are
compared with the fp64 oracle (bf16 operands, fp32 accumulation, one rounding);
at the backbone width (hidden 3072, 24 x 128 heads) sampled rows are checked.
"""
import numpy as np
import pytest

import oracle
from oracle import projection
from pvj_inputs import workload

from helpers import assert_close, say, to_dev, to_np

torch = pytest.importorskip("torch")
pvj = pytest.importorskip("packed_varlen_joint_amd")

pytestmark = pytest.mark.gpu

PACK = [(0, 0, 0), (3, 5, 7), (1, 1, 0), (0, 0, 1), (9, 17, 33), (0, 0, 130), (2, 40, 3),
        (12, 12, 0), (5, 0, 4)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pvj.load_library()


def _rand(shape, seed, scale=1.0):
    x = np.random.default_rng(seed).standard_normal(shape) * scale
    d = to_dev(x, "bf16")
    return d, to_np(d)


def test_identity_weights_equal_pack_rope_and_unpack():
    H, D = 2, 64
    HD = H * D
    plan = pvj.Plan(PACK, H, D, "bf16").upload()
    say("qkv/out projections with identity weights vs pack kernels (bitwise)")
    xt, _ = _rand((plan.n_text, HD), 1)
    xi, _ = _rand((plan.n_image, HD), 2)
    eye3 = torch.cat([torch.eye(HD)] * 3).to(torch.bfloat16).cuda().contiguous()
    q, k, v = pvj.qkv_proj_pack(plan, "text", xt, eye3, rope=True)
    pvj.qkv_proj_pack(plan, "image", xi, eye3, q=q, k=k, v=v, rope=True)
    torch.cuda.synchronize()
    t3, i3 = xt.view(-1, H, D), xi.view(-1, H, D)
    assert torch.equal(q, pvj.pack(plan, t3, i3, rope=True))
    assert torch.equal(k, q)
    assert torch.equal(v, pvj.pack(plan, t3, i3))
    eye = torch.eye(HD).to(torch.bfloat16).cuda().contiguous()
    yt = pvj.out_proj_unpack(plan, "text", v, eye)
    yi = pvj.out_proj_unpack(plan, "image", v, eye)
    torch.cuda.synchronize()
    assert torch.equal(yt, xt) and torch.equal(yi, xi)


@pytest.mark.parametrize("C,rope,frames", [(64, True, False), (192, True, False),
                                           (128, False, False), (128, True, True)])
def test_qkv_and_out_projection_vs_oracle(C, rope, frames):
    H, D = 2, 64
    HD = H * D
    samples = [s + (2,) for s in PACK] if frames else PACK
    plan = pvj.Plan(samples, H, D, "bf16").upload()
    say("projections C=%d rope=%d frames=%d" % (C, rope, frames))
    xt, xtn = _rand((plan.n_text, C), 3)
    xi, xin = _rand((plan.n_image, C), 4)
    wt, wtn = _rand((3 * HD, C), 5, C ** -0.5)
    wi, win = _rand((3 * HD, C), 6, C ** -0.5)
    bt, btn = _rand((3 * HD,), 7, 0.1)
    bi, bin_ = _rand((3 * HD,), 8, 0.1)
    q, k, v = pvj.qkv_proj_pack(plan, "text", xt, wt, bt, rope=rope)
    pvj.qkv_proj_pack(plan, "image", xi, wi, bi, q=q, k=k, v=v, rope=rope)
    torch.cuda.synchronize()
    rq, rk, rv = projection.qkv_project_pack(xtn, xin, wtn, btn, win, bin_, samples, H, D,
                                             rope=rope, axes=3 if frames else 2)
    assert_close("q", to_np(q), rq, "bf16")
    assert_close("k", to_np(k), rk, "bf16")
    assert_close("v", to_np(v), rv, "bf16")
    # output projection from a joint O
    o, on = _rand((plan.n_tokens, H, D), 9)
    ot, otn = _rand((C, HD), 10, HD ** -0.5)
    oi, oin = _rand((C, HD), 11, HD ** -0.5)
    ob, obn = _rand((C,), 12, 0.1)
    yt = pvj.out_proj_unpack(plan, "text", o, ot, ob)
    yi = pvj.out_proj_unpack(plan, "image", o, oi, ob)
    torch.cuda.synchronize()
    ryt, ryi = projection.out_project_unpack(on, otn, obn, oin, obn, samples)
    assert_close("y_text", to_np(yt), ryt, "bf16")
    assert_close("y_image", to_np(yi), ryi, "bf16")


@pytest.mark.parametrize("which", ["image", "text"])
def test_projection_backbone_width_sampled(which):
    # the training pack's streams at hidden 3072 (24 heads x 128): sampled rows
    # of Q, K, V and of the output projection against the oracle
    wl = workload("train_64k")
    H, D = wl.n_heads, wl.head_dim
    HD, C = H * D, H * D
    plan = pvj.Plan(wl.samples, H, D, "bf16").upload()
    n = plan.n_image if which == "image" else plan.n_text
    say("projections train_64k %s stream rows=%d hidden=%d" % (which, n, C))
    g = torch.Generator(device="cuda").manual_seed(3 if which == "image" else 4)
    x = torch.randn(n, C, device="cuda", generator=g).to(torch.bfloat16)
    w = (torch.randn(3 * HD, C, device="cuda", generator=g) * C ** -0.5).to(torch.bfloat16)
    b = (torch.randn(3 * HD, device="cuda", generator=g) * 0.1).to(torch.bfloat16)
    q = torch.zeros(plan.n_tokens, H, D, dtype=torch.bfloat16, device="cuda")
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    pvj.qkv_proj_pack(plan, which, x, w, b, q=q, k=k, v=v, rope=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 40)]))
    # joint rows and positions of the sampled stream rows
    cu = oracle.cu_seqlens(wl.samples)
    sizes = [s[0] * s[1] if which == "image" else s[2] for s in wl.samples]
    starts = np.cumsum([0] + sizes)
    jrows = []
    for r in rows:
        i = int(np.searchsorted(starts, r, side="right") - 1)
        skip = wl.samples[i][2] if which == "image" else 0
        jrows.append(int(cu[i]) + skip + int(r - starts[i]))
    jrows = np.array(jrows)
    pos = oracle.token_positions(wl.samples)[jrows]
    y = projection.linear(to_np(x[rows]), to_np(w), to_np(b))
    for part, t in enumerate((q, k, v)):
        ref = y[:, part * HD:(part + 1) * HD].reshape(-1, H, D)
        if part < 2:
            ref = oracle.rope2d_at(ref, pos)
        assert_close("qkv"[part], to_np(t[jrows]), ref, "bf16")
    wo = (torch.randn(C, HD, device="cuda", generator=g) * HD ** -0.5).to(torch.bfloat16)
    yo = pvj.out_proj_unpack(plan, which, q, wo)
    torch.cuda.synchronize()
    ref = projection.linear(to_np(q[jrows]).reshape(len(jrows), HD), to_np(wo))
    assert_close("y", to_np(yo[rows]), ref, "bf16")


def test_projection_errors():
    plan32 = pvj.Plan(PACK, 2, 64, "f32").upload()
    lib = pvj.load_library()
    # fp32 plans, bad stream, hidden not a multiple of 64: rejected before any launch
    assert lib.pvj_qkv_proj_pack(plan32.handle, 0, 64, 16, 16, None, 16, 16, 16, 0, None) == 2
    plan = pvj.Plan(PACK, 2, 64, "bf16").upload()
    assert lib.pvj_qkv_proj_pack(plan.handle, 5, 64, 16, 16, None, 16, 16, 16, 0, None) == 1
    assert lib.pvj_out_proj_unpack(plan.handle, 0, 96, 16, 16, None, 16, None) == 2
