"""The allocation-free attention backward (static scratch buffer, no workspace
argument) against the entry point that takes a caller workspace: the same
kernels, so the same bits, on two calls in a row, the second with a smaller
pack (the scratch keeps the first call's contents), plus its limits.
"""
import numpy as np
import pytest

from pvj_inputs import draw_tensors

from helpers import say, to_dev

torch = pytest.importorskip("torch")
pvj = pytest.importorskip("packed_varlen_joint_amd")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pvj.load_library()


def _case(samples, H, D, seed, prerotated):
    plan = pvj.Plan(samples, H, D, "bf16").upload()
    q, k, v, do = (to_dev(x, "bf16") for x in draw_tensors(plan.n_tokens, H, D, "bf16", seed, n=4))
    if prerotated:
        q, k = pvj.rope2d_apply(plan, q), pvj.rope2d_apply(plan, k)
    o, lse = pvj.varlen_attn_fwd(plan, q, k, v)
    ref = pvj.varlen_attn_bwd(plan, q, k, v, o, lse, do, rope_prerotated=prerotated)
    out = [torch.full_like(q, float("nan")) for _ in range(3)]
    got = pvj.varlen_attn_bwd_noalloc(plan, q, k, v, o, lse, do, *out,
                                      rope_prerotated=prerotated)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("prerotated", [True, False])
def test_noalloc_bwd_equals_workspace_bwd(prerotated):
    # first a larger pack (24 heads, ~9.6K tokens), then a smaller one
    cases = [([(64, 64, 256), (48, 80, 300), (20, 30, 77)], 24, 128, 11),
             ([(9, 17, 33), (0, 0, 100), (5, 7, 60)], 2, 128, 12)]
    for samples, H, D, seed in cases:
        say("noalloc bwd prerotated=%d H=%d samples=%s" % (prerotated, H, samples))
        ref, got = _case(samples, H, D, seed, prerotated)
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert bool(torch.isfinite(a.float()).all()), name
            assert torch.equal(a, b), name + " differs from the workspace entry point"


def test_noalloc_bwd_limits():
    # rejected before anything is enqueued: RoPE on load, and H * T above the
    # fixed scratch (Delta of 4,194,304 floats)
    lib = pvj.load_library()
    plan = pvj.Plan([(8, 8, 8)], 2, 128, "bf16").upload()
    t = torch.zeros(plan.n_tokens, 2, 128, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(2, plan.n_tokens, dtype=torch.float32, device="cuda")
    p = [x.data_ptr() for x in (t, t, t, t, lse, t, t, t, t)]
    assert lib.pvj_varlen_attn_bwd_noalloc(plan.handle, *p, 0.0, 1, None) == 2
    big = pvj.Plan([(128, 128, 0)] * 8, 33, 128, "bf16").upload()   # 33 x 131,072 > 4 Mi
    assert lib.pvj_varlen_attn_bwd_noalloc(big.handle, *p, 0.0, 0, None) == 5
