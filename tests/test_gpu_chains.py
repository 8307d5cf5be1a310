"""GPU parity of the memory-bound chains around the attention (adaptive layer
norm + modulation, gate + residual; forward and backward) against the oracle,
through the C ABI.

Row outputs are compared element by element; the per-sample parameter
gradients (fp32 sums over a sample's rows) against a bound scaled by the sum
of the absolute terms, since their error is fp32 summation error.  Both
streams in one call give the rows of the one-stream calls bit for bit, and
NaN rows of one sample reach no other sample's rows or sums.  Packs hold
empty, text-only and image-only samples and editing samples with frames; the
hidden sizes span the minimum (8), a ragged 8-column tail of a 512-column
reduction chunk, the backbone width (24 heads x 128 = 3072) and the maximum
(8192).
"""
import numpy as np
import pytest

from oracle import chains
from pvj_inputs import workload

from helpers import say, to_dev, to_np

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


def _draw(rows, cols, dt, seed, scale=1.0, shift=0.0):
    x = np.random.default_rng(seed).standard_normal((rows, cols)) * scale + shift
    d = to_dev(x, dt)
    return d, to_np(d)  # the oracle consumes exactly the rounded values


def _rel_bound(got, ref, dt, extra=0.0):
    tol = 2.0 ** -8 if dt == "bf16" else 2e-6
    err = np.abs(got - ref)
    bound = tol * np.abs(ref) + (1e-5 if dt == "bf16" else 1e-6) + extra
    say("   max_abs=%.3e (worst excess %.3e)" % (err.max() if err.size else 0,
                                                 (err - bound).max() if err.size else 0))
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound)


def _seg_sum(vals, si, B):
    # rows of a stream are in sample order: sum each sample's contiguous block
    out = np.zeros((B,) + vals.shape[1:])
    for b in range(B):
        sel = np.nonzero(si == b)[0]
        if sel.size:
            out[b] = vals[sel[0]:sel[-1] + 1].sum(axis=0)
    return out


def _sum_bound(got, ref, abs_sum):
    # fp32 sums of up to a few thousand terms: relative to the sum of |terms|
    err = np.abs(got - ref)
    bound = 2e-5 * abs_sum + 1e-6
    say("   sum max_abs=%.3e (bound min %.3e)" % (err.max() if err.size else 0,
                                                  bound.min() if bound.size else 0))
    assert np.all(err <= bound)


# 2568 and 2600 columns: the paired LayerNorm backward (2,561-3,072 columns)
# with a partial last unit per lane
CASES = [("bf16", 3072, "image"), ("bf16", 3072, "text"), ("bf16", 8, "image"),
         ("bf16", 520, "text"), ("f32", 64, "image"), ("f32", 8192, "text"),
         ("bf16", 8192, "image"), ("bf16", 2568, "image"), ("f32", 2600, "text")]


@pytest.mark.parametrize("dt,C,which", CASES)
def test_adaln_fwd_bwd(dt, C, which):
    say("adaln dt=%s hidden=%d stream=%s" % (dt, C, which))
    plan = pvj.Plan(PACK, 2, 64, dt).upload()
    rows = plan.n_text if which == "text" else plan.n_image
    st = chains.TEXT if which == "text" else chains.IMAGE
    B = len(PACK)
    x, xn = _draw(rows, C, dt, 1, 2.0, 0.5)
    sh, shn = _draw(B, C, dt, 2, 0.5)
    sc, scn = _draw(B, C, dt, 3, 0.5)
    dy, dyn = _draw(rows, C, dt, 4)
    y = pvj.adaln_modulate(plan, which, x, sh, sc)
    torch.cuda.synchronize()
    _rel_bound(to_np(y), chains.adaln_modulate(xn, shn, scn, PACK, st), dt)
    dx, dsh, dsc = pvj.adaln_modulate_bwd(plan, which, x, sc, dy)
    torch.cuda.synchronize()
    rdx, rdsh, rdsc = chains.adaln_modulate_bwd(xn, scn, dyn, PACK, st)
    ref_scale = np.abs(rdx).max() if rdx.size else 1.0
    _rel_bound(to_np(dx), rdx, dt, extra=(2e-3 if dt == "bf16" else 1e-5) * ref_scale)
    si = chains.stream_sample_index(PACK, st)
    xhat = chains.layer_norm_rows(xn)
    abs_sh = _seg_sum(np.abs(dyn), si, B)
    abs_sc = _seg_sum(np.abs(dyn * xhat), si, B)
    _sum_bound(to_np(dsh), rdsh, abs_sh)
    _sum_bound(to_np(dsc), rdsc, abs_sc)
    # deterministic: a second call gives the same bits
    dx2, dsh2, dsc2 = pvj.adaln_modulate_bwd(plan, which, x, sc, dy)
    torch.cuda.synchronize()
    assert torch.equal(dx, dx2) and torch.equal(dsh, dsh2) and torch.equal(dsc, dsc2)
    # in place forward
    xc = x.clone()
    pvj.adaln_modulate(plan, which, xc, sh, sc, y=xc)
    torch.cuda.synchronize()
    assert torch.equal(xc, y)


@pytest.mark.parametrize("dt,C,which", CASES)
def test_gate_residual_fwd_bwd(dt, C, which):
    say("gate dt=%s hidden=%d stream=%s" % (dt, C, which))
    plan = pvj.Plan(PACK, 2, 64, dt).upload()
    rows = plan.n_text if which == "text" else plan.n_image
    st = chains.TEXT if which == "text" else chains.IMAGE
    B = len(PACK)
    x, xn = _draw(rows, C, dt, 5)
    y, yn = _draw(rows, C, dt, 6)
    g, gn = _draw(B, C, dt, 7)
    dout, dn = _draw(rows, C, dt, 8)
    out = pvj.gate_residual(plan, which, x, y, g)
    torch.cuda.synchronize()
    _rel_bound(to_np(out), chains.gate_residual(xn, yn, gn, PACK, st), dt,
               extra=(2.0 ** -8 if dt == "bf16" else 2e-6) * np.abs(gn).max() * 4)
    dy, dg = pvj.gate_residual_bwd(plan, which, y, g, dout)
    torch.cuda.synchronize()
    _, rdy, rdg = chains.gate_residual_bwd(yn, gn, dn, PACK, st)
    _rel_bound(to_np(dy), rdy, dt)
    si = chains.stream_sample_index(PACK, st)
    abs_g = _seg_sum(np.abs(dn * yn), si, B)
    _sum_bound(to_np(dg), rdg, abs_g)
    # in place: out may be x
    xc = x.clone()
    pvj.gate_residual(plan, which, xc, y, g, out=xc)
    torch.cuda.synchronize()
    assert torch.equal(xc, out)


def test_chains_frames_pack():
    # an editing pack (samples with 0..3 frames): the image stream holds every frame
    samples = [(3, 5, 7, 2), (0, 0, 3, 0), (2, 4, 0, 3), (4, 4, 9, 1)]
    plan = pvj.Plan(samples, 2, 64, "bf16").upload()
    C, B, st = 256, len(samples), chains.IMAGE
    rows = plan.n_image
    assert rows == 3 * 5 * 2 + 2 * 4 * 3 + 16
    x, xn = _draw(rows, C, "bf16", 31)
    sh, shn = _draw(B, C, "bf16", 32, 0.3)
    sc, scn = _draw(B, C, "bf16", 33, 0.3)
    g, gn = _draw(B, C, "bf16", 34)
    y = pvj.adaln_modulate(plan, "image", x, sh, sc)
    out = pvj.gate_residual(plan, "image", x, y, g)
    torch.cuda.synchronize()
    ry = chains.adaln_modulate(xn, shn, scn, samples, st)
    _rel_bound(to_np(y), ry, "bf16")
    _rel_bound(to_np(out), chains.gate_residual(xn, to_np(y), gn, samples, st), "bf16",
               extra=2.0 ** -8 * np.abs(gn).max() * 4)


def test_chains_edit_workload_full():
    # the editing pack's image stream (two source/target pairs, 14336 rows) at
    # the backbone width, against the oracle on every row
    wl = workload("edit_1024")
    plan = pvj.Plan(wl.samples, wl.n_heads, wl.head_dim, "bf16").upload()
    C = wl.n_heads * wl.head_dim
    rows, B = plan.n_image, len(wl.samples)
    say("chains edit_1024 image stream rows=%d hidden=%d" % (rows, C))
    x, xn = _draw(rows, C, "bf16", 21)
    sh, shn = _draw(B, C, "bf16", 22, 0.3)
    sc, scn = _draw(B, C, "bf16", 23, 0.3)
    y = pvj.adaln_modulate(plan, "image", x, sh, sc)
    dy, dyn = _draw(rows, C, "bf16", 24)
    dx, dsh, dsc = pvj.adaln_modulate_bwd(plan, "image", x, sc, dy)
    torch.cuda.synchronize()
    _rel_bound(to_np(y), chains.adaln_modulate(xn, shn, scn, wl.samples, chains.IMAGE), "bf16")
    rdx, rdsh, rdsc = chains.adaln_modulate_bwd(xn, scn, dyn, wl.samples, chains.IMAGE)
    _rel_bound(to_np(dx), rdx, "bf16", extra=2e-3 * np.abs(rdx).max())
    si = chains.stream_sample_index(wl.samples, chains.IMAGE)
    abs_sh = _seg_sum(np.abs(dyn), si, B)
    abs_sc = _seg_sum(np.abs(dyn * chains.layer_norm_rows(xn)), si, B)
    _sum_bound(to_np(dsh), rdsh, abs_sh)
    _sum_bound(to_np(dsc), rdsc, abs_sc)


def test_chain_errors():
    plan = pvj.Plan(PACK, 2, 64, "bf16").upload()
    x = torch.zeros(plan.n_image, 12, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(len(PACK), 12, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pvj.PvjError):   # hidden not a multiple of 8
        pvj.adaln_modulate(plan, "image", x, v, v)
    lib = pvj.load_library()
    # stream selector 3 is refused before any launch (0, 1, 2: text, image, both)
    assert lib.pvj_adaln_modulate(plan.handle, 3, 64, 16, 16, 16, 16, 1e-6, None) == 1
    assert lib.pvj_gate_residual(plan.handle, 0, 16384, 16, 16, 16, 16, None) == 2


# both streams in one call: (dtype, hidden, pack); the hidden sizes take the
# paired LayerNorm backward (3072), the one-wave ones (520, 64) and the wide
# rows' range-split sums (8192)
BOTH_CASES = [("bf16", 3072, "mixed"), ("bf16", 520, "mixed"), ("f32", 64, "mixed"),
              ("bf16", 8192, "mixed"), ("bf16", 3072, "text_only"),
              ("bf16", 3072, "image_only"), ("bf16", 2568, "frames")]
BOTH_PACKS = {"mixed": PACK, "text_only": [(0, 0, 37), (0, 0, 5)],
              "image_only": [(7, 9, 0), (3, 4, 0), (0, 0, 0)],
              # an editing pack: samples of 0 to 3 frames
              "frames": [(3, 5, 7, 2), (0, 0, 3, 0), (2, 4, 0, 3), (4, 4, 9, 1)]}


@pytest.mark.parametrize("dt,C,pack", BOTH_CASES)
def test_chains_both_streams(dt, C, pack):
    # one call over [text rows; image rows] with per-sample vectors [2B, C]:
    # the row outputs equal the two one-stream calls bit for bit; the
    # parameter gradients hold the oracle's sums (another fixed order) and
    # repeat bit for bit
    samples = BOTH_PACKS[pack]
    say("chains both streams dt=%s hidden=%d pack=%s" % (dt, C, pack))
    plan = pvj.Plan(samples, 2, 64, dt).upload()
    nt, ni, B = plan.n_text, plan.n_image, len(samples)
    x, xn = _draw(nt + ni, C, dt, 41, 2.0, 0.5)
    y, yn = _draw(nt + ni, C, dt, 42)
    dy, dyn = _draw(nt + ni, C, dt, 43)
    sh, shn = _draw(2 * B, C, dt, 44, 0.5)
    sc, scn = _draw(2 * B, C, dt, 45, 0.5)
    g, gn = _draw(2 * B, C, dt, 46)
    parts = (("text", slice(0, nt), slice(0, B), chains.TEXT),
             ("image", slice(nt, nt + ni), slice(B, 2 * B), chains.IMAGE))

    a = pvj.adaln_modulate(plan, "both", x, sh, sc)
    o = pvj.gate_residual(plan, "both", x, y, g)
    dx, dsh, dsc = pvj.adaln_modulate_bwd(plan, "both", x, sc, dy)
    gy, dg = pvj.gate_residual_bwd(plan, "both", y, g, dy)
    torch.cuda.synchronize()
    for name, rs, vs, st in parts:
        if rs.stop == rs.start:
            continue
        say("  %s stream" % name)
        xs, ys, ds = x[rs].contiguous(), y[rs].contiguous(), dy[rs].contiguous()
        assert torch.equal(a[rs], pvj.adaln_modulate(plan, name, xs, sh[vs].contiguous(),
                                                     sc[vs].contiguous()))
        assert torch.equal(o[rs], pvj.gate_residual(plan, name, xs, ys, g[vs].contiguous()))
        ref_dx, _, _ = pvj.adaln_modulate_bwd(plan, name, xs, sc[vs].contiguous(), ds)
        ref_gy, _ = pvj.gate_residual_bwd(plan, name, ys, g[vs].contiguous(), ds)
        torch.cuda.synchronize()
        assert torch.equal(dx[rs], ref_dx)
        assert torch.equal(gy[rs], ref_gy)
        # the parameter gradients against the oracle
        xn_s, yn_s, dn_s = xn[rs], yn[rs], dyn[rs]
        _, rdsh, rdsc = chains.adaln_modulate_bwd(xn_s, scn[vs], dn_s, samples, st)
        _, _, rdg = chains.gate_residual_bwd(yn_s, gn[vs], dn_s, samples, st)
        si = chains.stream_sample_index(samples, st)
        xhat = chains.layer_norm_rows(xn_s)
        _sum_bound(to_np(dsh[vs]), rdsh, _seg_sum(np.abs(dn_s), si, B))
        _sum_bound(to_np(dsc[vs]), rdsc, _seg_sum(np.abs(dn_s * xhat), si, B))
        _sum_bound(to_np(dg[vs]), rdg, _seg_sum(np.abs(dn_s * yn_s), si, B))
    # segments without rows get zero gradients
    for name, rs, vs, st in parts:
        if rs.stop == rs.start:
            assert not bool(dsh[vs].any()) and not bool(dsc[vs].any()) and not bool(dg[vs].any())
    dx2, dsh2, dsc2 = pvj.adaln_modulate_bwd(plan, "both", x, sc, dy)
    gy2, dg2 = pvj.gate_residual_bwd(plan, "both", y, g, dy)
    torch.cuda.synchronize()
    for u, w in ((dx, dx2), (dsh, dsh2), (dsc, dsc2), (gy, gy2), (dg, dg2)):
        assert torch.equal(u, w)


@pytest.mark.parametrize("which", ["both", "image"])
def test_chain_nan_rows_stay_in_their_sample(which):
    # Sample 1's rows are NaN: every other sample's rows and parameter
    # gradients must be finite and bitwise those of the same call with
    # sample 1 finite (a slot's sums hold the rows of one sample only)
    samples = [(9, 17, 33), (3, 4, 50), (0, 0, 70), (5, 7, 60), (6, 6, 0)]
    C, B = 3072, len(samples)
    plan = pvj.Plan(samples, 2, 64, "bf16").upload()
    nt, ni = plan.n_text, plan.n_image
    say("chain NaN isolation stream=%s" % which)
    rows, nv = (nt + ni, 2 * B) if which == "both" else (ni, B)
    x, _ = _draw(rows, C, "bf16", 51, 2.0, 0.5)
    y, _ = _draw(rows, C, "bf16", 52)
    dy, _ = _draw(rows, C, "bf16", 53)
    sc, _ = _draw(nv, C, "bf16", 54, 0.5)
    g, _ = _draw(nv, C, "bf16", 55)
    # rows of sample 1 in this call's row order, and the rows of the others
    tcu = np.concatenate([[0], np.cumsum([s[2] for s in samples])])
    icu = np.concatenate([[0], np.cumsum([s[0] * s[1] for s in samples])])
    def rows_of(i):
        img = np.arange(icu[i], icu[i + 1]) + (nt if which == "both" else 0)
        txt = np.arange(tcu[i], tcu[i + 1]) if which == "both" else np.arange(0)
        return np.concatenate([txt, img]).astype(np.int64)
    bad = torch.as_tensor(rows_of(1), device="cuda")
    good = [i for i in range(B) if i != 1]
    vec = lambda i: [i, B + i] if which == "both" else [i]

    def run(poison):
        xs, ys, ds = x.clone(), y.clone(), dy.clone()
        if poison:
            for t in (xs, ys, ds):
                t[bad] = float("nan")
        dx, dsh, dsc = pvj.adaln_modulate_bwd(plan, which, xs, sc, ds)
        gy, dg = pvj.gate_residual_bwd(plan, which, ys, g, ds)
        a = pvj.adaln_modulate(plan, which, xs, sc, sc)
        o = pvj.gate_residual(plan, which, xs, ys, g)
        torch.cuda.synchronize()
        return (dx, gy, a, o), (dsh, dsc, dg)

    (r0, p0), (r1, p1) = run(False), run(True)
    for i in good:
        rr = torch.as_tensor(rows_of(i), device="cuda")
        for a, b in zip(r0, r1):
            assert bool(torch.isfinite(b[rr].float()).all())
            assert torch.equal(a[rr], b[rr])
        for a, b in zip(p0, p1):
            for j in vec(i):
                assert bool(torch.isfinite(b[j]).all())
                assert torch.equal(a[j], b[j])
