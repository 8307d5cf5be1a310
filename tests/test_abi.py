"""C-ABI library checks that need no GPU: the library loads, exports every
symbol the header declares, and its pure-host planner is right (offsets, RoPE
tables, work-list coverage and order, error codes).  No compute call is made.
"""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
from pvj_inputs import WORKLOADS, workload, random_small_pack

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pvj = pytest.importorskip("packed_varlen_joint_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pvj.library_path()):
        pytest.fail("libpvj.so is not built (python -m packed_varlen_joint_amd._build)")
    return pvj.load_library()


def test_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "pvj.h")).read()
    declared = re.findall(r"PVJ_API\s+[\w\s\*]+?\b(pvj_\w+)\s*\(", header)
    assert len(declared) >= 15
    raw = ctypes.CDLL(pvj.library_path())
    for name in declared:
        assert hasattr(raw, name), name
    assert lib.pvj_version().decode().startswith("pvj")


def _plan(samples, H=2, D=64, dtype="f32"):
    return pvj.Plan(samples, H, D, dtype)


@pytest.mark.parametrize("name", WORKLOADS)
def test_plan_offsets_match_oracle(lib, name):
    wl = workload(name)
    p = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    assert p.cu_seqlens == oracle.cu_seqlens(wl.samples).tolist()
    assert p.n_tokens == wl.n_tokens
    assert p.max_len == max(oracle.sample_lengths(wl.samples))


def _expected_splits(p, L):
    # the forward's tail split: the last query tile of a (sample, head) of a
    # sample of at most 8192 tokens is cut into parts of >= 16 key tiles of 64,
    # at most 4, bf16 plans only; the count depends on the sample length alone
    if p.dtype_code != pvj.PVJ_BF16 or L > 8192:
        return 1
    return max(1, min(4, int(math.ceil(L / 64)) // 16))


def _check_work_list(p, samples, which):
    items, tile = p.work_items(which)
    lens = oracle.sample_lengths(samples)
    assert len(items) % 8 == 0
    ranges = {}
    group_xcd = {}
    cost = {x: [] for x in range(8)}
    for b, (s, h, t, split) in enumerate(items):
        if s < 0:
            continue
        assert 0 <= s < len(samples) and 0 <= h < p.n_heads
        assert 0 <= t * tile < lens[s]
        L = int(lens[s])
        nkt = int(math.ceil(L / 64))
        if split == 0:
            kr = (0, nkt)
        else:
            # only forward items are split, and only the last query tile
            assert which == 0 and t == int(math.ceil(L / tile)) - 1
            S, j = (split & 15) + 1, (split >> 4) & 15
            assert S == _expected_splits(p, L) >= 2 and j < S
            kr = (nkt * j // S, nkt * (j + 1) // S)
        ranges.setdefault((s, h, t), []).append((kr, split))
        # every tile of a (sample, head) lands on the same XCD (slot % 8)
        assert group_xcd.setdefault((s, h), b % 8) == b % 8
        cost[b % 8].append(min(kr[1] * 64, L) - kr[0] * 64)
    want = {(s, h, t) for s in range(len(samples)) for h in range(p.n_heads)
            for t in range(int(math.ceil(lens[s] / tile)))}
    assert set(ranges) == want
    slots = []
    for (s, h, t), rs in ranges.items():
        # the key ranges of a tile partition its sample's key tiles
        rs.sort()
        assert rs[0][0][0] == 0 and rs[-1][0][1] == int(math.ceil(lens[s] / 64))
        assert all(a[0][1] == b[0][0] for a, b in zip(rs, rs[1:]))
        if which == 0 and t == int(math.ceil(lens[s] / tile)) - 1:
            assert len(rs) == _expected_splits(p, int(lens[s]))
        if len(rs) > 1:
            assert len({r[1] >> 8 for r in rs}) == 1
            slots.append((rs[0][1] >> 8, len(rs), (s, h, t)))
    if which == 0:
        # partial-result slots of the split tiles are disjoint and dense
        slots.sort()
        at = 0
        for first, n, _ in slots:
            assert first == at
            at += n
        split_list, _ = p.work_items(3)
        assert sorted(((it[3] >> 8), (it[3] & 15) + 1, tuple(it[:3])) for it in split_list) == slots
    for x in range(8):
        # inside each XCD the costlier items run first (LPT)
        c = cost[x]
        assert all(a >= b for a, b in zip(c, c[1:]))
        # idle slots only at the end of an XCD's list
        flags = [s >= 0 for (s, _, _, _) in items[x::8]]
        assert flags == sorted(flags, reverse=True)


@pytest.mark.parametrize("name", WORKLOADS)
def test_work_lists_cover_every_tile_once(lib, name):
    wl = workload(name)
    p = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    for which in (0, 1, 2):
        _check_work_list(p, wl.samples, which)


def test_work_lists_random_packs(lib):
    rng = np.random.default_rng(0)
    for _ in range(20):
        samples = random_small_pack(rng, int(rng.integers(0, 12)), max_side=40, max_text=300)
        p = _plan(samples, int(rng.integers(1, 5)), 128, "bf16")
        for which in (0, 1, 2):
            _check_work_list(p, samples, which)


def test_forward_split_depends_on_the_sample_only(lib):
    # a sample's forward items (tile, key range) are the same in any pack, and
    # the metadata buffer holds one partial-result slot per split part
    a, b = (40, 52, 30), (66, 66, 9)
    H, D = 2, 128
    def parts(p, s):
        items, _ = p.work_items(0)
        return sorted((h, t, it & 0xFF) for (ss, h, t, it) in items if ss == s)
    alone = _plan([b], H, D, "bf16")
    pack = _plan([a, (0, 0, 5), b], H, D, "bf16")
    assert parts(alone, 0) == parts(pack, 2)
    n_slots = sum((it[3] & 15) + 1 for it in pack.work_items(3)[0])
    assert n_slots == H * (2 + 4)
    assert pack.meta_bytes > n_slots * (D + 2) * 256 * 4
    # fp32 plans split nothing
    assert _plan([a, (0, 0, 5), b], H, D, "f32").work_items(3)[0] == []


def test_work_list_xcd_balance(lib):
    # the (sample, head) groups are dealt so no XCD carries much more than its share
    wl = workload("train_64k", 3)
    p = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    items, tile = p.work_items(2)  # the forward tiles, unsplit
    lens = oracle.sample_lengths(wl.samples)
    load = [sum(int(lens[s]) for (s, h, t, _) in items[x::8] if s >= 0) for x in range(8)]
    assert max(load) <= 1.10 * (sum(load) / 8)


def _oracle_pair_angle(D, axes, pos, k):
    """(cos, sin) the oracle gives pair k at position `pos` on pair k's axis:
    rotate the unit vector e_{2k} and read dims 2k, 2k+1."""
    dims = oracle.rope_axis_dims(D, axes)
    x = np.zeros((1, 1, D))
    x[0, 0, 2 * k] = 1.0
    a = int(np.searchsorted(np.cumsum(dims), 2 * k, side="right"))  # axis of dim 2k
    p = np.zeros((1, axes), dtype=np.int64)
    p[0, a] = pos
    y = oracle.rope_nd_at(x, p, dims)
    return y[0, 0, 2 * k], y[0, 0, 2 * k + 1]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("axes", [2, 3])
def test_rope_tables(lib, D, axes):
    samples = [(37, 5, 3), (2, 90, 1)] if axes == 2 else [(37, 5, 3, 3), (2, 90, 1, 100)]
    p = _plan(samples, 1, D)
    cos_t, sin_t, npos, npairs = p.rope_table()
    assert npos == (90 if axes == 2 else 100) and npairs == D // 2
    assert p.rope_axes() == (axes, tuple(oracle.rope_axis_dims(D, axes)))
    for pos in (0, 1, 17, 89):
        for k in range(npairs):
            c, s_ = _oracle_pair_angle(D, axes, pos, k)
            assert abs(cos_t[pos * npairs + k] - c) <= 6e-8
            assert abs(sin_t[pos * npairs + k] - s_) <= 6e-8


def test_frames_plan_offsets_and_work_lists(lib):
    rng = np.random.default_rng(5)
    for _ in range(10):
        samples = random_small_pack(rng, int(rng.integers(0, 9)), max_side=30, max_text=200,
                                    max_frames=3)
        p = _plan(samples, int(rng.integers(1, 4)), 128, "bf16")
        assert p.frames and p.rope_axes()[0] == 3
        assert p.cu_seqlens == oracle.cu_seqlens(samples).tolist()
        assert p.n_image == sum(h * w * f for (h, w, t, f) in samples)
        _check_work_list(p, samples, 0)
        _check_work_list(p, samples, 1)
    # a triple plan forced to frames mode is the one-frame editing plan
    p = pvj.Plan([(4, 5, 6)], 2, 64, "f32", frames=True)
    assert p.samples == [(4, 5, 6, 1)] and p.rope_axes()[0] == 3
    with pytest.raises(ValueError):
        pvj.Plan([(4, 5, 6, 2)], 2, 64, "f32", frames=False)


@pytest.mark.parametrize("name", ["edit_1024"])
def test_edit_workload_plan(lib, name):
    wl = workload(name)
    p = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    assert p.n_tokens == wl.n_tokens == int(oracle.sample_lengths(wl.samples).sum())
    assert p.rope_axes() == (3, (56, 56, 16))


def test_empty_and_degenerate_packs(lib):
    p = _plan([])
    assert p.n_tokens == 0 and p.cu_seqlens == [0]
    assert p.work_items(0)[0] == [] and p.work_items(1)[0] == []
    p = _plan([(0, 0, 0), (3, 0, 2), (0, 5, 0), (1, 1, 0)])
    assert p.cu_seqlens == [0, 0, 2, 2, 3]
    _check_work_list(p, [(0, 0, 0), (3, 0, 2), (0, 5, 0), (1, 1, 0)], 0)


def _create(lib, samples, H=2, D=64, dtype=0, theta=1e4, pairing=0, text_first=1):
    arr = (pvj._Sample * max(1, len(samples)))(*[pvj._Sample(*s) for s in samples])
    desc = pvj._Desc(H, D, dtype, theta, pairing, text_first)
    h = ctypes.c_void_p()
    st = lib.pvj_plan_create(arr, len(samples), ctypes.byref(desc), ctypes.byref(h))
    if st == 0:
        lib.pvj_plan_destroy(h)
    return st


def _create_frames(lib, samples, H=2, D=64):
    arr = (pvj._SampleFrames * max(1, len(samples)))(*[pvj._SampleFrames(*s) for s in samples])
    desc = pvj._Desc(H, D, 0, 1e4, 0, 1)
    h = ctypes.c_void_p()
    st = lib.pvj_plan_create_frames(arr, len(samples), ctypes.byref(desc), ctypes.byref(h))
    if st == 0:
        lib.pvj_plan_destroy(h)
    return st


def test_error_codes(lib):
    INVALID, UNSUP, OVERFLOW = 1, 2, 3
    assert _create(lib, [(1, 1, 1)]) == 0
    assert _create(lib, [(-1, 1, 1)]) == INVALID
    assert _create(lib, [(1, 1, -3)]) == INVALID
    assert _create(lib, [(1, 1, 1)], H=0) == INVALID
    assert _create(lib, [(1, 1, 1)], D=96) == UNSUP
    assert _create(lib, [(1, 1, 1)], dtype=7) == UNSUP
    assert _create(lib, [(1, 1, 1)], pairing=1) == UNSUP
    assert _create(lib, [(1, 1, 1)], text_first=0) == UNSUP
    assert _create(lib, [(1, 1, 1)], theta=-1.0) == INVALID
    assert _create(lib, [(32767, 2, 0)]) == 0
    assert _create(lib, [(32768, 2, 0)]) == UNSUP                  # latent side limit
    assert _create(lib, [(2, 40000, 0)]) == UNSUP
    assert _create(lib, [(4000, 4000, 0)] * 135, H=1) == OVERFLOW  # T > int32
    # one sample's span of a token tensor stays below 2 GiB (32-bit offsets)
    assert _create(lib, [(31, 33, 0)], H=4096, D=128, dtype=1) == 0    # 1023 rows x 2 MiB
    assert _create(lib, [(32, 32, 0)], H=4096, D=128, dtype=1) == UNSUP
    h = ctypes.c_void_p()
    assert lib.pvj_plan_create(None, 1, None, ctypes.byref(h)) == INVALID
    assert _create_frames(lib, [(2, 3, 4, 2)]) == 0
    assert _create_frames(lib, [(2, 3, 4, 0)]) == 0                # text only
    assert _create_frames(lib, [(2, 3, 4, -1)]) == INVALID
    assert _create_frames(lib, [(2, 3, 4, 32768)]) == UNSUP         # frame index limit
    assert _create_frames(lib, [(30000, 30000, 0, 3)]) == OVERFLOW
    assert _create_frames(lib, [(1, 1, 1, 1)], D=96) == UNSUP
    assert lib.pvj_status_string(5).decode() == "PVJ_ERR_WORKSPACE_TOO_SMALL"
    assert "int32" in lib.pvj_last_error().decode() or lib.pvj_last_error()


def test_compute_before_upload_is_rejected(lib):
    # validation happens before any device call: NOT_UPLOADED without touching HIP
    p = _plan([(2, 2, 1)], 1, 64, "f32")
    st = lib.pvj_varlen_attn_fwd(p.handle, 16, 16, 16, 16, None, 0.0, 0, None)
    assert st == 4
    assert lib.pvj_rope2d_apply(p.handle, 16, 16, 0, None) == 4
    assert lib.pvj_pack(p.handle, 16, 16, 16, None) == 4
    assert lib.pvj_unpack(p.handle, 16, 16, 16, None) == 4
    st = lib.pvj_varlen_attn_bwd(p.handle, 16, 16, 16, 16, 16, 16, 16, 16, 16, 256, 1 << 20,
                                 0.0, 0, None)
    assert st == 4
    assert lib.pvj_plan_upload(p.handle, None, 0, None) == 1
    assert lib.pvj_plan_upload(p.handle, 8, 1 << 20, None) == 1      # misaligned


def test_bwd_workspace_size(lib):
    # Delta fp32 [H, T], then room for the rotated Q' and K' in the plan dtype
    T, H, D = 11, 3, 64
    al = lambda x: (x + 255) // 256 * 256
    for dt, elt in (("f32", 4), ("bf16", 2)):
        p = _plan([(3, 3, 2)], H, D, dt)
        assert p.bwd_workspace_bytes() == al(T * H * 4) + 2 * al(T * H * D * elt)


def test_chain_workspace_streams(lib):
    # text, image and both streams in one call (the host-side query only)
    p = _plan([(3, 3, 2), (0, 0, 5), (4, 2, 0)], 2, 64, "bf16")
    sizes = {}
    for op in (0, 1):
        for which in (0, 1, 2):
            b = ctypes.c_size_t()
            assert lib.pvj_chain_bwd_workspace(p.handle, op, which, 3072, ctypes.byref(b)) == 0
            assert b.value > 0 and b.value % 256 == 0
            sizes[op, which] = b.value
        b = ctypes.c_size_t()
        assert lib.pvj_chain_bwd_workspace(p.handle, op, 3, 3072, ctypes.byref(b)) == 1
        assert lib.pvj_chain_bwd_workspace(p.handle, op, 2, 12, ctypes.byref(b)) == 2
    # both streams hold every row and twice the segments: no smaller than either
    for op in (0, 1):
        assert sizes[op, 2] >= max(sizes[op, 0], sizes[op, 1])
    # a both-streams call on a plan not yet uploaded is refused before any device call
    q = _plan([(3, 3, 2)], 1, 64, "bf16")
    assert lib.pvj_gate_residual(q.handle, 2, 64, 16, 16, 16, 16, None) == 4


def test_noalloc_bwd_limits_before_any_device_call(lib):
    # the allocation-free backward checks its fixed scratch size and flags
    # before touching HIP (the plan is not even uploaded here)
    too_big = _plan([(128, 128, 0)] * 8, 33, 128, "bf16")   # H * T = 4,325,376 floats
    fits = _plan([(128, 128, 0)] * 8, 32, 128, "bf16")      # exactly 16 MiB of Delta
    p = [16] * 9
    assert lib.pvj_varlen_attn_bwd_noalloc(too_big.handle, *p, 0.0, 0, None) == 5
    assert lib.pvj_varlen_attn_bwd_noalloc(fits.handle, *p, 0.0, 1, None) == 2   # ROPE_FUSED
    assert lib.pvj_varlen_attn_bwd_noalloc(fits.handle, *p, 0.0, 0, None) == 4   # not uploaded
    assert lib.pvj_varlen_attn_bwd_noalloc(None, *p, 0.0, 0, None) == 1


def test_stream_major_conditions_before_any_device_call(lib):
    # the stream-major layout (flag 4): bf16 plans, no RoPE on load, and
    # (T + 256) * H * D * 2 < 2^31; all checked before touching HIP
    SM, FUSED, PRE = 4, 1, 2
    f32 = _plan([(2, 2, 1)], 1, 64, "f32")
    bf = _plan([(2, 2, 1)], 1, 64, "bf16")
    p = [16] * 9
    assert lib.pvj_varlen_attn_fwd(f32.handle, 16, 16, 16, 16, None, 0.0, SM, None) == 2
    assert lib.pvj_varlen_attn_fwd(bf.handle, 16, 16, 16, 16, None, 0.0, SM | FUSED, None) == 2
    assert lib.pvj_varlen_attn_fwd(bf.handle, 16, 16, 16, 16, None, 0.0, SM, None) == 4
    assert lib.pvj_varlen_attn_fwd(bf.handle, 16, 16, 16, 16, None, 0.0, 8, None) == 1
    bwd = lambda plan, fl: lib.pvj_varlen_attn_bwd(plan.handle, 16, 16, 16, 16, 16, 16, 16, 16,
                                                   16, 256, 1 << 20, 0.0, fl, None)
    assert bwd(f32, SM | PRE) == 2
    assert bwd(bf, SM | FUSED) == 2
    assert bwd(bf, SM | PRE) == 4
    assert lib.pvj_varlen_attn_bwd_noalloc(f32.handle, *p, 0.0, SM, None) == 2
    assert lib.pvj_varlen_attn_bwd_noalloc(bf.handle, *p, 0.0, SM | PRE, None) == 4
    assert lib.pvj_rope2d_apply_stream_major(bf.handle, 16, 16, 0, None) == 4
    assert lib.pvj_rope2d_apply_stream_major(f32.handle, 16, 16, 0, None) == 4
    # 64 heads x 128 dims: 16 KiB per token, so T + 256 must stay below 131,072
    big = _plan([(256, 256, 0), (255, 256, 0)], 64, 128, "bf16")    # T = 130,816
    ok = _plan([(255, 256, 0), (256, 255, 0)], 64, 128, "bf16")     # T = 130,560
    assert lib.pvj_varlen_attn_fwd(big.handle, 16, 16, 16, 16, None, 0.0, SM, None) == 2
    assert "2^31" in lib.pvj_last_error().decode()
    assert lib.pvj_varlen_attn_fwd(big.handle, 16, 16, 16, 16, None, 0.0, 0, None) == 4
    assert lib.pvj_varlen_attn_fwd(ok.handle, 16, 16, 16, 16, None, 0.0, SM, None) == 4


def test_stream_major_row_map():
    # the binding's joint -> stream-major row map: text rows of all samples,
    # then image rows, each in sample order (zero-length parts included)
    import packed_varlen_joint_amd as pvj
    samples = [(2, 3, 5), (0, 0, 4), (1, 2, 0), (2, 2, 3), (0, 0, 0)]
    plan = pvj.Plan(samples, 2, 64, "bf16")
    perm = pvj.stream_major_rows(plan).tolist()
    want_text, want_img = [], []
    pos = 0
    for h, w, lt in samples:
        want_text += list(range(pos, pos + lt))
        want_img += list(range(pos + lt, pos + lt + h * w))
        pos += lt + h * w
    order = want_text + want_img   # joint row of each stream-major row
    assert sorted(perm) == list(range(plan.n_tokens))
    assert [order[r] for r in perm] == list(range(plan.n_tokens))
    assert plan.n_text == len(want_text) and plan.n_image == len(want_img)
    lib = pvj.load_library()
    buf = (ctypes.c_int32 * 4)()
    assert lib.pvj_plan_stream_major_rows(plan.handle, buf, plan.n_tokens + 1) == 1
    assert lib.pvj_plan_stream_major_rows(None, buf, 0) == 1
    empty = pvj.Plan([(0, 0, 0)], 1, 64, "bf16")
    assert lib.pvj_plan_stream_major_rows(empty.handle, None, 0) == 0
    # frames plans: each frame's grid follows the sample's text in the image rows
    fr = pvj.Plan([(2, 3, 4, 2), (1, 2, 0, 3), (0, 0, 5, 1)], 2, 64, "bf16")
    perm = pvj.stream_major_rows(fr).tolist()
    assert perm == [0, 1, 2, 3, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 19, 20,
                    21, 22, 23, 24, 25, 26, 4, 5, 6, 7, 8]


def test_chain_binding_checks_before_any_device_call(lib):
    # the binding refuses a bad stream name and tensors of the wrong shape or
    # device for the one-call form over both streams, before the library is
    # called (CPU tensors here: no device is touched)
    torch = pytest.importorskip("torch")
    p = _plan([(3, 3, 2), (0, 0, 5), (4, 2, 0)], 2, 64, "bf16")
    B, C = 3, 64
    rows = p.n_text + p.n_image
    x = torch.zeros(rows, C, dtype=torch.bfloat16)
    v2 = torch.zeros(2 * B, C, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pvj.adaln_modulate(p, "bogus", x, v2, v2)
    with pytest.raises(ValueError):   # per-sample vectors must be [2B, C] for both streams
        pvj.adaln_modulate(p, "both", x, v2[:B], v2[:B])
    with pytest.raises(ValueError):   # rows must be n_text + n_image
        pvj.gate_residual(p, "both", x[:-1], x[:-1], v2)
    with pytest.raises(ValueError):   # CPU tensors are refused
        pvj.gate_residual(p, "both", x, x, v2)
    assert pvj.chain_workspace_bytes(p, pvj.CHAIN_GATE, "both", C) > 0
    with pytest.raises(ValueError):
        pvj.chain_workspace_bytes(p, pvj.CHAIN_GATE, "neither", C)
