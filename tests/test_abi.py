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


def _check_work_list(p, samples, which):
    items, tile = p.work_items(which)
    lens = oracle.sample_lengths(samples)
    assert len(items) % 8 == 0
    seen = {}
    group_xcd = {}
    for b, (s, h, t, pad) in enumerate(items):
        if s < 0:
            continue
        assert 0 <= s < len(samples) and 0 <= h < p.n_heads and pad == 0
        assert 0 <= t * tile < lens[s]
        key = (s, h, t)
        assert key not in seen, key
        seen[key] = b
        # every tile of a (sample, head) lands on the same XCD (slot % 8)
        assert group_xcd.setdefault((s, h), b % 8) == b % 8
    want = {(s, h, t) for s in range(len(samples)) for h in range(p.n_heads)
            for t in range(int(math.ceil(lens[s] / tile)))}
    assert set(seen) == want
    # inside each XCD, longer samples run first (LPT)
    for x in range(8):
        ls = [lens[s] for (s, h, t, _) in items[x::8] if s >= 0]
        assert all(a >= b for a, b in zip(ls, ls[1:]))
        # idle slots only at the end of an XCD's list
        flags = [s >= 0 for (s, _, _, _) in items[x::8]]
        assert flags == sorted(flags, reverse=True)


@pytest.mark.parametrize("name", WORKLOADS)
def test_work_lists_cover_every_tile_once(lib, name):
    wl = workload(name)
    p = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    _check_work_list(p, wl.samples, 0)
    _check_work_list(p, wl.samples, 1)


def test_work_lists_random_packs(lib):
    rng = np.random.default_rng(0)
    for _ in range(20):
        samples = random_small_pack(rng, int(rng.integers(0, 12)), max_side=40, max_text=300)
        p = _plan(samples, int(rng.integers(1, 5)), 128, "bf16")
        _check_work_list(p, samples, 0)
        _check_work_list(p, samples, 1)


def test_work_list_xcd_balance(lib):
    # the (sample, head) groups are dealt so no XCD carries much more than its share
    wl = workload("train_64k", 3)
    p = _plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype)
    items, tile = p.work_items(0)
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
