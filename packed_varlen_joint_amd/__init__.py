"""Python binding of libpvj: packed variable-length joint text+image attention
with per-sample 2D RoPE on MI355X (gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels of
``libpvj.so`` behind the C ABI declared in ``include/pvj.h``.  PyTorch supplies
device memory and the current HIP stream.  There is no fallback: if the
library is missing, importing the compute functions raises.

    plan = Plan(samples=[(64, 64, 256), (64, 64, 16)], n_heads=24, head_dim=128,
                dtype=torch.bfloat16)
    plan.upload()                       # metadata -> device (torch buffer)
    o, lse = varlen_attn_fwd(plan, q, k, v, rope_fused=True)
    dq, dk, dv = varlen_attn_bwd(plan, q, k, v, o, lse, do, rope_fused=True)

Tensors are contiguous ``[T, H, D]`` (packed tokens, heads, head dim); LSE is
fp32 ``[H, T]``.  A sample is ``(h_lat, w_lat, l_text)``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional, Sequence, Tuple

__all__ = ["Plan", "PvjError", "pack", "unpack", "rope2d_apply", "stream_major_rows",
           "varlen_attn_fwd",
           "varlen_attn_bwd", "varlen_attn_bwd_noalloc", "library_path", "load_library",
           "profile_enable", "profile_read"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# PVJ_LIBRARY may point at another build of the same library (same ABI)
_LIB_PATH = os.environ.get("PVJ_LIBRARY") or os.path.join(_HERE, "libpvj.so")

PVJ_BF16 = 0
PVJ_F32 = 1
PVJ_ROPE_INTERLEAVED = 0
PVJ_FLAG_ROPE_FUSED = 1
PVJ_FLAG_ROPE_PREROTATED = 2
# token tensors hold all text rows (sample order), then all image rows
PVJ_FLAG_STREAM_MAJOR = 4

KERNELS = {"pack": 0, "unpack": 1, "rope2d": 2, "attn_fwd": 3, "bwd_pre": 4, "attn_bwd": 5,
           "attn_bwd_dq": 6, "chain_fwd": 7, "chain_bwd": 8, "proj": 9}
STREAMS = {"text": 0, "image": 1}
# the chain ops also take both streams in one call: rows [n_text + n_image,
# hidden] (text rows first), per-sample vectors [2 * n_samples, hidden]
CHAIN_STREAMS = {"text": 0, "image": 1, "both": 2}
CHAIN_ADALN, CHAIN_GATE = 0, 1


class PvjError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__("%s (%d): %s" % (name, status, detail))
        self.status = status
        self.name = name


class _Sample(ctypes.Structure):
    _fields_ = [("h_lat", ctypes.c_int32), ("w_lat", ctypes.c_int32), ("l_text", ctypes.c_int32)]


class _SampleFrames(ctypes.Structure):
    _fields_ = [("h_lat", ctypes.c_int32), ("w_lat", ctypes.c_int32), ("l_text", ctypes.c_int32),
                ("n_frames", ctypes.c_int32)]


class _Desc(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rope_pairing", ctypes.c_int32), ("text_first", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libpvj.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libpvj.so not found at %s; build it with "
                          "`python -m packed_varlen_joint_amd._build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I32, I64, SZ, U32, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                               ctypes.c_uint32, ctypes.c_float)
    sigs = {
        "pvj_plan_create": (I32, [ctypes.POINTER(_Sample), I32, ctypes.POINTER(_Desc),
                                  ctypes.POINTER(P)]),
        "pvj_plan_create_frames": (I32, [ctypes.POINTER(_SampleFrames), I32,
                                         ctypes.POINTER(_Desc), ctypes.POINTER(P)]),
        "pvj_plan_rope_axes": (I32, [P, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "pvj_plan_info": (I32, [P, ctypes.POINTER(I64), ctypes.POINTER(I32),
                                ctypes.POINTER(ctypes.POINTER(I32)), ctypes.POINTER(SZ)]),
        "pvj_plan_streams": (I32, [P, ctypes.POINTER(I64), ctypes.POINTER(I64)]),
        "pvj_plan_stream_major_rows": (I32, [P, ctypes.POINTER(I32), I64]),
        "pvj_plan_upload": (I32, [P, P, SZ, P]),
        "pvj_plan_destroy": (None, [P]),
        "pvj_pack": (I32, [P, P, P, P, P]),
        "pvj_unpack": (I32, [P, P, P, P, P]),
        "pvj_pack_rope": (I32, [P, P, P, P, I32, P]),
        "pvj_unpack_rope": (I32, [P, P, P, P, I32, P]),
        "pvj_rope2d_apply": (I32, [P, P, P, I32, P]),
        "pvj_rope2d_apply_stream_major": (I32, [P, P, P, I32, P]),
        "pvj_varlen_attn_fwd": (I32, [P, P, P, P, P, P, F, U32, P]),
        "pvj_varlen_attn_bwd_workspace": (I32, [P, ctypes.POINTER(SZ)]),
        "pvj_varlen_attn_bwd": (I32, [P, P, P, P, P, P, P, P, P, P, P, SZ, F, U32, P]),
        "pvj_varlen_attn_bwd_noalloc": (I32, [P, P, P, P, P, P, P, P, P, P, F, U32, P]),
        "pvj_plan_work_items": (I32, [P, I32, ctypes.POINTER(ctypes.POINTER(I32)),
                                      ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "pvj_plan_rope_table": (I32, [P, ctypes.POINTER(ctypes.POINTER(ctypes.c_float)),
                                      ctypes.POINTER(ctypes.POINTER(ctypes.c_float)),
                                      ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "pvj_adaln_modulate": (I32, [P, I32, I32, P, P, P, P, F, P]),
        "pvj_gate_residual": (I32, [P, I32, I32, P, P, P, P, P]),
        "pvj_chain_bwd_workspace": (I32, [P, I32, I32, I32, ctypes.POINTER(SZ)]),
        "pvj_adaln_modulate_bwd": (I32, [P, I32, I32, P, P, P, P, P, P, F, P, SZ, P]),
        "pvj_gate_residual_bwd": (I32, [P, I32, I32, P, P, P, P, P, P, SZ, P]),
        "pvj_qkv_proj_pack": (I32, [P, I32, I32, P, P, P, P, P, P, U32, P]),
        "pvj_out_proj_unpack": (I32, [P, I32, I32, P, P, P, P, P]),
        "pvj_diag_mfma_peak": (I32, [I32, I32, P, SZ, ctypes.POINTER(ctypes.c_double), P]),
        "pvj_profile_enable": (I32, [I32]),
        "pvj_profile_read": (I32, [I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64)]),
        "pvj_status_string": (ctypes.c_char_p, [I32]),
        "pvj_last_error": (ctypes.c_char_p, []),
        "pvj_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise PvjError(status, lib.pvj_status_string(status).decode(),
                       lib.pvj_last_error().decode())


def _torch():
    import torch
    return torch


def _dtype_code(dtype) -> int:
    torch = _torch()
    if dtype in (torch.bfloat16, "bf16"):
        return PVJ_BF16
    if dtype in (torch.float32, "f32"):
        return PVJ_F32
    raise ValueError("dtype must be bfloat16 or float32, got %r" % (dtype,))


class Plan:
    """Per-pack plan: offsets, RoPE tables and work lists (built on the host by
    ``pvj_plan_create``), plus the device copy of that metadata.

    ``samples`` holds (h_lat, w_lat, l_text) triples, or, for an editing pack
    with a frame axis, (h_lat, w_lat, l_text, n_frames) quadruples, which make
    the plan's RoPE 3-axis (``pvj_plan_create_frames``).  ``frames=True``
    forces the 3-axis plan for triples too (one frame each)."""

    def __init__(self, samples: Sequence[Tuple[int, ...]], n_heads: int, head_dim: int,
                 dtype="bf16", rope_theta: float = 10000.0, frames: bool = None):
        lib = load_library()
        raw = [tuple(int(x) for x in s) for s in samples]
        if any(len(s) not in (3, 4) for s in raw):
            raise ValueError("each sample is (h_lat, w_lat, l_text[, n_frames])")
        if frames is None:
            frames = any(len(s) == 4 for s in raw)
        if not frames and any(len(s) == 4 for s in raw):
            raise ValueError("samples with n_frames need a frames plan")
        self.frames = bool(frames)
        self.samples = [s if len(s) == 4 or not frames else s + (1,) for s in raw]
        desc = _Desc(int(n_heads), int(head_dim), _dtype_code(dtype), float(rope_theta),
                     PVJ_ROPE_INTERLEAVED, 1)
        h = ctypes.c_void_p()
        if frames:
            arr = (_SampleFrames * max(1, len(self.samples)))(
                *[_SampleFrames(*s) for s in self.samples])
            _check(lib.pvj_plan_create_frames(arr, len(self.samples), ctypes.byref(desc),
                                              ctypes.byref(h)))
        else:
            arr = (_Sample * max(1, len(self.samples)))(*[_Sample(*s) for s in self.samples])
            _check(lib.pvj_plan_create(arr, len(self.samples), ctypes.byref(desc),
                                       ctypes.byref(h)))
        self._h = h
        self.n_heads = int(n_heads)
        self.head_dim = int(head_dim)
        self.dtype_code = desc.dtype
        T = ctypes.c_int64()
        ml = ctypes.c_int32()
        cu = ctypes.POINTER(ctypes.c_int32)()
        mb = ctypes.c_size_t()
        _check(lib.pvj_plan_info(h, ctypes.byref(T), ctypes.byref(ml), ctypes.byref(cu),
                                 ctypes.byref(mb)))
        self.n_tokens = T.value
        self.max_len = ml.value
        self.cu_seqlens = [cu[i] for i in range(len(self.samples) + 1)]
        self.meta_bytes = mb.value
        nt = ctypes.c_int64()
        ni = ctypes.c_int64()
        _check(lib.pvj_plan_streams(h, ctypes.byref(nt), ctypes.byref(ni)))
        self.n_text = nt.value
        self.n_image = ni.value
        self._meta = None

    @property
    def handle(self):
        return self._h

    @property
    def torch_dtype(self):
        torch = _torch()
        return torch.bfloat16 if self.dtype_code == PVJ_BF16 else torch.float32

    def upload(self, device=None, stream=None) -> "Plan":
        """Copy the metadata into a torch-allocated device buffer on ``device``."""
        torch = _torch()
        device = torch.device(device) if device is not None else torch.device(
            "cuda", torch.cuda.current_device())
        with torch.cuda.device(device):
            buf = torch.empty(max(256, self.meta_bytes), dtype=torch.uint8, device=device)
            s = stream if stream is not None else torch.cuda.current_stream()
            _check(load_library().pvj_plan_upload(self._h, buf.data_ptr(), buf.numel(),
                                                  s.cuda_stream))
        self._meta = buf
        return self

    def work_items(self, which: int):
        """(items [n][4] list, tile_rows) of a work list: 0 forward (with split
        tiles), 1 backward dK/dV, 2 backward dQ, 3 the forward's split tiles."""
        lib = load_library()
        p = ctypes.POINTER(ctypes.c_int32)()
        n = ctypes.c_int32()
        tr = ctypes.c_int32()
        _check(lib.pvj_plan_work_items(self._h, which, ctypes.byref(p), ctypes.byref(n),
                                       ctypes.byref(tr)))
        return [tuple(p[4 * i + j] for j in range(4)) for i in range(n.value)], tr.value

    def rope_table(self):
        """(cos, sin, n_pos, n_pairs): flat [n_pos][n_pairs] fp32 tables."""
        lib = load_library()
        c = ctypes.POINTER(ctypes.c_float)()
        s = ctypes.POINTER(ctypes.c_float)()
        npos = ctypes.c_int32()
        npairs = ctypes.c_int32()
        _check(lib.pvj_plan_rope_table(self._h, ctypes.byref(c), ctypes.byref(s),
                                       ctypes.byref(npos), ctypes.byref(npairs)))
        n = npos.value * npairs.value
        return [c[i] for i in range(n)], [s[i] for i in range(n)], npos.value, npairs.value

    def rope_axes(self):
        """(n_axes, dims): 2 or 3 RoPE axes and the head-dim size of each."""
        n = ctypes.c_int32()
        dims = (ctypes.c_int32 * 3)()
        _check(load_library().pvj_plan_rope_axes(self._h, ctypes.byref(n), dims))
        return n.value, tuple(dims[i] for i in range(n.value))

    def bwd_workspace_bytes(self) -> int:
        b = ctypes.c_size_t()
        _check(load_library().pvj_varlen_attn_bwd_workspace(self._h, ctypes.byref(b)))
        return b.value

    def close(self):
        if getattr(self, "_h", None):
            load_library().pvj_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def profile_enable(on: bool = True):
    """Start (clearing earlier records) or stop per-kernel event timing in the library."""
    _check(load_library().pvj_profile_enable(1 if on else 0))


def profile_read(kernel: str):
    """(total milliseconds, launches) of one kernel kind since profile_enable(True)."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(load_library().pvj_profile_read(KERNELS[kernel], ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _check_tokens(plan: Plan, name: str, t, rows: Optional[int] = None):
    torch = _torch()
    rows = plan.n_tokens if rows is None else rows
    want = (rows, plan.n_heads, plan.head_dim)
    if tuple(t.shape) != want:
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), want))
    if t.dtype != plan.torch_dtype:
        raise ValueError("%s: dtype %s, expected %s" % (name, t.dtype, plan.torch_dtype))
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % name)


def _check_lse(plan: Plan, lse):
    torch = _torch()
    want = (plan.n_heads, plan.n_tokens)
    if tuple(lse.shape) != want:
        raise ValueError("lse: shape %s, expected %s" % (tuple(lse.shape), want))
    if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 device tensor")


def _empty_tokens(plan: Plan, like, rows=None):
    torch = _torch()
    rows = plan.n_tokens if rows is None else rows
    return torch.empty((rows, plan.n_heads, plan.head_dim), dtype=plan.torch_dtype,
                       device=like.device)


def pack(plan: Plan, text, image, joint=None, rope: bool = False, inverse: bool = False):
    """Joint [T,H,D] from the text [sum t,H,D] and image [sum h*w,H,D] streams
    (``rope``: rotated by the plan's RoPE in the same pass)."""
    _check_tokens(plan, "text", text, plan.n_text)
    _check_tokens(plan, "image", image, plan.n_image)
    joint = _empty_tokens(plan, text) if joint is None else joint
    _check_tokens(plan, "joint", joint)
    lib = load_library()
    if rope:
        _check(lib.pvj_pack_rope(plan.handle, _ptr(text), _ptr(image), _ptr(joint),
                                 int(bool(inverse)), _stream()))
    else:
        _check(lib.pvj_pack(plan.handle, _ptr(text), _ptr(image), _ptr(joint), _stream()))
    return joint


def unpack(plan: Plan, joint, text=None, image=None, rope: bool = False, inverse: bool = False):
    """Inverse of ``pack``: (text, image) streams from the joint tensor
    (``rope``: each row rotated by the plan's RoPE in the same pass)."""
    _check_tokens(plan, "joint", joint)
    text = _empty_tokens(plan, joint, plan.n_text) if text is None else text
    image = _empty_tokens(plan, joint, plan.n_image) if image is None else image
    _check_tokens(plan, "text", text, plan.n_text)
    _check_tokens(plan, "image", image, plan.n_image)
    lib = load_library()
    if rope:
        _check(lib.pvj_unpack_rope(plan.handle, _ptr(joint), _ptr(text), _ptr(image),
                                   int(bool(inverse)), _stream()))
    else:
        _check(lib.pvj_unpack(plan.handle, _ptr(joint), _ptr(text), _ptr(image), _stream()))
    return text, image


def rope2d_apply(plan: Plan, x, y=None, inverse: bool = False, stream_major: bool = False):
    """Per-sample 2D RoPE of x [T,H,D] into y (y is x: in place).

    ``stream_major``: x and y hold all text rows, then all image rows."""
    _check_tokens(plan, "x", x)
    y = _empty_tokens(plan, x) if y is None else y
    _check_tokens(plan, "y", y)
    lib = load_library()
    fn = lib.pvj_rope2d_apply_stream_major if stream_major else lib.pvj_rope2d_apply
    _check(fn(plan.handle, _ptr(x), _ptr(y), int(bool(inverse)), _stream()))
    return y


def stream_major_rows(plan: Plan):
    """Row of every token of the joint layout in the stream-major layout (from
    the plan): an int64 CPU tensor ``perm`` with ``sm[perm] == joint`` row for
    row (text rows of all samples first, then their image rows, each in sample
    order)."""
    torch = _torch()
    T = plan.n_tokens
    buf = (ctypes.c_int32 * max(1, T))()
    _check(load_library().pvj_plan_stream_major_rows(plan.handle, buf, T))
    return torch.frombuffer(buf, dtype=torch.int32)[:T].to(torch.int64)


def varlen_attn_fwd(plan: Plan, q, k, v, softmax_scale: float = 0.0, rope_fused: bool = False,
                    out=None, lse=None, want_lse: bool = True, stream_major: bool = False):
    """Packed varlen joint attention forward; returns (O [T,H,D], LSE fp32 [H,T] or None).

    ``stream_major``: every token tensor (and LSE's columns) in the stream-major
    row order (all text rows, then all image rows; bf16 plans, no ``rope_fused``)."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_tokens(plan, n, t)
    out = _empty_tokens(plan, q) if out is None else out
    _check_tokens(plan, "out", out)
    if lse is None and want_lse:
        lse = torch.empty((plan.n_heads, plan.n_tokens), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_lse(plan, lse)
    flags = (PVJ_FLAG_ROPE_FUSED if rope_fused else 0) | (
        PVJ_FLAG_STREAM_MAJOR if stream_major else 0)
    _check(load_library().pvj_varlen_attn_fwd(plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                              _ptr(lse), float(softmax_scale), flags, _stream()))
    return out, lse


def varlen_attn_bwd(plan: Plan, q, k, v, o, lse, dout, softmax_scale: float = 0.0,
                    rope_fused: bool = False, dq=None, dk=None, dv=None, workspace=None,
                    rope_prerotated: bool = False, stream_major: bool = False):
    """Packed varlen joint attention backward; returns (dQ, dK, dV).

    ``rope_prerotated``: q and k already hold R Q and R K (``pack(..., rope=True)``);
    dQ and dK still come back with respect to the un-rotated Q and K.
    ``stream_major``: as in ``varlen_attn_fwd``."""
    torch = _torch()
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tokens(plan, n, t)
    _check_lse(plan, lse)
    dq = _empty_tokens(plan, q) if dq is None else dq
    dk = _empty_tokens(plan, q) if dk is None else dk
    dv = _empty_tokens(plan, q) if dv is None else dv
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tokens(plan, n, t)
    nbytes = plan.bwd_workspace_bytes()
    if workspace is None:
        workspace = torch.empty(max(256, nbytes), dtype=torch.uint8, device=q.device)
    elif (workspace.dtype != torch.uint8 or not workspace.is_cuda
          or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous uint8 device tensor")
    flags = (PVJ_FLAG_ROPE_FUSED if rope_fused else 0) | (
        PVJ_FLAG_ROPE_PREROTATED if rope_prerotated else 0) | (
        PVJ_FLAG_STREAM_MAJOR if stream_major else 0)
    _check(load_library().pvj_varlen_attn_bwd(
        plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
        _ptr(dk), _ptr(dv), _ptr(workspace), workspace.numel(), float(softmax_scale), flags,
        _stream()))
    return dq, dk, dv


def varlen_attn_bwd_noalloc(plan: Plan, q, k, v, o, lse, dout, dq, dk, dv,
                            softmax_scale: float = 0.0, rope_prerotated: bool = False,
                            stream_major: bool = False):
    """``varlen_attn_bwd`` without any device allocation: the library keeps the
    backward's scratch (Delta) in a fixed static device buffer (16 MiB per GPU,
    so H * T <= 4,194,304) and the caller passes every tensor, outputs
    included.  RoPE on load is not offered; pass Q, K pre-rotated with
    ``rope_prerotated``.  Calls that overlap in time on one GPU race on the
    shared buffer."""
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq),
                 ("dk", dk), ("dv", dv)):
        _check_tokens(plan, n, t)
    _check_lse(plan, lse)
    flags = (PVJ_FLAG_ROPE_PREROTATED if rope_prerotated else 0) | (
        PVJ_FLAG_STREAM_MAJOR if stream_major else 0)
    _check(load_library().pvj_varlen_attn_bwd_noalloc(
        plan.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
        _ptr(dk), _ptr(dv), float(softmax_scale), flags, _stream()))
    return dq, dk, dv


# ---------------------------------------------------------------------------
# memory-bound chains around the attention (one modality stream, or both)
# ---------------------------------------------------------------------------

def _stream_rows(plan: Plan, which: str) -> int:
    if which not in STREAMS:
        raise ValueError("stream must be 'text' or 'image'")
    return plan.n_text if which == "text" else plan.n_image


def _chain_rows(plan: Plan, which: str):
    """(rows, per-sample vector rows) of a chain call on `which`."""
    if which not in CHAIN_STREAMS:
        raise ValueError("stream must be 'text', 'image' or 'both'")
    B = len(plan.samples)
    if which == "both":
        return plan.n_text + plan.n_image, 2 * B
    return _stream_rows(plan, which), B


def _check_2d(name, t, rows, cols, dtype):
    if t is None or t.dim() != 2 or tuple(t.shape) != (rows, cols):
        raise ValueError("%s must be [%d, %d]" % (name, rows, cols))
    if t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError("%s must be a contiguous %s CUDA tensor" % (name, dtype))


def chain_workspace_bytes(plan: Plan, op: int, which: str, hidden: int) -> int:
    b = ctypes.c_size_t()
    _chain_rows(plan, which)
    _check(load_library().pvj_chain_bwd_workspace(plan.handle, op, CHAIN_STREAMS[which],
                                                  int(hidden), ctypes.byref(b)))
    return b.value


def adaln_modulate(plan: Plan, which: str, x, shift, scale, y=None, eps: float = 1e-6):
    """y = LN(x) (1 + scale_i) + shift_i on one stream ([rows, hidden]), or on
    both (which="both": text rows then image rows, per-sample vectors
    [2 * n_samples, hidden], the text stream's first)."""
    (rows, nv), hidden = _chain_rows(plan, which), int(x.shape[-1])
    _check_2d("x", x, rows, hidden, plan.torch_dtype)
    _check_2d("shift", shift, nv, hidden, plan.torch_dtype)
    _check_2d("scale", scale, nv, hidden, plan.torch_dtype)
    y = _torch().empty_like(x) if y is None else y
    _check_2d("y", y, rows, hidden, plan.torch_dtype)
    _check(load_library().pvj_adaln_modulate(plan.handle, CHAIN_STREAMS[which], hidden, _ptr(x),
                                             _ptr(shift), _ptr(scale), _ptr(y), float(eps),
                                             _stream()))
    return y


def gate_residual(plan: Plan, which: str, x, y, gate, out=None):
    """out = x + gate_i * y on one stream, or on both (see adaln_modulate)."""
    (rows, nv), hidden = _chain_rows(plan, which), int(x.shape[-1])
    for n, t in (("x", x), ("y", y)):
        _check_2d(n, t, rows, hidden, plan.torch_dtype)
    _check_2d("gate", gate, nv, hidden, plan.torch_dtype)
    out = _torch().empty_like(x) if out is None else out
    _check_2d("out", out, rows, hidden, plan.torch_dtype)
    _check(load_library().pvj_gate_residual(plan.handle, CHAIN_STREAMS[which], hidden, _ptr(x),
                                            _ptr(y), _ptr(gate), _ptr(out), _stream()))
    return out


def _ws(plan, op, which, hidden, like, workspace):
    n = chain_workspace_bytes(plan, op, which, hidden)
    if workspace is None:
        workspace = _torch().empty(max(256, n), dtype=_torch().uint8, device=like.device)
    return workspace


def adaln_modulate_bwd(plan: Plan, which: str, x, scale, dy, eps: float = 1e-6, dx=None,
                       workspace=None):
    """(dx, dshift fp32, dscale fp32) for ``adaln_modulate``."""
    torch = _torch()
    (rows, nv), hidden = _chain_rows(plan, which), int(x.shape[-1])
    for n, t in (("x", x), ("dy", dy)):
        _check_2d(n, t, rows, hidden, plan.torch_dtype)
    _check_2d("scale", scale, nv, hidden, plan.torch_dtype)
    dx = torch.empty_like(x) if dx is None else dx
    _check_2d("dx", dx, rows, hidden, plan.torch_dtype)
    dshift = torch.empty(nv, hidden, dtype=torch.float32, device=x.device)
    dscale = torch.empty(nv, hidden, dtype=torch.float32, device=x.device)
    workspace = _ws(plan, CHAIN_ADALN, which, hidden, x, workspace)
    _check(load_library().pvj_adaln_modulate_bwd(
        plan.handle, CHAIN_STREAMS[which], hidden, _ptr(x), _ptr(scale), _ptr(dy), _ptr(dx),
        _ptr(dshift), _ptr(dscale), float(eps), _ptr(workspace), workspace.numel(), _stream()))
    return dx, dshift, dscale


def gate_residual_bwd(plan: Plan, which: str, y, gate, dout, dy=None, workspace=None):
    """(dy, dgate fp32) for ``gate_residual``; the gradient of x is dout itself."""
    torch = _torch()
    (rows, nv), hidden = _chain_rows(plan, which), int(y.shape[-1])
    for n, t in (("y", y), ("dout", dout)):
        _check_2d(n, t, rows, hidden, plan.torch_dtype)
    _check_2d("gate", gate, nv, hidden, plan.torch_dtype)
    dy = torch.empty_like(y) if dy is None else dy
    _check_2d("dy", dy, rows, hidden, plan.torch_dtype)
    dgate = torch.empty(nv, hidden, dtype=torch.float32, device=y.device)
    workspace = _ws(plan, CHAIN_GATE, which, hidden, y, workspace)
    _check(load_library().pvj_gate_residual_bwd(
        plan.handle, CHAIN_STREAMS[which], hidden, _ptr(y), _ptr(gate), _ptr(dout), _ptr(dy),
        _ptr(dgate), _ptr(workspace), workspace.numel(), _stream()))
    return dy, dgate


def diag_mfma_peak(rounds: int = 4, iters: int = 20000, reps: int = 3) -> float:
    """Sustained bf16 matrix-core TFLOP/s of the chip (best of `reps` timed runs
    of the library's matrix-core-only kernel, after one warm-up run)."""
    torch = _torch()
    sink = torch.empty(131072 * rounds, dtype=torch.float32, device="cuda")
    flop = ctypes.c_double()
    lib = load_library()
    best = 0.0
    for r in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _check(lib.pvj_diag_mfma_peak(rounds, iters, _ptr(sink), sink.numel(), ctypes.byref(flop),
                                      _stream()))
        e1.record()
        torch.cuda.synchronize()
        if r > 0:
            best = max(best, flop.value / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    return best


# ---------------------------------------------------------------------------
# projections with the pack / unpack fused in (bf16 plans)
# ---------------------------------------------------------------------------

def qkv_proj_pack(plan: Plan, which: str, x, w, bias=None, q=None, k=None, v=None,
                  rope: bool = True):
    """Joint Q, K, V rows of one stream from x [rows, hidden] @ w[3HD, hidden]^T + bias
    (RoPE on Q and K when ``rope``); pass the same q, k, v for both streams."""
    rows, hidden = _stream_rows(plan, which), int(x.shape[-1])
    hd = plan.n_heads * plan.head_dim
    _check_2d("x", x, rows, hidden, plan.torch_dtype)
    _check_2d("w", w, 3 * hd, hidden, plan.torch_dtype)
    if bias is not None and (bias.dim() != 1 or bias.numel() != 3 * hd):
        raise ValueError("bias must be [3 H D]")
    q = _empty_tokens(plan, x) if q is None else q
    k = _empty_tokens(plan, x) if k is None else k
    v = _empty_tokens(plan, x) if v is None else v
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check_tokens(plan, n, t)
    _check(load_library().pvj_qkv_proj_pack(
        plan.handle, STREAMS[which], hidden, _ptr(x), _ptr(w), _ptr(bias), _ptr(q), _ptr(k),
        _ptr(v), PVJ_FLAG_ROPE_FUSED if rope else 0, _stream()))
    return q, k, v


def out_proj_unpack(plan: Plan, which: str, o, w, bias=None, y=None):
    """y [rows, hidden] = (the stream's rows of the joint o) @ w[hidden, HD]^T + bias."""
    rows, hidden = _stream_rows(plan, which), int(w.shape[0])
    hd = plan.n_heads * plan.head_dim
    _check_tokens(plan, "o", o)
    _check_2d("w", w, hidden, hd, plan.torch_dtype)
    if bias is not None and (bias.dim() != 1 or bias.numel() != hidden):
        raise ValueError("bias must be [hidden]")
    y = _torch().empty(rows, hidden, dtype=plan.torch_dtype, device=o.device) if y is None else y
    _check_2d("y", y, rows, hidden, plan.torch_dtype)
    _check(load_library().pvj_out_proj_unpack(plan.handle, STREAMS[which], hidden, _ptr(o),
                                              _ptr(w), _ptr(bias), _ptr(y), _stream()))
    return y
