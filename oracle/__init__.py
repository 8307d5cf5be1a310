"""CPU oracle for packed variable-length joint attention with per-sample 2D RoPE.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (the HIP library and its binding) never calls it, and this package never
imports the product path: the two share no code.

Everything here is plain fp64 NumPy, one sample and one head at a time, written
from the definitions on the Mage-Flow pages:

* Mage-Flow review page (startedourmission.github.io), section
  "Native-Resolution MMDiT": text and image tokens are concatenated and go
  through joint self-attention; variable-resolution latent sequences and the
  text conditions are packed into one contiguous batch without padding, and
  per-sample cumulative offsets confine attention to each sample, so no
  block-diagonal mask is built; the CFG branches share one pack.
* same page, section "Mage-VAE": 16x downsampling with the 2x patchify absorbed,
  so one latent token covers 16x16 pixels.
* Hugging Face paper page (huggingface.co/papers/2607.19064), "Highlights", and
  the model-card mirror "microsoft/Mage-Flow", section "Architecture": per-sample
  2D rotary embeddings on the packed variable-length image+text sequence.

The pages do not fix these conventions; the oracle takes the plainest reading:

* token order inside a sample: text first, then image; image tokens flattened
  row-major, positions 0-based;
* text tokens sit at position (0, 0), i.e. they are not rotated;
* 2D RoPE: the first half of the head dimension is rotated by the latent row,
  the second half by the latent column; each half is a standard 1D rotary
  embedding of dimension D/2 with adjacent (interleaved) pairs
  (2k, 2k+1) and frequency theta**(-k / (D/4)), theta = 10000;
  Q and K are rotated, V is not; every head uses the same angles;
* editing mode (review page, "Native-Resolution MMDiT": the edit model adds a
  frame axis to the 2D RoPE, so every visual token has an (h, w, f) index): a
  sample (h, w, t, F) holds t text tokens then F image grids of h x w, frame
  after frame, each row-major; text sits at (0, 0, 0); image token p is at
  (row, col, frame) = ((p mod hw) // w, p mod w, p // hw).  The head dim is
  split into consecutive row | col | frame parts of (D-16)/2, (D-16)/2 and 16
  dims, each a 1D rotary embedding of its own dimension d_a with frequency
  theta**(-k / (d_a/2)) (the plain 2D mode is the special case of two D/2
  parts);
* attention is non-causal, softmax scale 1/sqrt(D), no bias, no dropout;
* LSE is the natural-log log-sum-exp of the scaled logits, fp32 ``[H, T]``.

Parity status: the exact pairing and frequency layout of the 2D RoPE, and the
head-dim split and frame layout of the 3-axis RoPE, are not fixed by the
pages, so those layouts are "parity unpinned" beyond their stated convention;
every other function is pinned by the ``-m "not gpu"`` tests.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

Sample = Tuple[int, int, int]  # (h_lat, w_lat, l_text)

ROPE_THETA = 10000.0


# ----------------------------------------------------------------------------
# packing: lengths, offsets, positions
# ----------------------------------------------------------------------------

def _frames(s) -> int:
    return int(s[3]) if len(s) > 3 else 1


def sample_lengths(samples: Sequence[Sample]) -> np.ndarray:
    """Tokens per sample: text tokens plus one image token per latent cell.

    Review page, "Native-Resolution MMDiT": each image becomes a variable-length
    latent token sequence and its text condition is kept at its own length (no
    padding).  Review page, "Mage-VAE": one latent cell per 16x16 pixels.  An
    editing sample (h, w, t, F) carries F grids (source and target frames).
    """
    return np.array([int(s[2]) + int(s[0]) * int(s[1]) * _frames(s) for s in samples],
                    dtype=np.int64)


def cu_seqlens(samples: Sequence[Sample]) -> np.ndarray:
    """Per-sample cumulative offsets: cu[0] = 0, cu[i+1] = cu[i] + L_i.

    Review page, "Native-Resolution MMDiT": the packed batch is one contiguous
    token axis and attention is confined by per-sample cumulative offsets.
    Samples stay in input order.
    """
    lens = sample_lengths(samples)
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    for i, n in enumerate(lens):
        cu[i + 1] = cu[i] + n
    return cu


def token_positions(samples: Sequence[Sample]) -> np.ndarray:
    """(row, col) RoPE position of every packed token, shape [T, 2], int64.

    Per-sample 2D positions (HF paper page, "Highlights": per-sample 2D RoPE):
    each sample restarts at its own origin.  Text tokens come first and sit at
    (0, 0); image token p (0-based, row-major) of a w-wide grid is at
    (p // w, p % w).
    """
    rows: List[Tuple[int, int]] = []
    for s in samples:
        h, w, t = s[0], s[1], s[2]
        for _ in range(t):
            rows.append((0, 0))
        for _f in range(_frames(s)):
            for r in range(h):
                for c in range(w):
                    rows.append((r, c))
    return np.array(rows, dtype=np.int64).reshape(-1, 2)


def token_positions3(samples: Sequence[Sample]) -> np.ndarray:
    """(row, col, frame) RoPE position of every packed token, shape [T, 3].

    Review page, "Native-Resolution MMDiT" (editing): a frame axis is added to
    the 2D RoPE.  Text tokens are at (0, 0, 0); image grids follow frame after
    frame, each row-major.
    """
    rows: List[Tuple[int, int, int]] = []
    for s in samples:
        h, w, t = s[0], s[1], s[2]
        for _ in range(t):
            rows.append((0, 0, 0))
        for f in range(_frames(s)):
            for r in range(h):
                for c in range(w):
                    rows.append((r, c, f))
    return np.array(rows, dtype=np.int64).reshape(-1, 3)


def rope_axis_dims(head_dim: int, axes: int):
    """Head-dim parts of the rotary axes: (D/2, D/2) for (row, col); for
    (row, col, frame): ((D-16)/2, (D-16)/2, 16)."""
    if axes == 2:
        return (head_dim // 2, head_dim // 2)
    return ((head_dim - 16) // 2, (head_dim - 16) // 2, 16)


# ----------------------------------------------------------------------------
# 2D RoPE
# ----------------------------------------------------------------------------

def rope_frequencies(head_dim: int, theta: float = ROPE_THETA) -> np.ndarray:
    """omega_k = theta ** (-k / (D/4)), k = 0 .. D/4 - 1 (one 1D RoPE of dim D/2 per axis)."""
    npair = head_dim // 4
    return np.array([theta ** (-k / npair) for k in range(npair)], dtype=np.float64)


def rope_nd_at(x: np.ndarray, pos: np.ndarray, dims, theta: float = ROPE_THETA,
               inverse: bool = False) -> np.ndarray:
    """Rotate ``x`` [N, H, D] by the positions ``pos`` [N, A] on A axes.

    Axis a owns the consecutive head dims of part a (sizes ``dims``, summing to
    D) and is a 1D rotary embedding of dimension d_a: pair k (dims
    base + 2k, base + 2k + 1) turns by pos_a * theta**(-k / (d_a/2)).
    """
    x = np.asarray(x, dtype=np.float64)
    n, nh, d = x.shape
    assert sum(dims) == d and pos.shape[1] == len(dims)
    out = x.copy()
    sign = -1.0 if inverse else 1.0
    base = 0
    for axis, da in enumerate(dims):
        p = pos[:, axis].astype(np.float64)
        for k in range(da // 2):
            omega = theta ** (-k / (da // 2))
            phi = sign * p * omega
            c = np.cos(phi)[:, None]
            s = np.sin(phi)[:, None]
            a = x[:, :, base + 2 * k]
            b = x[:, :, base + 2 * k + 1]
            out[:, :, base + 2 * k] = a * c - b * s
            out[:, :, base + 2 * k + 1] = a * s + b * c
        base += da
    return out


def rope3d(x: np.ndarray, samples: Sequence[Sample], theta: float = ROPE_THETA,
           inverse: bool = False) -> np.ndarray:
    """Per-sample 3-axis (row, col, frame) RoPE of a packed tensor [T, H, D]."""
    d = x.shape[2]
    return rope_nd_at(x, token_positions3(samples), rope_axis_dims(d, 3), theta, inverse)


def rope_apply(x, samples, theta: float = ROPE_THETA, inverse: bool = False, axes: int = 2):
    """The RoPE of the given mode: 2 axes (row, col) or 3 axes (row, col, frame)."""
    return rope3d(x, samples, theta, inverse) if axes == 3 else rope2d(x, samples, theta, inverse)


def rope2d_at(x: np.ndarray, pos: np.ndarray, theta: float = ROPE_THETA,
              inverse: bool = False) -> np.ndarray:
    """Rotate ``x`` [N, H, D] by the 2D positions ``pos`` [N, 2] (row, col).

    Dims [0, D/2) belong to the row axis and [D/2, D) to the column axis.  Pair
    k of an axis is dims (base + 2k, base + 2k + 1), rotated by the angle
    phi = p_axis * omega_k:  (a, b) -> (a cos phi - b sin phi, a sin phi + b cos phi).
    ``inverse`` rotates by -phi (the transpose of the rotation).
    """
    x = np.asarray(x, dtype=np.float64)
    n, nh, d = x.shape
    assert d % 4 == 0
    half = d // 2
    omega = rope_frequencies(d, theta)
    out = x.copy()
    sign = -1.0 if inverse else 1.0
    for axis in range(2):
        base = axis * half
        p = pos[:, axis].astype(np.float64)
        for k in range(d // 4):
            phi = sign * p * omega[k]                    # [N]
            c = np.cos(phi)[:, None]
            s = np.sin(phi)[:, None]
            a = x[:, :, base + 2 * k]
            b = x[:, :, base + 2 * k + 1]
            out[:, :, base + 2 * k] = a * c - b * s
            out[:, :, base + 2 * k + 1] = a * s + b * c
    return out


def rope2d(x: np.ndarray, samples: Sequence[Sample], theta: float = ROPE_THETA,
           inverse: bool = False) -> np.ndarray:
    """Per-sample 2D RoPE of a packed tensor [T, H, D] (see ``rope2d_at``)."""
    return rope2d_at(x, token_positions(samples), theta, inverse)


# ----------------------------------------------------------------------------
# attention, one sample and one head at a time
# ----------------------------------------------------------------------------

def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)


def _attn_one(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """softmax(scale * q k^T) v for one sample and head; also the natural-log LSE."""
    s = scale * (q @ k.T)                                 # [L, L]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    p = e / z
    o = p @ v
    lse = (m + np.log(z))[:, 0]
    return o, lse, p


def attn_fwd(q, k, v, samples: Sequence[Sample], scale: float = None, rope: bool = False,
             theta: float = ROPE_THETA, axes: int = 2):
    """Packed varlen joint attention forward.

    Review page, "Native-Resolution MMDiT": joint self-attention over each
    sample's concatenated text and image tokens, confined to the sample by its
    cumulative offsets.  With ``rope`` the per-sample 2D RoPE is applied to Q
    and K first (``axes`` = 3: the row, col, frame RoPE of editing samples).
    Returns O [T, H, D] and LSE [H, T] (fp64).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, H, D = q.shape
    if scale is None:
        scale = default_scale(D)
    if rope:
        q = rope_apply(q, samples, theta, axes=axes)
        k = rope_apply(k, samples, theta, axes=axes)
    cu = cu_seqlens(samples)
    o = np.zeros((T, H, D))
    lse = np.zeros((H, T))
    for i in range(len(samples)):
        a, b = int(cu[i]), int(cu[i + 1])
        if a == b:
            continue
        for h in range(H):
            oi, li, _ = _attn_one(q[a:b, h], k[a:b, h], v[a:b, h], scale)
            o[a:b, h] = oi
            lse[h, a:b] = li
    return o, lse


def attn_fwd_rows(q, k, v, samples: Sequence[Sample], sample: int, head: int, rows,
                  scale: float = None, rope: bool = False, theta: float = ROPE_THETA,
                  axes: int = 2):
    """Selected output rows of ``attn_fwd`` for one (sample, head).

    ``rows`` are local query indices inside the sample.  Each output row of the
    attention depends only on its own query and the sample's keys and values,
    so this evaluates the same definition at chosen outputs (used to check very
    large packs without computing every row).  Returns O [len(rows), D] and LSE.
    """
    cu = cu_seqlens(samples)
    a, b = int(cu[sample]), int(cu[sample + 1])
    D = q.shape[2]
    if scale is None:
        scale = default_scale(D)
    qi = np.asarray(q[a:b, head:head + 1], np.float64)
    ki = np.asarray(k[a:b, head:head + 1], np.float64)
    vi = np.asarray(v[a:b, head], np.float64)
    if rope:
        qi = rope_apply(qi, [samples[sample]], theta, axes=axes)
        ki = rope_apply(ki, [samples[sample]], theta, axes=axes)
    rows = np.asarray(rows, dtype=np.int64)
    o, lse, _ = _attn_one(qi[rows, 0], ki[:, 0], vi, scale)
    return o, lse


def attn_bwd(q, k, v, do, samples: Sequence[Sample], scale: float = None, rope: bool = False,
             theta: float = ROPE_THETA, axes: int = 2):
    """Gradients of L = sum(O * dO) with respect to Q, K, V.

    Per sample and head, with P the softmax probabilities:
      dV = P^T dO;  dP = dO V^T;  Delta = rowsum(dO * O);  dS = P * (dP - Delta);
      dQ' = scale * dS K';  dK' = scale * dS^T Q'.
    With ``rope``, Q' = R Q and K' = R K, so dQ = R^T dQ' and dK = R^T dK'
    (the inverse rotation), since R is orthogonal.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    T, H, D = q.shape
    if scale is None:
        scale = default_scale(D)
    if rope:
        q = rope_apply(q, samples, theta, axes=axes)
        k = rope_apply(k, samples, theta, axes=axes)
    cu = cu_seqlens(samples)
    dq = np.zeros((T, H, D))
    dk = np.zeros((T, H, D))
    dv = np.zeros((T, H, D))
    for i in range(len(samples)):
        a, b = int(cu[i]), int(cu[i + 1])
        if a == b:
            continue
        for h in range(H):
            qi, ki, vi, doi = q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h]
            oi, _, p = _attn_one(qi, ki, vi, scale)
            dv[a:b, h] = p.T @ doi
            dp = doi @ vi.T
            delta = (doi * oi).sum(axis=1, keepdims=True)
            ds = p * (dp - delta)
            dq[a:b, h] = scale * (ds @ ki)
            dk[a:b, h] = scale * (ds.T @ qi)
    if rope:
        dq = rope_apply(dq, samples, theta, inverse=True, axes=axes)
        dk = rope_apply(dk, samples, theta, inverse=True, axes=axes)
    return dq, dk, dv


def attn_bwd_delta(o, do) -> np.ndarray:
    """Delta[h, t] = sum_d dO[t, h, d] * O[t, h, d], the softmax-backward row term."""
    o = np.asarray(o, np.float64)
    do = np.asarray(do, np.float64)
    return (o * do).sum(axis=2).T.copy()


def dense_masked_attn_fwd(q, k, v, samples: Sequence[Sample], scale: float = None):
    """Brute-force twin of ``attn_fwd`` (no RoPE): dense T x T logits over the
    whole pack with an explicit block-diagonal mask (-inf off the diagonal
    blocks), row softmax over all T columns.  This is the mask the pages say the
    offsets make unnecessary (review page, "Native-Resolution MMDiT").
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, H, D = q.shape
    if scale is None:
        scale = default_scale(D)
    owner = np.empty(T, dtype=np.int64)
    j = 0
    for i, n in enumerate(sample_lengths(samples)):
        owner[j:j + n] = i
        j += n
    mask = owner[:, None] == owner[None, :]
    o = np.zeros((T, H, D))
    lse = np.zeros((H, T))
    for h in range(H):
        s = scale * (q[:, h] @ k[:, h].T)
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.where(mask, np.exp(s - m), 0.0)
        z = e.sum(axis=1, keepdims=True)
        o[:, h] = (e / z) @ v[:, h]
        lse[h] = (m + np.log(z))[:, 0]
    return o, lse


# ----------------------------------------------------------------------------
# the two modality streams
# ----------------------------------------------------------------------------

def pack_joint(text: np.ndarray, image: np.ndarray, samples: Sequence[Sample]) -> np.ndarray:
    """Joint per-sample [text_i; image_i] rows from the two modality streams.

    Review page, "Native-Resolution MMDiT": modality-specific layers keep text
    and image in separate streams, and their tokens are concatenated for the
    joint attention.  ``text`` is [sum t_i, H, D], ``image`` [sum h_i w_i, H, D],
    each stream packed in sample order without padding.
    """
    parts = []
    ta = ia = 0
    for smp in samples:
        t, n = smp[2], smp[0] * smp[1] * _frames(smp)
        parts.append(text[ta:ta + t])
        parts.append(image[ia:ia + n])
        ta += t
        ia += n
    assert ta == text.shape[0] and ia == image.shape[0]
    return np.concatenate(parts, axis=0) if parts else text[:0].copy()


def unpack_joint(joint: np.ndarray, samples: Sequence[Sample]):
    """Inverse of ``pack_joint``: split joint rows back into the two streams."""
    texts, images = [], []
    j = 0
    for smp in samples:
        t, n = smp[2], smp[0] * smp[1] * _frames(smp)
        texts.append(joint[j:j + t])
        images.append(joint[j + t:j + t + n])
        j += t + n
    assert j == joint.shape[0]
    if not samples:
        return joint[:0].copy(), joint[:0].copy()
    return np.concatenate(texts, axis=0), np.concatenate(images, axis=0)
