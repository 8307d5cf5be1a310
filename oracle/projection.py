"""CPU oracle for the projections around the joint attention with the pack and
unpack fused into them.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle``).

Mage-Flow review page, section "Native-Resolution MMDiT": the backbone keeps
modality-specific normalization and projection layers for the text and image
streams and concatenates their tokens for the joint attention.  So each stream
has its own QKV projection and output projection, and the joint layout exists
only between them.  The pages do not write the layer out; plainest reading,
taken here: a linear layer with bias per stream, ``y = x W^T + b``, with the
QKV output split as [Q | K | V] along the features and each part as [H, D]
(head-major), and the RoPE of the plan applied to Q and K after the
projection.

Every function is the composition of definitions already in the oracle (the
per-sample pack/unpack and RoPE) and a library matrix product, in fp64.
"""
from __future__ import annotations

import numpy as np

from . import pack_joint, rope_apply, unpack_joint


def linear(x, w, b=None):
    """x [N, K] @ w[N_out, K]^T (+ b[N_out])."""
    y = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    if b is not None:
        y = y + np.asarray(b, np.float64)[None, :]
    return y


def qkv_project_pack(x_text, x_img, w_text, b_text, w_img, b_img, samples, n_heads, head_dim,
                     rope=True, axes=2):
    """Joint Q, K, V [T, H, D] from the two streams' QKV projections; RoPE on Q, K."""
    hd = n_heads * head_dim
    yt = linear(x_text, w_text, b_text)
    yi = linear(x_img, w_img, b_img)
    out = []
    for part in range(3):
        t = yt[:, part * hd:(part + 1) * hd].reshape(-1, n_heads, head_dim)
        i = yi[:, part * hd:(part + 1) * hd].reshape(-1, n_heads, head_dim)
        j = pack_joint(t, i, samples)
        if rope and part < 2:
            j = rope_apply(j, samples, axes=axes)
        out.append(j)
    return out


def out_project_unpack(o_joint, w_text, b_text, w_img, b_img, samples):
    """(y_text, y_img): each stream's rows of the joint O, through its output projection."""
    o_joint = np.asarray(o_joint, np.float64)
    t, i = unpack_joint(o_joint, samples)
    return (linear(t.reshape(t.shape[0], -1), w_text, b_text),
            linear(i.reshape(i.shape[0], -1), w_img, b_img))
