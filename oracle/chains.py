"""CPU oracle for the memory-bound chains around the joint attention.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle``): only the tests,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it; it imports nothing from the product path.

Mage-Flow review page, section "Kernel fusion": the diffusion-backbone blocks
carry chains of memory-bound operations around their main operators
(normalization, adaptive modulation, RoPE application, gating, activation and
residual addition), and fusing each chain so that only its final output is
written back is where most of the measured speed-up comes from.  Same page,
section "Native-Resolution MMDiT": the backbone follows the MMDiT block design
with modality-specific normalization and projection, i.e. the text and image
streams keep separate parameters.

The pages name the operations but not their formulas.  Plainest reading, the
one the MMDiT block design they cite uses (adaptive layer norm with gated
residuals), taken here:

* normalization: LayerNorm over the hidden dimension without affine
  parameters, population variance, ``eps`` = 1e-6;
* adaptive modulation before the QKV projection:
  ``y = LN(x) * (1 + scale_i) + shift_i`` where ``shift_i, scale_i`` are the
  per-sample, per-stream modulation vectors (computed from the sample's
  conditioning outside this chain);
* gate + residual after the output projection: ``out = x + gate_i * y``;
* a token's sample ``i`` is the sample whose slice of its stream (text or image,
  packed in sample order without padding) holds the token.

Everything is fp64 NumPy, one token row at a time where it matters.  The
backward functions are the derivatives of the definitions above, written out;
the ``-m "not gpu"`` tests pin them against finite differences and autograd.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

from . import _frames

LN_EPS = 1e-6
TEXT, IMAGE = 0, 1


def stream_sample_index(samples: Sequence, stream: int) -> np.ndarray:
    """Sample index of every row of a stream (text: t_i rows of sample i, in
    order; image: h_i * w_i * F_i rows of sample i, in order)."""
    idx = []
    for i, s in enumerate(samples):
        n = int(s[2]) if stream == TEXT else int(s[0]) * int(s[1]) * _frames(s)
        idx += [i] * n
    return np.array(idx, dtype=np.int64)


def layer_norm_rows(x: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """(x - mean) / sqrt(var + eps) over the last axis (population variance)."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def adaln_modulate(x, shift, scale, samples, stream, eps: float = LN_EPS) -> np.ndarray:
    """y[t] = LN(x[t]) * (1 + scale[i(t)]) + shift[i(t)] for the rows of one stream.

    x: [N, C]; shift, scale: [B, C]."""
    x = np.asarray(x, np.float64)
    shift = np.asarray(shift, np.float64)
    scale = np.asarray(scale, np.float64)
    si = stream_sample_index(samples, stream)
    assert si.shape[0] == x.shape[0]
    return layer_norm_rows(x, eps) * (1.0 + scale[si]) + shift[si]


def adaln_modulate_bwd(x, scale, dy, samples, stream, eps: float = LN_EPS):
    """Gradients of sum(y * dy) for ``adaln_modulate``: (dx, dshift, dscale).

    With xhat = (x - mu) r, r = (var + eps)^(-1/2) and g = dy (1 + scale_i):
      dshift_i = sum over the sample's rows of dy;
      dscale_i = sum over the sample's rows of dy * xhat;
      dx = r (g - mean(g) - xhat mean(g xhat))   (means over the hidden axis).
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    scale = np.asarray(scale, np.float64)
    si = stream_sample_index(samples, stream)
    B = scale.shape[0]
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(var + eps)
    xhat = (x - mu) * r
    g = dy * (1.0 + scale[si])
    dx = r * (g - g.mean(axis=-1, keepdims=True) - xhat * (g * xhat).mean(axis=-1, keepdims=True))
    dshift = np.zeros((B, x.shape[1]))
    dscale = np.zeros((B, x.shape[1]))
    for t in range(x.shape[0]):
        dshift[si[t]] += dy[t]
        dscale[si[t]] += dy[t] * xhat[t]
    return dx, dshift, dscale


def gate_residual(x, y, gate, samples, stream) -> np.ndarray:
    """out[t] = x[t] + gate[i(t)] * y[t]."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    gate = np.asarray(gate, np.float64)
    si = stream_sample_index(samples, stream)
    return x + gate[si] * y


def gate_residual_bwd(y, gate, dout, samples, stream):
    """Gradients of sum(out * dout): (dx, dy, dgate) with dx = dout,
    dy = gate_i * dout and dgate_i = sum over the sample's rows of dout * y."""
    y = np.asarray(y, np.float64)
    dout = np.asarray(dout, np.float64)
    gate = np.asarray(gate, np.float64)
    si = stream_sample_index(samples, stream)
    dgate = np.zeros_like(gate)
    for t in range(y.shape[0]):
        dgate[si[t]] += dout[t] * y[t]
    return dout.copy(), gate[si] * dout, dgate
