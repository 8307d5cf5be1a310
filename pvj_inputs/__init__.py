"""Seeded synthetic inputs for packed variable-length joint text+image attention.

This module is the only code shared by the oracle side (``oracle/``, the tests)
and the HIP side (the binding, ``bench.py``).  It draws sample shapes and
random tensors; it holds none of the method's arithmetic (no offsets, no
positions, no rotation, no attention).

Workloads (sizes follow the Mage-Flow pages; the draws are synthetic stand-ins
for the native-resolution training data the pages train on, which is not
available here):

* ``tiny_f32``     two samples, 16x16 grid + 32 text and 8x32 grid + 16 text,
                   2 heads, head_dim 64, fp32, forward only.
* ``single_1024``  one 1024x1024 image: 64x64 latent grid (one token per 16x16
                   pixels, Mage-Flow review page, section "Mage-VAE") plus 256
                   text tokens, 24 heads, head_dim 128, bf16, forward only.
* ``cfg_1024``     the classifier-free-guidance pack (review page, section
                   "Native-Resolution MMDiT": conditional and unconditional
                   branches in one forward): cond 64x64 + 256 text, uncond
                   64x64 + 16 text, the uncond image rows identical to the cond
                   image rows; forward only.
* ``train_64k``    native-resolution training pack under a 65,536-token budget
                   (review page, section "Native-Resolution MMDiT": packing under
                   a fixed token budget; heights and widths 512..2048): pixel H,
                   W drawn from {512, 576, ..., 2048}, text length from
                   [32, 512]; samples are appended until the next one would
                   exceed the budget; forward + backward.
* ``extreme``      2048x2048, 2048x512, 512x2048 and four 512x512 samples, each
                   with text length drawn from [16, 512]; forward + backward.
* ``infer_multi``  a multi-prompt inference pack (review page, section
                   "Native-Resolution MMDiT": the classifier-free-guidance
                   branches of a sample share one pack; HF model card, "Python
                   API": a list of per-sample heights and widths in one call):
                   6 prompts, pixel sides drawn from {512, 576, ..., 2048},
                   text length from [32, 512]; each prompt contributes a
                   conditional sample and an unconditional sample with 16
                   text tokens whose image rows are copies of the conditional
                   ones; forward only.
* ``edit_1024``    an editing pack (review page, section "Native-Resolution
                   MMDiT": the edit model joins source and target latents under
                   a frame axis): a 1024x1024 pair (two 64x64 frames) with 256
                   text tokens and a 768x1024 pair (two 48x64 frames) with 128
                   text tokens; 3-axis RoPE; forward + backward.

A sample is the triple ``(h_lat, w_lat, l_text)`` (latent rows, latent columns,
text tokens), or for an editing pack the quadruple ``(h_lat, w_lat, l_text,
n_frames)``.  Tensors are packed ``[T, H, D]`` with samples in input order.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

Sample = Tuple[int, ...]  # (h_lat, w_lat, l_text[, n_frames])

PIXELS_PER_TOKEN_SIDE = 16  # Mage-VAE: 16x spatial downsampling, patchify absorbed
TRAIN_TOKEN_BUDGET = 65536


@dataclass
class Workload:
    name: str
    samples: List[Sample]
    n_heads: int
    head_dim: int
    dtype: str  # "bf16" or "f32"
    backward: bool
    seed: int
    # (cond_index, uncond_index) pairs whose image rows must be identical
    shared_image: List[Tuple[int, int]] = field(default_factory=list)

    @property
    def n_tokens(self) -> int:
        # the total row count of the packed tensors (inputs are sized by it)
        return int(sum(_rows(s) for s in self.samples))

    @property
    def frames(self) -> bool:
        return any(len(s) == 4 for s in self.samples)


def _rows(s: Sample) -> int:
    """Rows a sample occupies in the packed tensors (for sizing inputs)."""
    return s[2] + s[0] * s[1] * (s[3] if len(s) == 4 else 1)


def draw_train_pack(seed: int, budget: int = TRAIN_TOKEN_BUDGET) -> List[Sample]:
    """Draw native-resolution samples until the next one would exceed ``budget``.

    Pixel sides come from {512, 576, ..., 2048} (25 values), so the aspect ratio
    is at most 4:1 by construction; the text length is uniform on [32, 512].
    The draw stops at the first sample that does not fit.
    """
    rng = np.random.default_rng(seed)
    out: List[Sample] = []
    used = 0
    while True:
        hp = 512 + 64 * int(rng.integers(0, 25))
        wp = 512 + 64 * int(rng.integers(0, 25))
        t = int(rng.integers(32, 513))
        h, w = hp // PIXELS_PER_TOKEN_SIDE, wp // PIXELS_PER_TOKEN_SIDE
        n = h * w + t
        if used + n > budget:
            break
        out.append((h, w, t))
        used += n
    return out


def draw_extreme_pack(seed: int) -> List[Sample]:
    """2048^2, 2048x512, 512x2048, 4 x 512^2; text lengths uniform on [16, 512]."""
    rng = np.random.default_rng(seed)
    grids = [(128, 128), (128, 32), (32, 128), (32, 32), (32, 32), (32, 32), (32, 32)]
    return [(h, w, int(rng.integers(16, 513))) for (h, w) in grids]


def draw_multi_prompt_pack(seed: int, n_prompts: int = 6):
    """(samples, shared_image) of a multi-prompt CFG pack: per prompt a
    conditional sample (h, w, t) then its unconditional twin (h, w, 16)."""
    rng = np.random.default_rng(seed)
    samples: List[Sample] = []
    shared = []
    for _ in range(n_prompts):
        hp = 512 + 64 * int(rng.integers(0, 25))
        wp = 512 + 64 * int(rng.integers(0, 25))
        t = int(rng.integers(32, 513))
        h, w = hp // PIXELS_PER_TOKEN_SIDE, wp // PIXELS_PER_TOKEN_SIDE
        shared.append((len(samples), len(samples) + 1))
        samples += [(h, w, t), (h, w, 16)]
    return samples, shared


def workload(name: str, seed: int = 0) -> Workload:
    if name == "tiny_f32":
        return Workload(name, [(16, 16, 32), (8, 32, 16)], 2, 64, "f32", False, seed)
    if name == "single_1024":
        return Workload(name, [(64, 64, 256)], 24, 128, "bf16", False, seed)
    if name == "cfg_1024":
        return Workload(name, [(64, 64, 256), (64, 64, 16)], 24, 128, "bf16", False, seed,
                        shared_image=[(0, 1)])
    if name == "train_64k":
        return Workload(name, draw_train_pack(seed), 24, 128, "bf16", True, 1000 + seed)
    if name == "extreme":
        return Workload(name, draw_extreme_pack(seed), 24, 128, "bf16", True, seed)
    if name == "infer_multi":
        smp, shared = draw_multi_prompt_pack(seed)
        return Workload(name, smp, 24, 128, "bf16", False, 3000 + seed, shared_image=shared)
    if name == "edit_1024":
        return Workload(name, [(64, 64, 256, 2), (48, 64, 128, 2)], 24, 128, "bf16", True,
                        2000 + seed)
    raise KeyError(name)


WORKLOADS = ["tiny_f32", "single_1024", "cfg_1024", "train_64k", "extreme", "edit_1024",
             "infer_multi"]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even); returned as fp32 values."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(
        torch.float32).numpy()


def draw_tensors(n_tokens: int, n_heads: int, head_dim: int, dtype: str, seed: int,
                 n: int = 4, samples: Optional[List[Sample]] = None,
                 shared_image: Optional[List[Tuple[int, int]]] = None) -> List[np.ndarray]:
    """Draw ``n`` tensors [T, H, D] ~ N(0, 1) in the order Q, K, V, dO.

    For bf16 workloads the values are rounded to bf16; both sides consume
    exactly these values.  ``shared_image`` copies the image rows of one
    sample over those of another (same grid), for every tensor.
    """
    rng = np.random.default_rng(seed)
    outs = []
    for _ in range(n):
        x = rng.standard_normal((n_tokens, n_heads, head_dim), dtype=np.float32)
        if shared_image:
            starts = np.concatenate([[0], np.cumsum([_rows(s) for s in samples])])
            for (src, dst) in shared_image:
                hs, ws, ts = samples[src][:3]
                hd, wd, td = samples[dst][:3]
                assert (hs, ws) == (hd, wd)
                a = int(starts[src]) + ts
                b = int(starts[dst]) + td
                x[b:b + hs * ws] = x[a:a + hs * ws]
        if dtype == "bf16":
            x = round_bf16(x)
        outs.append(x)
    return outs


def workload_tensors(wl: Workload, n: int = 4) -> List[np.ndarray]:
    return draw_tensors(wl.n_tokens, wl.n_heads, wl.head_dim, wl.dtype, wl.seed, n=n,
                        samples=wl.samples, shared_image=wl.shared_image)


def random_small_pack(rng: np.random.Generator, n_samples: int, max_side: int = 6,
                      max_text: int = 7, allow_empty: bool = True,
                      max_frames: int = 0) -> List[Sample]:
    """Tiny random packs for brute-force checks (may include empty/text-only/image-only).

    With ``max_frames`` > 0 every sample is a quadruple with n_frames drawn from
    [0 or 1, max_frames] (0 only when ``allow_empty``)."""
    out = []
    lo = 0 if allow_empty else 1
    for _ in range(n_samples):
        h = int(rng.integers(lo, max_side + 1))
        w = int(rng.integers(lo, max_side + 1)) if h > 0 else 0
        t = int(rng.integers(lo, max_text + 1))
        f = int(rng.integers(lo, max_frames + 1)) if max_frames > 0 else 1
        if not allow_empty and h * w * f + t == 0:
            t = 1
        out.append((h, w, t, f) if max_frames > 0 else (h, w, t))
    return out
