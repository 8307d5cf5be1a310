#!/usr/bin/env python
"""Throughput of the packed variable-length joint-attention hot path on one MI355X.

One step = the whole path over one synthetic pack, with every input already
resident in HBM when the timed region starts:
  plan (host planner + metadata upload) -> pack Q and K with the 2D RoPE in
  the same pass, pack V -> attention forward -> unpack O -> pack dO ->
  attention backward (Delta preprocess, dK/dV kernel, dQ kernel; both rotate
  their gradient back with the inverse RoPE in the epilogue) -> unpack dQ,
  dK, dV.
`--rope load` instead packs Q and K plainly and rotates them on load inside
the attention kernels (forward) and in the backward preprocess.

Default workload: the native-resolution training pack (65,536-token budget,
seed 0: 7 samples, 55,151 tokens, 24 heads, head_dim 128, bf16), the pack on
which forward + backward is measured.  FLOPs are algorithmic, per sample
(never T^2): forward 4*H*D*sum(L_i^2), backward 10*H*D*sum(L_i^2) (five
products including the score recompute), so a step is 14*H*D*sum(L_i^2).

Prints one JSON line.  `--gpus N` with N > 1 is refused: this path is
measured on one GPU (the pack is one GPU's data-parallel share).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed varlen attn TFLOP/s (fwd, fwd+bwd) + % bf16 MFMA peak; tokens/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0


def _src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "packed_varlen_joint_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "attn_fwd": ("k_attn_fwd.hip", "pvj_device.h"),
    "attn_bwd": ("k_attn_bwd.hip", "pvj_device.h"),
    "attn_bwd_dq": ("k_attn_dq.hip", "pvj_device.h"),
}


def _traffic(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    try:
        rec = json.load(open(path)).get(kernel)
    except Exception:
        return None
    if not rec or rec.get("src_hash") != _src_hash(*KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


class PackStep:
    """One pass of the hot path over one pack.  `backward` overrides the
    workload's own (a training pack timed forward only); `reuse_plan` builds
    and uploads the plan once (an inference loop over denoising steps keeps
    the same per-sample resolutions), otherwise every step plans again."""

    def __init__(self, wl, seed, rope="pack", backward=None, reuse_plan=False):
        import torch
        import packed_varlen_joint_amd as pvj
        self.pvj = pvj
        self.wl = wl
        self.rope = rope
        self.backward = wl.backward if backward is None else backward
        self.reuse_plan = reuse_plan
        H, D = wl.n_heads, wl.head_dim
        dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        probe = pvj.Plan(wl.samples, H, D, wl.dtype)
        nt, ni = probe.n_text, probe.n_image
        T = wl.n_tokens
        g = torch.Generator(device="cuda").manual_seed(seed)
        mk = lambda n: torch.randn(n, H, D, device="cuda", generator=g).to(dt)
        # the two modality streams (text, image) of Q, K, V and the output gradient
        self.streams = {x: (mk(nt), mk(ni)) for x in ("q", "k", "v", "do")}
        self.joint = {x: torch.empty(T, H, D, device="cuda", dtype=dt)
                      for x in ("q", "k", "v", "do", "o", "dq", "dk", "dv")}
        self.out_streams = {x: (torch.empty(nt, H, D, device="cuda", dtype=dt),
                                torch.empty(ni, H, D, device="cuda", dtype=dt))
                            for x in ("o", "dq", "dk", "dv")}
        self.lse = torch.empty(H, T, device="cuda", dtype=torch.float32)
        self.ws = torch.empty(max(256, probe.bwd_workspace_bytes()), device="cuda",
                              dtype=torch.uint8)
        self.plan = None

    def __call__(self):
        pvj, wl, j = self.pvj, self.wl, self.joint
        if self.reuse_plan and self.plan is not None:
            plan = self.plan
        else:
            plan = pvj.Plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype).upload()
        in_pack = self.rope == "pack"
        for x in ("q", "k", "v"):
            pvj.pack(plan, *self.streams[x], joint=j[x], rope=in_pack and x != "v")
        pvj.varlen_attn_fwd(plan, j["q"], j["k"], j["v"], rope_fused=not in_pack, out=j["o"],
                            lse=self.lse)
        pvj.unpack(plan, j["o"], *self.out_streams["o"])
        if self.backward:
            pvj.pack(plan, *self.streams["do"], joint=j["do"])
            pvj.varlen_attn_bwd(plan, j["q"], j["k"], j["v"], j["o"], self.lse, j["do"],
                                rope_fused=not in_pack, rope_prerotated=in_pack,
                                dq=j["dq"], dk=j["dk"], dv=j["dv"], workspace=self.ws)
            for x in ("dq", "dk", "dv"):
                pvj.unpack(plan, j[x], *self.out_streams[x])
        self.plan = plan


class StreamMajorStep:
    """The same pass with every token tensor in the stream-major layout: the
    text stream's rows and then the image stream's rows of Q, K, V, dO (and of
    O, dQ, dK, dV) are two views of one allocation, which the attention reads
    and writes directly, so no pack or unpack pass runs; RoPE is a standalone
    pass on Q and K, and the backward unrotates dQ', dK' in its epilogues.
    The outputs are bitwise those of PackStep's for the same stream inputs."""

    def __init__(self, wl, seed):
        import torch
        import packed_varlen_joint_amd as pvj
        self.pvj = pvj
        self.wl = wl
        self.backward = wl.backward
        H, D = wl.n_heads, wl.head_dim
        probe = pvj.Plan(wl.samples, H, D, wl.dtype)
        nt, T = probe.n_text, wl.n_tokens
        g = torch.Generator(device="cuda").manual_seed(seed)
        mk = lambda: torch.randn(T, H, D, device="cuda", generator=g).to(torch.bfloat16)
        self.t = {x: mk() for x in ("q", "k", "v", "do")}
        for x in ("qr", "kr", "o", "dq", "dk", "dv"):
            self.t[x] = torch.empty(T, H, D, device="cuda", dtype=torch.bfloat16)
        # the streams a model's projections write and read: views of the tensors
        self.streams = {x: (y[:nt], y[nt:]) for x, y in self.t.items()}
        self.lse = torch.empty(H, T, device="cuda", dtype=torch.float32)
        self.ws = torch.empty(max(256, probe.bwd_workspace_bytes()), device="cuda",
                              dtype=torch.uint8)
        self.plan = None

    def __call__(self):
        pvj, wl, t = self.pvj, self.wl, self.t
        plan = pvj.Plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype).upload()
        pvj.rope2d_apply(plan, t["q"], t["qr"], stream_major=True)
        pvj.rope2d_apply(plan, t["k"], t["kr"], stream_major=True)
        pvj.varlen_attn_fwd(plan, t["qr"], t["kr"], t["v"], out=t["o"], lse=self.lse,
                            stream_major=True)
        if self.backward:
            pvj.varlen_attn_bwd(plan, t["qr"], t["kr"], t["v"], t["o"], self.lse, t["do"],
                                rope_prerotated=True, dq=t["dq"], dk=t["dk"], dv=t["dv"],
                                workspace=self.ws, stream_major=True)
        self.plan = plan


def stream_major_bench(wl, steps, warmup, seed=0):
    """The training step in the stream-major layout (StreamMajorStep)."""
    step = StreamMajorStep(wl, seed)
    ms, kms = time_step(step, steps, warmup)
    S2 = _sum_len_sq(step.plan, len(wl.samples))
    f = (14.0 if step.backward else 4.0) * wl.n_heads * wl.head_dim * S2
    kt = sum(kms.values())
    out = {"workload": wl.name, "seed": seed, "layout": "stream-major",
           "step": "plan+rope Q,K+attn fwd" + ("+attn bwd" if step.backward else ""),
           "ms_per_step": round(ms, 4), "tflops": round(f / (ms * 1e-3) / 1e12, 2),
           "tokens_per_s": round(wl.n_tokens / (ms * 1e-3), 1),
           "attn_kernel_ms": round(kt, 4) if kt else None}
    for k, v in kms.items():
        out[k + "_ms"] = round(v, 4)
    out["median_of_50_steps"] = median_steps(step, 50)
    return out


def _sum_len_sq(plan, n):
    cu = plan.cu_seqlens
    return float(sum((cu[i + 1] - cu[i]) ** 2 for i in range(n)))


def time_step(step, steps, warmup):
    """Mean wall time of `steps` steps (synchronised around the loop) and the
    attention kernels' mean times per step (HIP events on the launch stream)."""
    import torch
    pvj = step.pvj
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    pvj.profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    kms = {}
    for k in ("attn_fwd", "attn_bwd", "attn_bwd_dq"):
        tot, n = pvj.profile_read(k)
        if n:
            kms[k] = tot / steps
    pvj.profile_enable(False)
    return ms, kms


def pack_bench(name, steps, warmup=2, seed=0, backward=None, reuse_plan=False):
    """One of the other packs (the multi-prompt CFG inference pack, the 1024^2
    packs, the extreme-shape pack, the two-frame editing pack with 3-axis
    RoPE, other training-pack seeds), timed like the main step: plan, pack
    with RoPE, attention forward, unpack O, and for training packs pack dO,
    attention backward and unpack the gradients.  Reports the step rate and
    the attention kernels' own rate (events on the launch stream)."""
    from pvj_inputs import workload
    wl = workload(name, seed)
    step = PackStep(wl, seed, backward=backward, reuse_plan=reuse_plan)
    ms, kms = time_step(step, steps, warmup)
    S2 = _sum_len_sq(step.plan, len(wl.samples))
    bwd = step.backward
    f = (14.0 if bwd else 4.0) * wl.n_heads * wl.head_dim * S2
    kt = sum(kms.values())
    out = {"workload": wl.name, "seed": seed, "n_samples": len(wl.samples),
           "n_tokens": wl.n_tokens, "sum_len_sq": int(S2), "backward": bwd,
           "plan": "built once, reused" if reuse_plan else "built every step",
           "ms_per_step": round(ms, 4),
           "tflops": round(f / (ms * 1e-3) / 1e12, 2),
           "attn_kernel_ms": round(kt, 4) if kt else None,
           "attn_kernel_tflops": round(f / (kt * 1e-3) / 1e12, 2) if kt else None,
           "attn_kernel_frac_of_peak": round(f / (kt * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
           if kt else None,
           "tokens_per_s": round(wl.n_tokens / (ms * 1e-3), 1)}
    if "attn_fwd" in kms:
        out["fwd_ms"] = round(kms["attn_fwd"], 4)
        out["fwd_tflops"] = round(4.0 * wl.n_heads * wl.head_dim * S2 /
                                  (kms["attn_fwd"] * 1e-3) / 1e12, 2)
    if bwd and "attn_bwd" in kms and "attn_bwd_dq" in kms:
        tb = kms["attn_bwd"] + kms["attn_bwd_dq"]
        out["bwd_ms"] = round(tb, 4)
        out["bwd_tflops"] = round(10.0 * wl.n_heads * wl.head_dim * S2 / (tb * 1e-3) / 1e12, 2)
    return out


def seeds_bench(name, seeds, steps, warmup=2):
    """The training pack for several draws (seeds), forward + backward, and the
    mean of the per-seed rates."""
    import torch
    per = []
    for sd in seeds:
        per.append(pack_bench(name, steps, warmup, seed=sd))
        torch.cuda.empty_cache()
    keys = ("ms_per_step", "tflops", "attn_kernel_tflops", "attn_kernel_frac_of_peak",
            "fwd_tflops", "bwd_tflops", "tokens_per_s", "n_tokens")
    mean = {k: round(sum(r[k] for r in per) / len(per), 4) for k in keys}
    return {"per_seed": per, "mean": mean}


def cfg_packed_vs_separate(steps, warmup=2):
    """The 1024^2 CFG pack (cond + uncond in one pack) against the two samples
    as separate single-sample calls, each a full forward step (plan, pack with
    RoPE, forward, unpack); kernel-level and step-level times and their ratio
    (separate / packed)."""
    from pvj_inputs import workload, Workload
    wl = workload("cfg_1024")
    packed = PackStep(wl, 0)
    parts = [PackStep(Workload("cfg_1024_part%d" % i, [s], wl.n_heads, wl.head_dim, wl.dtype,
                               False, wl.seed), 0) for i, s in enumerate(wl.samples)]

    def both():
        for p in parts:
            p()
    both.pvj = packed.pvj
    ms_p, k_p = time_step(packed, steps, warmup)
    ms_s, k_s = time_step(both, steps, warmup)
    kp, ks = k_p.get("attn_fwd", 0.0), k_s.get("attn_fwd", 0.0)
    return {"packed_step_ms": round(ms_p, 4), "separate_step_ms": round(ms_s, 4),
            "step_ratio": round(ms_s / ms_p, 4),
            "packed_attn_kernel_ms": round(kp, 4), "separate_attn_kernel_ms": round(ks, 4),
            "attn_kernel_ratio": round(ks / kp, 4) if kp else None,
            "_note": "separate = the two samples as two single-sample plans and calls per step; "
                     "ratio > 1 means the pack is faster"}


def median_steps(step, n):
    """Median, min and max of n individually synchronised steps (ms)."""
    import torch
    ts = []
    for _ in range(n):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        step()
        torch.cuda.synchronize()
        ts.append((time.perf_counter() - t0) * 1e3)
    ts.sort()
    return {"n": n, "median_ms": round(ts[n // 2], 4), "min_ms": round(ts[0], 4),
            "max_ms": round(ts[-1], 4), "total_s": round(sum(ts) / 1e3, 3)}


def rope_bench(wl, reps):
    """The standalone per-sample 2D RoPE kernel on one [T, H, D] tensor of the
    pack (out of place): algorithmic bytes = one read and one write."""
    import torch
    import packed_varlen_joint_amd as pvj
    plan = pvj.Plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype).upload()
    dt = plan.torch_dtype
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn(plan.n_tokens, wl.n_heads, wl.head_dim, device="cuda", generator=g).to(dt)
    y = torch.empty_like(x)
    for _ in range(3):
        pvj.rope2d_apply(plan, x, y)
    torch.cuda.synchronize()
    pvj.profile_enable(True)
    for _ in range(reps):
        pvj.rope2d_apply(plan, x, y)
    torch.cuda.synchronize()
    tot, n = pvj.profile_read("rope2d")
    pvj.profile_enable(False)
    ms = tot / n
    nbytes = 2 * x.numel() * x.element_size()
    return {"ms": round(ms, 4), "bytes": nbytes, "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "_note": "[%d, %d, %d] %s, read + write once, mean of %d launches (events)" % (
                plan.n_tokens, wl.n_heads, wl.head_dim, wl.dtype, reps)}


def chain_bench(wl, reps):
    """HBM-bound chains around the attention on both streams of the pack, at the
    backbone width H*D: adaptive layer norm + modulation and gate + residual,
    forward and backward.  Each op runs as one call over both streams (rows
    [text; image], per-sample vectors [2B, C]) and, for comparison, as two
    one-stream calls.  Timed with events on torch's current stream (the stream
    the library launches on); bytes are algorithmic (each tensor read or
    written once)."""
    import torch
    import packed_varlen_joint_amd as pvj
    plan = pvj.Plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype).upload()
    C = wl.n_heads * wl.head_dim
    dt = plan.torch_dtype
    elt = 2 if wl.dtype == "bf16" else 4
    B = len(wl.samples)
    nt, ni = plan.n_text, plan.n_image
    rows = nt + ni
    g = torch.Generator(device="cuda").manual_seed(7)
    mk = lambda r: torch.randn(r, C, device="cuda", generator=g).to(dt)

    def wsp(op, which):
        return torch.empty(max(256, pvj.chain_workspace_bytes(plan, op, which, C)),
                           dtype=torch.uint8, device="cuda")

    full = dict(x=mk(rows), y=mk(rows), d=mk(rows), sh=mk(2 * B), sc=mk(2 * B), gt=mk(2 * B),
                o=torch.empty(rows, C, device="cuda", dtype=dt),
                dx=torch.empty(rows, C, device="cuda", dtype=dt),
                ws_a=wsp(pvj.CHAIN_ADALN, "both"), ws_g=wsp(pvj.CHAIN_GATE, "both"))
    # the one-stream calls work on the text and image halves of the same data
    per = {}
    for which, rs, vs in (("text", slice(0, nt), slice(0, B)),
                          ("image", slice(nt, rows), slice(B, 2 * B))):
        t = {k: (v[rs] if k in ("x", "y", "d", "o", "dx") else v[vs].contiguous())
             for k, v in full.items() if not k.startswith("ws")}
        t.update(ws_a=wsp(pvj.CHAIN_ADALN, which), ws_g=wsp(pvj.CHAIN_GATE, which))
        per[which] = t
    ops = {
        "adaln_fwd": (2, lambda w, t: pvj.adaln_modulate(plan, w, t["x"], t["sh"], t["sc"],
                                                         y=t["o"])),
        "gate_residual_fwd": (3, lambda w, t: pvj.gate_residual(plan, w, t["x"], t["y"], t["gt"],
                                                                out=t["o"])),
        "adaln_bwd": (3, lambda w, t: pvj.adaln_modulate_bwd(plan, w, t["x"], t["sc"], t["d"],
                                                             dx=t["dx"], workspace=t["ws_a"])),
        "gate_residual_bwd": (3, lambda w, t: pvj.gate_residual_bwd(plan, w, t["y"], t["gt"],
                                                                    t["d"], dy=t["dx"],
                                                                    workspace=t["ws_g"])),
    }

    def timed(calls):
        for _ in range(2):
            for c in calls:
                c()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for c in calls:
                c()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {}
    for name, (ntens, fn) in ops.items():
        one = [lambda fn=fn: fn("both", full)]
        two = [lambda fn=fn, w=w: fn(w, per[w]) for w in ("text", "image")
               if (nt if w == "text" else ni) > 0]
        ms = timed(one)
        ms2 = timed(two)
        nbytes = ntens * rows * C * elt
        out[name] = {"ms": round(ms, 4), "bytes": nbytes,
                     "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "two_stream_calls_ms": round(ms2, 4),
                     "two_stream_calls_frac_hbm": round(
                         nbytes / (ms2 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    out["_note"] = ("one call over both streams (text rows then image rows), hidden %d, "
                    "algorithmic bytes = tensors read + written once (%d rows); "
                    "two_stream_calls_*: the same work as one call per stream" % (C, rows))
    return out


def proj_bench(wl, reps):
    """The per-stream projections with the pack / unpack fused in, at the
    backbone width (hidden = H*D): QKV projection writing joint Q, K, V with
    RoPE, and the output projection reading the joint O; both streams per call,
    algorithmic FLOP 2 * rows * hidden * out_features."""
    import torch
    import packed_varlen_joint_amd as pvj
    plan = pvj.Plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype).upload()
    HD = wl.n_heads * wl.head_dim
    C = HD
    g = torch.Generator(device="cuda").manual_seed(11)
    mk = lambda *sh: (torch.randn(*sh, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    xs = {"text": mk(plan.n_text, C), "image": mk(plan.n_image, C)}
    wq = {w: mk(3 * HD, C) for w in xs}
    wo = {w: mk(C, HD) for w in xs}
    q, k, v = (torch.empty(plan.n_tokens, wl.n_heads, wl.head_dim, device="cuda",
                           dtype=torch.bfloat16) for _ in range(3))
    ys = {w: torch.empty(xs[w].shape[0], C, device="cuda", dtype=torch.bfloat16) for w in xs}
    rows = plan.n_text + plan.n_image
    # the unfused pair for comparison: the library GEMM (torch -> hipBLASLt) per
    # stream and projection, then the separate pack (+RoPE) / unpack passes
    import torch.nn.functional as F
    wparts = {w: [wq[w][i * HD:(i + 1) * HD].contiguous() for i in range(3)] for w in xs}
    st = {w: [torch.empty(xs[w].shape[0], wl.n_heads, wl.head_dim, device="cuda",
                          dtype=torch.bfloat16) for _ in range(3)] for w in xs}
    o_t = torch.empty(plan.n_text, wl.n_heads, wl.head_dim, device="cuda", dtype=torch.bfloat16)
    o_i = torch.empty(plan.n_image, wl.n_heads, wl.head_dim, device="cuda", dtype=torch.bfloat16)

    def qkv_unfused():
        for w in xs:
            for i in range(3):
                torch.matmul(xs[w], wparts[w][i].t(), out=st[w][i].view(-1, HD))
        for i, (dst, rope) in enumerate(((q, True), (k, True), (v, False))):
            pvj.pack(plan, st["text"][i], st["image"][i], dst, rope=rope)

    def out_unfused():
        pvj.unpack(plan, q, o_t, o_i)
        torch.matmul(o_t.view(-1, HD), wo["text"].t(), out=ys["text"])
        torch.matmul(o_i.view(-1, HD), wo["image"].t(), out=ys["image"])

    # the stream-major layout: the library GEMMs write Q, K, V straight into
    # the text rows and the image rows of one tensor each, RoPE is one pass
    # over Q and K in place, and the output GEMMs read O's two row ranges; no
    # pack or unpack pass
    nt = plan.n_text
    sm = [torch.empty(plan.n_tokens, wl.n_heads, wl.head_dim, device="cuda",
                      dtype=torch.bfloat16) for _ in range(3)]

    def qkv_stream_major():
        for w, rr in (("text", slice(0, nt)), ("image", slice(nt, None))):
            for i in range(3):
                torch.matmul(xs[w], wparts[w][i].t(), out=sm[i][rr].view(-1, HD))
        pvj.rope2d_apply(plan, sm[0], sm[0], stream_major=True)
        pvj.rope2d_apply(plan, sm[1], sm[1], stream_major=True)

    def out_stream_major():
        torch.matmul(sm[2][:nt].view(-1, HD), wo["text"].t(), out=ys["text"])
        torch.matmul(sm[2][nt:].view(-1, HD), wo["image"].t(), out=ys["image"])

    ops = {
        "qkv_proj_pack": (2.0 * rows * C * 3 * HD, lambda: [pvj.qkv_proj_pack(
            plan, w, xs[w], wq[w], q=q, k=k, v=v, rope=True) for w in xs]),
        "out_proj_unpack": (2.0 * rows * HD * C, lambda: [pvj.out_proj_unpack(
            plan, w, q, wo[w], y=ys[w]) for w in xs]),
        "qkv_library_gemm_then_pack": (2.0 * rows * C * 3 * HD, qkv_unfused),
        "out_unpack_then_library_gemm": (2.0 * rows * HD * C, out_unfused),
        "qkv_library_gemm_stream_major": (2.0 * rows * C * 3 * HD, qkv_stream_major),
        "out_library_gemm_stream_major": (2.0 * rows * HD * C, out_stream_major),
    }
    out = {}
    for name, (flop, fn) in ops.items():
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = flop / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                     "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    out["fused_over_unfused_time"] = {
        "qkv": round(out["qkv_proj_pack"]["ms"] / out["qkv_library_gemm_then_pack"]["ms"], 3),
        "out": round(out["out_proj_unpack"]["ms"] / out["out_unpack_then_library_gemm"]["ms"], 3)}
    out["_note"] = ("both streams per call, hidden %d, %d rows; *_library_* = torch matmul "
                    "(hipBLASLt) per stream and projection plus the separate pack (+RoPE) or "
                    "unpack pass; *_stream_major = the same GEMMs writing / reading the "
                    "stream-major tensors' row ranges, RoPE one in-place pass over Q and K, "
                    "no pack or unpack" % (C, rows))
    return out


def cpu_baseline(wl, seconds):
    """The oracle (fp64 NumPy, as it stands) on a bounded sample of the workload:
    forward + backward of (sample, head) slices, smallest samples first, until
    about `seconds` of CPU work."""
    import numpy as np
    import oracle
    from pvj_inputs import draw_tensors
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    lens = oracle.sample_lengths(wl.samples)
    axes = 3 if wl.frames else 2
    order = sorted(range(len(wl.samples)), key=lambda i: lens[i])
    flops = 0.0
    done = []
    t0 = time.perf_counter()
    for i in order:
        s = wl.samples[i]
        L = int(lens[i])
        if L == 0:
            continue
        for h in range(wl.n_heads):
            q, k, v, do = draw_tensors(L, 1, wl.head_dim, wl.dtype, 7 + i * 100 + h, n=4)
            oracle.attn_fwd(q, k, v, [s], rope=True, axes=axes)
            oracle.attn_bwd(q, k, v, do, [s], rope=True, axes=axes)
            flops += 14.0 * wl.head_dim * L * L
            done.append((i, h, L))
            if time.perf_counter() - t0 >= seconds:
                break
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    lens = sorted({L for (_, _, L) in done})
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "fp64 oracle forward+backward (RoPE) of %d (sample, head) slices of the "
                      "workload pack, sample lengths %s, %.1f s" % (len(done), lens, dt)}


def cpu_baseline_one_thread(seconds):
    """The oracle's forward on the single 1024^2 sample (4,352 tokens), one BLAS
    thread, head by head for about `seconds`."""
    import numpy as np
    import oracle
    from pvj_inputs import draw_tensors, workload
    from threadpoolctl import threadpool_limits
    wl = workload("single_1024")
    L = int(oracle.sample_lengths(wl.samples)[0])
    done = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for h in range(wl.n_heads):
            q, k, v = draw_tensors(L, 1, wl.head_dim, wl.dtype, 11 + h, n=3)
            oracle.attn_fwd(q, k, v, wl.samples, rope=True)
            done += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    flops = 4.0 * wl.head_dim * L * L * done
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": "fp64 oracle forward (RoPE) of %d of the 24 heads of the single 1024^2 "
                      "sample (L = %d), one BLAS thread, %.1f s" % (done, L, dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="train_64k")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chains", action="store_true",
                    help="skip the memory-bound chain measurements (reported beside the step)")
    ap.add_argument("--rope", choices=("pack", "load"), default="pack",
                    help="RoPE fused into the Q/K pack (default) or applied on load inside "
                         "the attention kernels")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 512 MiB device copy (3 times), the reference for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    ap.add_argument("--only", choices=("rope", "cfg_1024", "single_1024", "infer_multi",
                                       "extreme_fwd", "chains", "projections",
                                       "stream_major"),
                    help="run just this measurement (for profiling) and print its JSON")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the pack is one GPU's data-parallel share "
              "(--gpus %d refused)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import packed_varlen_joint_amd as pvj
    from pvj_inputs import workload

    torch.cuda.set_device(0)
    if args.copy_calib:
        n = 512 * 1024 * 1024
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n, "launches": 3}), flush=True)
        return
    if args.only:
        if args.only == "rope":
            res = rope_bench(workload(args.workload, args.seed), 20)
        elif args.only == "chains":
            res = chain_bench(workload(args.workload, args.seed), 10)
        elif args.only == "projections":
            res = proj_bench(workload(args.workload, args.seed), 5)
        elif args.only == "stream_major":
            res = stream_major_bench(workload(args.workload, args.seed), args.steps,
                                     args.warmup, args.seed)
        elif args.only == "extreme_fwd":
            res = pack_bench("extreme", args.steps, args.warmup, backward=False)
        else:
            res = pack_bench(args.only, args.steps, args.warmup)
        print(json.dumps({"only": args.only, "result": res}), flush=True)
        return
    wl = workload(args.workload, args.seed)
    H, D = wl.n_heads, wl.head_dim
    probe = pvj.Plan(wl.samples, H, D, wl.dtype)
    cu = probe.cu_seqlens
    lens = [cu[i + 1] - cu[i] for i in range(len(wl.samples))]
    S2 = float(sum(L * L for L in lens))
    f_fwd = 4.0 * H * D * S2
    f_bwd = 10.0 * H * D * S2
    f_step = f_fwd + (f_bwd if wl.backward else 0.0)

    step = PackStep(wl, args.seed, args.rope)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    pvj.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = {}
    for name in pvj.KERNELS:
        ms, n = pvj.profile_read(name)
        if n:
            kern[name] = {"avg_ms": ms / n, "launches_per_step": n / args.steps,
                          "ms_per_step": ms / args.steps}
    pvj.profile_enable(False)

    ms_step = (t1 - t0) * 1e3 / args.steps
    value = f_step / (ms_step * 1e-3) / 1e12
    dom = max(kern, key=lambda k: kern[k]["ms_per_step"])
    # algorithmic FLOP per launch: the forward's two products; the dK/dV kernel's
    # score recompute, dP, dV and dK (8 of the backward's 10); the dQ kernel's
    # dQ product only (its second score/dP recompute is not counted)
    hd = H * D * S2
    per_launch = {"attn_fwd": 4.0 * hd, "attn_bwd": 8.0 * hd, "attn_bwd_dq": 2.0 * hd}
    executed = {"attn_fwd": 4.0 * hd, "attn_bwd": 8.0 * hd, "attn_bwd_dq": 6.0 * hd}
    roof = None
    if dom in per_launch:
        ach = per_launch[dom] / (kern[dom]["avg_ms"] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": _traffic(dom)}
    for k in kern:
        if k in per_launch:
            kern[k]["algorithmic_tflops"] = per_launch[k] / (kern[k]["avg_ms"] * 1e-3) / 1e12
            kern[k]["executed_tflops"] = executed[k] / (kern[k]["avg_ms"] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "seed": args.seed, "n_samples": len(wl.samples),
                   "n_tokens": wl.n_tokens, "heads": H, "head_dim": D,
                   "sum_len_sq": int(S2), "backward": wl.backward,
                   "rope": ("3-axis " if wl.frames else "2D ") + (
                       "fused into the Q/K pack" if args.rope == "pack" else "fused on load"),
                   "step": "plan+pack+attn fwd+unpack" + ("+pack dO+attn bwd+unpack grads"
                                                           if wl.backward else "")},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "tokens_per_s": round(wl.n_tokens / (ms_step * 1e-3), 1),
        "tflops_step_no_recompute": round((f_fwd + (8.0 * H * D * S2 if wl.backward else 0)) /
                                          (ms_step * 1e-3) / 1e12, 2),
        "kernels": {k: {kk: round(vv, 4) for kk, vv in v.items()} for k, v in kern.items()},
        "roofline": roof,
    }
    if "attn_fwd" in kern:
        out["fwd_tflops"] = round(f_fwd / (kern["attn_fwd"]["avg_ms"] * 1e-3) / 1e12, 2)
    if "attn_bwd" in kern and "attn_bwd_dq" in kern:
        t_bwd = kern["attn_bwd"]["avg_ms"] + kern["attn_bwd_dq"]["avg_ms"]
        out["bwd_tflops"] = round(f_bwd / (t_bwd * 1e-3) / 1e12, 2)
        out["fwd_bwd_kernel_tflops"] = round(
            (f_fwd + f_bwd) / ((kern["attn_fwd"]["avg_ms"] + t_bwd) * 1e-3) / 1e12, 2)
    if roof is not None:
        # the chip's sustained matrix-core rate, measured live beside the published peak
        ceil = pvj.diag_mfma_peak()
        roof["measured_ceiling"] = round(ceil, 1)
        roof["frac_of_measured_ceiling"] = round(roof["achieved"] / ceil, 4)
    # the same step, 50 times, each synchronised and timed on its own
    out["median_of_50_steps"] = median_steps(step, 50)
    del step
    torch.cuda.empty_cache()
    if wl.dtype == "bf16" and args.rope == "pack":
        # the same step with the token tensors in the stream-major layout
        sm = stream_major_bench(wl, args.steps, args.warmup, args.seed)
        sm["over_joint_step_time"] = round(sm["ms_per_step"] / ms_step, 4)
        out["stream_major_step"] = sm
        torch.cuda.empty_cache()
    if not args.no_chains:
        out["chains"] = chain_bench(wl, 10)
        out["rope_standalone"] = rope_bench(wl, 20)
        out["inference"] = pack_bench("infer_multi", 5)
        out["inference_reused_plan"] = pack_bench("infer_multi", 5, reuse_plan=True)
        out["other_packs"] = {
            "cfg_1024": pack_bench("cfg_1024", 20),
            "cfg_1024_reused_plan": pack_bench("cfg_1024", 20, reuse_plan=True),
            "single_1024": pack_bench("single_1024", 20),
            "extreme": pack_bench("extreme", 5),
            "extreme_fwd": pack_bench("extreme", 10, backward=False),
            "edit_1024": pack_bench("edit_1024", 5),
        }
        out["cfg_packed_vs_separate"] = cfg_packed_vs_separate(20)
        if args.workload == "train_64k":
            out["train_64k_seeds"] = seeds_bench("train_64k", range(5), 10)
        torch.cuda.empty_cache()
        if wl.dtype == "bf16":
            out["projections"] = proj_bench(wl, 5)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
        out["cpu_baseline_one_thread"] = cpu_baseline_one_thread(5.0)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
