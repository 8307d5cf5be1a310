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
    def __init__(self, wl, seed, rope="pack"):
        import torch
        import packed_varlen_joint_amd as pvj
        self.pvj = pvj
        self.wl = wl
        self.rope = rope
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
        plan = pvj.Plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype).upload()
        in_pack = self.rope == "pack"
        for x in ("q", "k", "v"):
            pvj.pack(plan, *self.streams[x], joint=j[x], rope=in_pack and x != "v")
        pvj.varlen_attn_fwd(plan, j["q"], j["k"], j["v"], rope_fused=not in_pack, out=j["o"],
                            lse=self.lse)
        pvj.unpack(plan, j["o"], *self.out_streams["o"])
        if wl.backward:
            pvj.pack(plan, *self.streams["do"], joint=j["do"])
            pvj.varlen_attn_bwd(plan, j["q"], j["k"], j["v"], j["o"], self.lse, j["do"],
                                rope_fused=not in_pack, rope_prerotated=in_pack,
                                dq=j["dq"], dk=j["dk"], dv=j["dv"], workspace=self.ws)
            for x in ("dq", "dk", "dv"):
                pvj.unpack(plan, j[x], *self.out_streams[x])
        self.plan = plan


def pack_bench(name, steps, warmup=2):
    """One of the other packs (the multi-prompt CFG inference pack, the 1024^2
    CFG pack, the extreme-shape pack, the two-frame editing pack with 3-axis
    RoPE), timed like the main step: plan, pack with
    RoPE, attention forward, unpack O, and for training packs pack dO, attention
    backward and unpack the gradients.  Reports the step rate and the attention
    kernels' own rate (events on the launch stream)."""
    import torch
    import packed_varlen_joint_amd as pvj
    from pvj_inputs import workload
    wl = workload(name)
    step = PackStep(wl, 0)
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
    cu = step.plan.cu_seqlens
    S2 = float(sum((cu[i + 1] - cu[i]) ** 2 for i in range(len(wl.samples))))
    f = (14.0 if wl.backward else 4.0) * wl.n_heads * wl.head_dim * S2
    kt = sum(kms.values())
    return {"workload": wl.name, "n_samples": len(wl.samples), "n_tokens": wl.n_tokens,
            "backward": wl.backward, "ms_per_step": round(ms, 4),
            "tflops": round(f / (ms * 1e-3) / 1e12, 2),
            "attn_kernel_tflops": round(f / (kt * 1e-3) / 1e12, 2) if kt else None,
            "attn_kernel_frac_of_peak": round(f / (kt * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
            if kt else None,
            "tokens_per_s": round(wl.n_tokens / (ms * 1e-3), 1)}


def chain_bench(wl, reps):
    """HBM-bound chains around the attention on both streams of the pack, at the
    backbone width H*D: adaptive layer norm + modulation and gate + residual,
    forward and backward.  Timed with events on torch's current stream (the
    stream the library launches on); bytes are algorithmic (each tensor read
    or written once)."""
    import torch
    import packed_varlen_joint_amd as pvj
    plan = pvj.Plan(wl.samples, wl.n_heads, wl.head_dim, wl.dtype).upload()
    C = wl.n_heads * wl.head_dim
    dt = plan.torch_dtype
    elt = 2 if wl.dtype == "bf16" else 4
    B = len(wl.samples)
    g = torch.Generator(device="cuda").manual_seed(7)
    out = {}
    streams = [("text", plan.n_text), ("image", plan.n_image)]
    data = {}
    for which, n in streams:
        mk = lambda r: torch.randn(r, C, device="cuda", generator=g).to(dt)
        data[which] = dict(x=mk(n), y=mk(n), d=mk(n), sh=mk(B), sc=mk(B), gt=mk(B),
                           o=torch.empty(n, C, device="cuda", dtype=dt),
                           dx=torch.empty(n, C, device="cuda", dtype=dt),
                           ws_a=torch.empty(max(256, pvj.chain_workspace_bytes(
                               plan, pvj.CHAIN_ADALN, which, C)), dtype=torch.uint8,
                               device="cuda"),
                           ws_g=torch.empty(max(256, pvj.chain_workspace_bytes(
                               plan, pvj.CHAIN_GATE, which, C)), dtype=torch.uint8,
                               device="cuda"))
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
    rows = plan.n_text + plan.n_image
    for name, (ntens, fn) in ops.items():
        for _ in range(2):
            for w, _n in streams:
                fn(w, data[w])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for w, _n in streams:
                fn(w, data[w])
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = ntens * rows * C * elt
        out[name] = {"ms": round(ms, 4), "bytes": nbytes,
                     "GB_per_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    out["_note"] = ("both streams per call, hidden %d, algorithmic bytes = tensors read + "
                    "written once (%d rows)" % (C, rows))
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
    ops = {
        "qkv_proj_pack": (2.0 * rows * C * 3 * HD, lambda: [pvj.qkv_proj_pack(
            plan, w, xs[w], wq[w], q=q, k=k, v=v, rope=True) for w in xs]),
        "out_proj_unpack": (2.0 * rows * HD * C, lambda: [pvj.out_proj_unpack(
            plan, w, q, wo[w], y=ys[w]) for w in xs]),
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
    out["_note"] = "both streams per call, hidden %d, %d rows" % (C, rows)
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
    if not args.no_chains:
        out["chains"] = chain_bench(wl, 10)
        out["inference"] = pack_bench("infer_multi", 5)
        out["other_packs"] = {n: pack_bench(n, 5) for n in ("cfg_1024", "extreme", "edit_1024")}
        if wl.dtype == "bf16":
            out["projections"] = proj_bench(wl, 5)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
