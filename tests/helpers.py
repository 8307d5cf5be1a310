"""Shared helpers for the GPU parity tests: device upload, tolerances, guard bands."""
import sys

import numpy as np

# bf16 bar: max-abs <= 2e-2 and mean-abs <= 2e-3 on O, dQ, dK, dV; plus a
# relative-RMS bar of 1e-2 (bf16 rounding is ~2^-9 relative, so this catches
# errors the absolute bars miss when outputs are small).  fp32 bar: 1e-4.
TOL = {
    "bf16": dict(max_abs=2e-2, mean_abs=2e-3, rel_rms=1e-2),
    "f32": dict(max_abs=1e-4, mean_abs=1e-4, rel_rms=1e-5),
}
LSE_TOL = {"bf16": 1e-2, "f32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(dt):
    import torch
    return torch.bfloat16 if dt == "bf16" else torch.float32


def to_dev(x, dt):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch_dtype(dt)).cuda()


def to_np(t):
    import torch
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    if d.size == 0:
        return dict(max_abs=0.0, mean_abs=0.0, rel_rms=0.0)
    nref = np.sqrt((ref ** 2).sum())
    return dict(max_abs=float(d.max()), mean_abs=float(d.mean()),
                rel_rms=float(np.sqrt((d ** 2).sum()) / max(nref, 1e-30)))


def assert_close(name, got, ref, dt):
    e = errors(got, ref)
    say("   %-10s max_abs=%.3e mean_abs=%.3e rel_rms=%.3e" % (name, e["max_abs"], e["mean_abs"],
                                                             e["rel_rms"]))
    assert np.all(np.isfinite(got)), name + ": non-finite output"
    t = TOL[dt]
    for k in ("max_abs", "mean_abs", "rel_rms"):
        assert e[k] <= t[k], "%s %s %.3e > %.3e" % (name, k, e[k], t[k])
    return e


def assert_lse(got, ref, dt):
    d = float(np.abs(np.asarray(got, np.float64) - ref).max()) if np.size(ref) else 0.0
    say("   %-10s max_abs=%.3e" % ("lse", d))
    assert d <= LSE_TOL[dt], "lse max_abs %.3e" % d


SENTINEL = 12288.0  # exactly representable in bf16


class Guarded:
    """A [rows, H, D] device tensor with sentinel-filled margins before and after,
    to catch writes outside the output at ragged tile tails."""

    def __init__(self, rows, H, D, dt, margin_rows=64):
        import torch
        self.full = torch.full((rows + 2 * margin_rows, H, D), SENTINEL, dtype=torch_dtype(dt),
                               device="cuda")
        self.m = margin_rows
        self.rows = rows
        self.t = self.full[margin_rows:margin_rows + rows]

    def check(self, name=""):
        a = self.full[:self.m].float()
        b = self.full[self.m + self.rows:].float()
        assert bool((a == SENTINEL).all()) and bool((b == SENTINEL).all()), \
            "write outside the output %s" % name


class GuardedLse:
    def __init__(self, H, T, margin=256):
        import torch
        self.full = torch.full((H * T + 2 * margin,), SENTINEL, dtype=torch.float32, device="cuda")
        self.m = margin
        self.t = self.full[margin:margin + H * T].view(H, T)
        self.n = H * T

    def check(self):
        assert bool((self.full[:self.m] == SENTINEL).all())
        assert bool((self.full[self.m + self.n:] == SENTINEL).all())
