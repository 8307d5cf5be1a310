"""Pins of the oracle's memory-bound chains (LayerNorm + adaptive modulation,
gate + residual) against what fixes them independently: the layer-norm
invariants and the library routine it reduces to, hand-computed per-sample
selection, finite differences and autograd for the backward."""
import numpy as np
import pytest

from oracle import chains

torch = pytest.importorskip("torch")

SAMPLES = [(2, 3, 4), (0, 0, 2), (1, 2, 0), (3, 1, 1, 2)]


def _rows(n, c, seed):
    return np.random.default_rng(seed).standard_normal((n, c))


def test_stream_sample_index_hand_example():
    # text rows: 4 of sample 0, 2 of sample 1, 0 of sample 2, 1 of sample 3
    assert chains.stream_sample_index(SAMPLES, chains.TEXT).tolist() == [0, 0, 0, 0, 1, 1, 3]
    # image rows: 6, 0, 2, then 3 x 1 x 2 frames = 6
    assert chains.stream_sample_index(SAMPLES, chains.IMAGE).tolist() == \
        [0] * 6 + [2] * 2 + [3] * 6


def test_layer_norm_invariants_and_library():
    x = _rows(9, 48, 1) * 3.0 + 2.0
    y = chains.layer_norm_rows(x, 0.0)
    assert np.allclose(y.mean(axis=1), 0.0, atol=1e-14)
    assert np.allclose((y ** 2).mean(axis=1), 1.0, atol=1e-12)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (48,), eps=1e-6).numpy()
    assert np.abs(chains.layer_norm_rows(x) - ref).max() < 1e-12
    # a constant row normalizes to zeros; scaling a row leaves LN unchanged
    assert np.all(chains.layer_norm_rows(np.full((1, 16), 5.0)) == 0.0)
    assert np.abs(chains.layer_norm_rows(7.0 * x, 0.0) - y).max() < 1e-12


def test_modulate_selects_per_sample_vectors():
    C = 8
    x = _rows(7, C, 2)
    shift = np.arange(4 * C, dtype=np.float64).reshape(4, C)
    scale = -0.5 * np.ones((4, C))
    scale[3] = 1.0
    y = chains.adaln_modulate(x, shift, scale, SAMPLES, chains.TEXT)
    ln = chains.layer_norm_rows(x)
    # text rows 0-3 -> sample 0, rows 4-5 -> sample 1, row 6 -> sample 3
    assert np.allclose(y[0], 0.5 * ln[0] + shift[0])
    assert np.allclose(y[5], 0.5 * ln[5] + shift[1])
    assert np.allclose(y[6], 2.0 * ln[6] + shift[3])
    # zero modulation is the plain layer norm
    z = chains.adaln_modulate(x, np.zeros((4, C)), np.zeros((4, C)), SAMPLES, chains.TEXT)
    assert np.abs(z - ln).max() == 0.0


def _fd(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        g[i] = (f(xp) - f(xm)) / (2 * h)
    return g


@pytest.mark.parametrize("stream", [chains.TEXT, chains.IMAGE])
def test_modulate_bwd_finite_differences(stream):
    C = 6
    n = len(chains.stream_sample_index(SAMPLES, stream))
    x, dy = _rows(n, C, 3), _rows(n, C, 4)
    shift, scale = _rows(4, C, 5), 0.3 * _rows(4, C, 6)
    dx, dsh, dsc = chains.adaln_modulate_bwd(x, scale, dy, SAMPLES, stream)
    L = lambda xx, sh, sc: float((chains.adaln_modulate(xx, sh, sc, SAMPLES, stream) * dy).sum())
    assert np.abs(dx - _fd(lambda v: L(v, shift, scale), x)).max() < 1e-6
    assert np.abs(dsh - _fd(lambda v: L(x, v, scale), shift)).max() < 1e-6
    assert np.abs(dsc - _fd(lambda v: L(x, shift, v), scale)).max() < 1e-6


def test_modulate_bwd_autograd():
    C = 32
    stream = chains.IMAGE
    si = chains.stream_sample_index(SAMPLES, stream)
    n = len(si)
    x, dy = _rows(n, C, 7), _rows(n, C, 8)
    shift, scale = _rows(4, C, 9), _rows(4, C, 10)
    tx = torch.from_numpy(x).requires_grad_()
    tsh = torch.from_numpy(shift).requires_grad_()
    tsc = torch.from_numpy(scale).requires_grad_()
    idx = torch.from_numpy(si)
    y = torch.nn.functional.layer_norm(tx, (C,), eps=1e-6) * (1 + tsc[idx]) + tsh[idx]
    (y * torch.from_numpy(dy)).sum().backward()
    dx, dsh, dsc = chains.adaln_modulate_bwd(x, scale, dy, SAMPLES, stream)
    assert np.abs(dx - tx.grad.numpy()).max() < 1e-11
    assert np.abs(dsh - tsh.grad.numpy()).max() < 1e-11
    assert np.abs(dsc - tsc.grad.numpy()).max() < 1e-11


def test_gate_residual_special_cases_and_bwd():
    C = 5
    stream = chains.IMAGE
    n = len(chains.stream_sample_index(SAMPLES, stream))
    x, y, dout = _rows(n, C, 11), _rows(n, C, 12), _rows(n, C, 13)
    assert np.all(chains.gate_residual(x, y, np.zeros((4, C)), SAMPLES, stream) == x)
    assert np.abs(chains.gate_residual(x, y, np.ones((4, C)), SAMPLES, stream) - (x + y)).max() == 0
    gate = _rows(4, C, 14)
    dx, dy, dg = chains.gate_residual_bwd(y, gate, dout, SAMPLES, stream)
    L = lambda xx, yy, gg: float((chains.gate_residual(xx, yy, gg, SAMPLES, stream) * dout).sum())
    assert np.abs(dx - _fd(lambda v: L(v, y, gate), x)).max() < 1e-6
    assert np.abs(dy - _fd(lambda v: L(x, v, gate), y)).max() < 1e-6
    assert np.abs(dg - _fd(lambda v: L(x, y, v), gate)).max() < 1e-6
    # samples with no rows in the stream get zero gate gradient (sample 1 here)
    assert np.all(dg[1] == 0.0)
