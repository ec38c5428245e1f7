"""Pins of the float64 oracle's backward: finite differences, invariants, library autograd."""
import numpy as np
import pytest
import torch

from oracle import oracle as ora
from lm_head_cross_pg_amd import synth


def _fd_grads(H, E, y, c, g, mask=None, h=1e-5):
    dH = np.zeros_like(H)
    dE = np.zeros_like(E)
    for idx in np.ndindex(*H.shape):
        Hp, Hm = H.copy(), H.copy()
        Hp[idx] += h
        Hm[idx] -= h
        dH[idx] = (ora.loss(Hp, E, y, c, g, mask) - ora.loss(Hm, E, y, c, g, mask)) / (2 * h)
    for idx in np.ndindex(*E.shape):
        Ep, Em = E.copy(), E.copy()
        Ep[idx] += h
        Em[idx] -= h
        dE[idx] = (ora.loss(H, Ep, y, c, g, mask) - ora.loss(H, Em, y, c, g, mask)) / (2 * h)
    return dH, dE


def _check(an, fd, rel):
    scale = np.max(np.abs(fd))
    assert np.max(np.abs(an - fd)) <= rel * scale
    assert np.linalg.norm(an - fd) <= rel * np.linalg.norm(fd)


@pytest.mark.slow
def test_finite_differences_fd_shape():
    """The finite-difference shape of the training workload: T=64, D=32, V=128, c=30, g=1/T."""
    inp = synth.make_inputs("fd", seed=0)
    H = synth.as_f64(inp["hidden"], "f32")
    E = synth.as_f64(inp["embed"], "f32")
    y = inp["target"]
    g = 1.0 / H.shape[0]
    dH, dE = ora.backward(H, E, y, 30.0, g)
    fdH, fdE = _fd_grads(H, E, y, 30.0, g)
    _check(dH, fdH, 1e-6)
    _check(dE, fdE, 1e-6)


@pytest.mark.parametrize("c", [2.0, 0.0])
def test_finite_differences_strong_curvature(c):
    """Logits of several c so that the softcap derivative (1 - tanh^2) is far from 1."""
    rng = np.random.default_rng(21)
    H = rng.standard_normal((6, 4)) * 3.0
    E = rng.standard_normal((9, 4)) * 1.0
    y = rng.integers(0, 9, size=6)
    mask = np.array([1, 1, 0, 1, 0, 1], dtype=np.uint8)
    g = 1.0 / mask.sum()
    z = H @ E.T
    assert np.max(np.abs(z)) > 2 * 2.0           # curvature region of the c = 2 cap is reached
    dH, dE = ora.backward(H, E, y, c, g, mask)
    fdH, fdE = _fd_grads(H, E, y, c, g, mask)
    _check(dH, fdH, 1e-6)
    _check(dE, fdE, 1e-6)
    np.testing.assert_array_equal(dH[[2, 4]], 0.0)


def test_gradient_invariants():
    """<dH,H> = <dE,E> = <dZ,Z>, and rows of dS sum to zero."""
    rng = np.random.default_rng(22)
    H = rng.standard_normal((20, 8)) * 4.0
    E = rng.standard_normal((15, 8)) * 0.8
    y = rng.integers(0, 15, size=20)
    c, g = 5.0, 0.05
    dH, dE = ora.backward(H, E, y, c, g)
    z = ora.logits(H, E)
    s = ora.softcap(z, c)
    p = np.exp(s - ora.log_sum_exp(s)[:, None])
    onehot = np.eye(15)[y]
    dS = g * (p - onehot)
    np.testing.assert_allclose(dS.sum(axis=1), 0.0, atol=1e-15)
    dZ = dS * ora.softcap_derivative(z, c)
    a, b, cc = np.sum(dH * H), np.sum(dE * E), np.sum(dZ * z)
    assert a == pytest.approx(cc, rel=1e-12) and b == pytest.approx(cc, rel=1e-12)


def test_no_cap_matches_torch_autograd():
    rng = np.random.default_rng(23)
    H = rng.standard_normal((17, 6)) * 2.0
    E = rng.standard_normal((11, 6)) * 0.7
    y = rng.integers(0, 11, size=17)
    Ht = torch.tensor(H, requires_grad=True)
    Et = torch.tensor(E, requires_grad=True)
    loss = torch.nn.functional.cross_entropy(Ht @ Et.T, torch.tensor(y), reduction="mean")
    loss.backward()
    dH, dE = ora.backward(H, E, y, 0.0, 1.0 / 17)
    np.testing.assert_allclose(dH, Ht.grad.numpy(), rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dE, Et.grad.numpy(), rtol=1e-11, atol=1e-14)


def test_softcap_matches_torch_autograd():
    """Softcapped logits through torch's float64 tanh and cross-entropy autograd."""
    rng = np.random.default_rng(24)
    H = rng.standard_normal((13, 5)) * 6.0
    E = rng.standard_normal((10, 5)) * 1.0
    y = rng.integers(0, 10, size=13)
    c = 4.0
    Ht = torch.tensor(H, requires_grad=True)
    Et = torch.tensor(E, requires_grad=True)
    s = c * torch.tanh((Ht @ Et.T) / c)
    torch.nn.functional.cross_entropy(s, torch.tensor(y), reduction="sum").backward()
    dH, dE = ora.backward(H, E, y, c, 1.0)
    np.testing.assert_allclose(dH, Ht.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dE, Et.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_embed_grad_rows_matches_full_backward():
    rng = np.random.default_rng(25)
    H = rng.standard_normal((30, 8)) * 3.0
    E = rng.standard_normal((20, 8)) * 0.5
    y = rng.integers(0, 20, size=30)
    mask = (rng.random(30) < 0.6).astype(np.uint8)
    c, g = 6.0, 1.0 / mask.sum()
    _, dE = ora.backward(H, E, y, c, g, mask)
    _, lse = ora.forward(H, E, y, c)
    rows = np.array([0, 3, 19, 7])
    np.testing.assert_allclose(ora.embed_grad_rows(H, E, y, c, g, lse, rows, mask), dE[rows],
                               rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("caps", [(2.0, 5.0), (5.0, 0.0), (0.0, 3.0)])
def test_finite_differences_asymmetric_caps(caps):
    """Separate caps for z >= 0 and z < 0, with logits spanning both sides' curvature."""
    rng = np.random.default_rng(26)
    H = rng.standard_normal((6, 4)) * 3.0
    E = rng.standard_normal((9, 4)) * 1.0
    y = rng.integers(0, 9, size=6)
    mask = np.array([1, 0, 1, 1, 1, 0], dtype=np.uint8)
    g = 1.0 / mask.sum()
    z = H @ E.T
    assert np.max(z) > 4.0 and np.min(z) < -4.0
    dH, dE = ora.backward(H, E, y, caps, g, mask)
    fdH, fdE = _fd_grads(H, E, y, caps, g, mask)
    _check(dH, fdH, 1e-6)
    _check(dE, fdE, 1e-6)


def test_asymmetric_caps_match_torch_autograd():
    rng = np.random.default_rng(27)
    H = rng.standard_normal((13, 5)) * 6.0
    E = rng.standard_normal((10, 5)) * 1.0
    y = rng.integers(0, 10, size=13)
    cp, cn = 4.0, 9.0
    Ht = torch.tensor(H, requires_grad=True)
    Et = torch.tensor(E, requires_grad=True)
    z = Ht @ Et.T
    s = torch.where(z >= 0, cp * torch.tanh(z / cp), cn * torch.tanh(z / cn))
    torch.nn.functional.cross_entropy(s, torch.tensor(y), reduction="sum").backward()
    dH, dE = ora.backward(H, E, y, (cp, cn), 1.0)
    np.testing.assert_allclose(dH, Ht.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dE, Et.grad.numpy(), rtol=1e-11, atol=1e-13)


def test_out_of_range_target_poisons_gradients():
    """A scored row whose target lies outside [0, V) (above V or negative, which must not wrap
    around to the last entry) has NaN nats, so its dH row and all of dE are NaN; its other dH rows
    are those of the same call with that row unscored, and unscored it changes nothing."""
    inp = synth.make_inputs("fd", 3)
    H, E = synth.as_f64(inp["hidden"], "f32"), synth.as_f64(inp["embed"], "f32")
    y = inp["target"].astype(np.int64).copy()
    T, V = H.shape[0], E.shape[0]
    y[4], y[9] = V, -1
    dH, dE = ora.backward(H, E, y, 30.0, 1.0 / T)
    assert np.isnan(dH[[4, 9]]).all() and np.isnan(dE).all()
    keep = np.ones(T, np.uint8)
    keep[[4, 9]] = 0
    mH, mE = ora.backward(H, E, y, 30.0, 1.0 / T, keep)
    assert np.all(mH[[4, 9]] == 0.0) and np.all(np.isfinite(mE))
    rest = np.delete(np.arange(T), [4, 9])
    np.testing.assert_allclose(dH[rest], mH[rest], rtol=1e-12, atol=0)
    # unscored rows enter nothing: the same as dropping them
    sH, sE = ora.backward(H[rest], E, y[rest], 30.0, 1.0 / T)
    np.testing.assert_allclose(mH[rest], sH, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(mE, sE, rtol=1e-10, atol=1e-300)
    # the columns of dE are the forward's sensitivity: y = -1 must not act as y = V - 1
    y2 = y.copy()
    y2[9] = V - 1
    aH, _ = ora.backward(H, E, y2, 30.0, 1.0 / T, keep | (np.arange(T) == 9))
    assert np.all(np.isfinite(aH[9]))
