"""Pins of the oracle's read epilogue, y = sigmoid(g) * RMSNorm(o) with a
head-wise RMSNorm over the d_v channels of one (token, head) and a gain
vector (paper §3.4 "Read-out", last sentence; Fig. 2), against things other
than itself:

* closed forms: a constant row normalises to its sign; a zero row gives 0;
* torch's own rms_norm and sigmoid (float64, CPU) for the forward, and torch
  autograd through them for every gradient;
* central finite differences of the oracle's forward for its backward;
* invariants: with eps = 0 the output is invariant to a positive scale of o,
  odd in o, and the gradient of o is orthogonal to o in every row.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rows(rng, R, d, scale=1.0):
    return rng.standard_normal((R, d)) * scale


@pytest.mark.parametrize("d", [1, 7, 64, 128])
def test_constant_rows_normalise_to_their_sign(d):
    rng = np.random.default_rng(d)
    c = np.array([3.5, -0.25, 1e-3, -70.0])
    o = np.repeat(c[:, None], d, axis=1)
    g = rows(rng, 4, d)
    gain = rng.standard_normal(d)
    y = oracle.epilogue_forward(o, g, gain, eps=0.0)
    ref = (1.0 / (1.0 + np.exp(-g))) * np.sign(c)[:, None] * gain[None, :]
    np.testing.assert_allclose(y, ref, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("d,eps,with_gain", [(16, 1e-6, True), (128, 1e-5, False),
                                             (33, 0.0, True), (64, 0.5, True)])
def test_forward_matches_torch_rms_norm(d, eps, with_gain):
    rng = np.random.default_rng(10 + d)
    o, g = rows(rng, 50, d, 2.0), rows(rng, 50, d)
    gain = rng.standard_normal(d) if with_gain else None
    y = oracle.epilogue_forward(o, g, gain, eps=eps)
    to, tg = torch.from_numpy(o), torch.from_numpy(g)
    tw = torch.from_numpy(gain) if with_gain else None
    ref = torch.sigmoid(tg) * F.rms_norm(to, (d,), tw, eps)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("d,eps,with_gain", [(16, 1e-6, True), (128, 1e-5, False),
                                             (5, 0.0, True), (64, 0.5, True)])
def test_backward_matches_torch_autograd(d, eps, with_gain):
    rng = np.random.default_rng(20 + d)
    R = 40
    o, g, dy = rows(rng, R, d, 1.5), rows(rng, R, d), rows(rng, R, d)
    gain = rng.standard_normal(d) if with_gain else None
    d_o, d_g, d_gain = oracle.epilogue_backward(o, g, dy, gain, eps=eps)
    to = torch.tensor(o, requires_grad=True)
    tg = torch.tensor(g, requires_grad=True)
    tw = torch.tensor(gain if with_gain else np.ones(d), requires_grad=True)
    y = torch.sigmoid(tg) * F.rms_norm(to, (d,), tw, eps)
    y.backward(torch.from_numpy(dy))
    np.testing.assert_allclose(d_o, to.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(d_g, tg.grad.numpy(), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(d_gain, tw.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_backward_matches_finite_differences():
    rng = np.random.default_rng(3)
    R, d, eps = 3, 12, 1e-3
    o, g, dy = rows(rng, R, d), rows(rng, R, d), rows(rng, R, d)
    gain = rng.standard_normal(d)
    d_o, d_g, d_gain = oracle.epilogue_backward(o, g, dy, gain, eps=eps)

    def loss(o_, g_, w_):
        return float(np.sum(oracle.epilogue_forward(o_, g_, w_, eps=eps) * dy))

    h = 1e-6
    for (r, c) in [(0, 0), (1, 5), (2, 11)]:
        for arr, grad in ((o, d_o), (g, d_g)):
            plus, minus = arr.copy(), arr.copy()
            plus[r, c] += h
            minus[r, c] -= h
            args_p = (plus, g, gain) if arr is o else (o, plus, gain)
            args_m = (minus, g, gain) if arr is o else (o, minus, gain)
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[r, c]) <= 1e-7 * max(1.0, abs(fd))
    for c in (0, 7):
        wp, wm = gain.copy(), gain.copy()
        wp[c] += h
        wm[c] -= h
        fd = (loss(o, g, wp) - loss(o, g, wm)) / (2 * h)
        assert abs(fd - d_gain[c]) <= 1e-7 * max(1.0, abs(fd))


def test_scale_invariance_and_orthogonal_gradient():
    # eps = 0: y(alpha o) = y(o) for alpha > 0 and y(-o) = -y(o), so the
    # derivative along o vanishes: sum_c d_o[c] o[c] = 0 in every row
    rng = np.random.default_rng(4)
    R, d = 20, 48
    o, g, dy = rows(rng, R, d), rows(rng, R, d), rows(rng, R, d)
    gain = rng.standard_normal(d)
    y = oracle.epilogue_forward(o, g, gain, eps=0.0)
    np.testing.assert_allclose(oracle.epilogue_forward(7.25 * o, g, gain, eps=0.0), y, rtol=1e-13)
    np.testing.assert_allclose(oracle.epilogue_forward(-o, g, gain, eps=0.0), -y, rtol=1e-13)
    d_o, _, _ = oracle.epilogue_backward(o, g, dy, gain, eps=0.0)
    radial = np.sum(d_o * o, axis=1)
    assert np.max(np.abs(radial)) <= 1e-12 * np.max(np.abs(d_o)) * np.max(np.abs(o)) * d


def test_zero_row():
    # a masked token's read output is 0: y = 0, no gate or gain gradient, and
    # d_o = dz * gain / sqrt(eps)
    rng = np.random.default_rng(5)
    d, eps = 10, 1e-4
    o = np.zeros((1, d))
    g, dy = rows(rng, 1, d), rows(rng, 1, d)
    gain = rng.standard_normal(d)
    y = oracle.epilogue_forward(o, g, gain, eps=eps)
    assert np.all(y == 0.0)
    d_o, d_g, d_gain = oracle.epilogue_backward(o, g, dy, gain, eps=eps)
    assert np.all(d_g == 0.0) and np.all(d_gain == 0.0)
    s = 1.0 / (1.0 + np.exp(-g))
    np.testing.assert_allclose(d_o, dy * s * gain / np.sqrt(eps), rtol=1e-13)
