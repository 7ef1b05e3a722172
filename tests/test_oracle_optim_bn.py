"""Pins of the oracle's optimizer (Adam + LARC + polynomial decay) and batch
normalisation against facts outside the oracle: hand-worked values, closed
forms, invariants, and torch's float64 Adam / batch_norm as library special
cases."""
import numpy as np
import pytest
import torch

import oracle


# ------------------------------------------------------------ decay schedule
def test_poly_decay_closed_forms():
    d = oracle.poly_decay
    assert d(1e-3, 1e-5, 100, 1.0, 0) == 1e-3
    assert d(1e-3, 1e-5, 100, 1.0, 50) == pytest.approx((1e-3 + 1e-5) / 2, rel=1e-15)
    assert d(1e-3, 1e-5, 100, 1.0, 100) == pytest.approx(1e-5, rel=1e-15)
    assert d(1e-3, 1e-5, 100, 1.0, 1000) == pytest.approx(1e-5, rel=1e-15)     # held after T
    # power 2 at half way: a quarter of the span above the end rate
    assert d(1.0, 0.0, 10, 2.0, 5) == pytest.approx(0.25, rel=1e-15)
    # linear decay to 0.01x of the initial rate (Oyama et al.): 1% at T
    assert d(0.02, 0.0002, 400, 1.0, 400) == pytest.approx(0.0002, rel=1e-12)


# ------------------------------------------------------------------ Adam
def test_first_adam_step_is_a_sign_step():
    # After one update the bias-corrected moments are g and g^2, so the
    # direction is g / (|g| + eps): almost exactly sign(g).
    r = np.random.default_rng(0)
    w, g = r.standard_normal(100), r.standard_normal(100)
    z = np.zeros(100)
    w1, m, v, lr_l = oracle.adam_larc_step(w, g, z, z, 1, 0.1, 0.9, 0.999, 1e-8, 0.0)
    assert lr_l == 0.1
    assert np.allclose(w1, w - 0.1 * g / (np.abs(g) + 1e-8), rtol=0, atol=1e-15)
    assert np.allclose(m, 0.1 * g, rtol=1e-15) and np.allclose(v, 0.001 * g * g, rtol=1e-12)


def test_adam_constant_gradient_recurrence():
    # With a constant gradient c the bias-corrected moments stay c and c^2 at
    # every step, so every update moves w by lr * c / (|c| + eps).
    w, m, v = np.array([1.0]), np.zeros(1), np.zeros(1)
    c = np.array([-0.25])
    for t in range(1, 8):
        w_new, m, v, _ = oracle.adam_larc_step(w, c, m, v, t, 0.01, 0.9, 0.999, 1e-8, 0.0)
        assert w_new[0] - w[0] == pytest.approx(0.01 * 0.25 / (0.25 + 1e-8), rel=1e-12)
        assert m[0] == pytest.approx(c[0] * (1 - 0.9 ** t), rel=1e-12)
        w = w_new


def test_adam_matches_torch_float64_without_larc():
    r = np.random.default_rng(3)
    w0 = r.standard_normal((7, 5))
    grads = [r.standard_normal((7, 5)) for _ in range(6)]
    p = torch.from_numpy(w0.copy()).requires_grad_()
    opt = torch.optim.Adam([p], lr=3e-3, betas=(0.9, 0.999), eps=1e-8)
    w, m, v = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
    for t, g in enumerate(grads, 1):
        p.grad = torch.from_numpy(g.copy())
        opt.step()
        w, m, v, _ = oracle.adam_larc_step(w, g, m, v, t, 3e-3, 0.9, 0.999, 1e-8, 0.0)
        assert np.allclose(w, p.detach().numpy(), rtol=1e-13, atol=1e-15)


# ------------------------------------------------------------------- LARC
def test_larc_clips_the_rate_at_the_layer_trust_ratio():
    # ||w|| = 5, ||g|| = 10: trust 0.1 gives 0.1 * 5 / 10 = 0.05, below the
    # nominal 0.1, so the layer moves at 0.05; first-step direction g/(|g|+eps).
    w, g, z = np.array([3.0, 4.0]), np.array([0.0, 10.0]), np.zeros(2)
    w1, _, _, lr_l = oracle.adam_larc_step(w, g, z, z, 1, 0.1, 0.9, 0.999, 1e-8, 0.1)
    assert lr_l == pytest.approx(0.05, rel=1e-15)
    assert w1[0] == 3.0 and w1[1] == pytest.approx(4.0 - 0.05 * 10.0 / (10.0 + 1e-8), rel=1e-15)
    # nominal rate below the trust ratio: LARC leaves it alone
    _, _, _, lr_l = oracle.adam_larc_step(w, g, z, z, 1, 0.01, 0.9, 0.999, 1e-8, 0.1)
    assert lr_l == 0.01
    # zero weights or zero gradient: no layer-wise scaling
    _, _, _, lr_l = oracle.adam_larc_step(np.zeros(2), g, z, z, 1, 0.1, 0.9, 0.999, 1e-8, 0.1)
    assert lr_l == 0.1
    _, _, _, lr_l = oracle.adam_larc_step(w, np.zeros(2), z, z, 1, 0.1, 0.9, 0.999, 1e-8, 0.1)
    assert lr_l == 0.1


def test_larc_rate_is_invariant_to_scaling_the_gradient_direction_only():
    # Scaling the weights by s scales the trust ratio by s; scaling the
    # gradient by s divides it by s (the ratio uses the norms only).
    r = np.random.default_rng(4)
    w, g, z = r.standard_normal(50), r.standard_normal(50), np.zeros(50)
    base = oracle.adam_larc_step(w, g, z, z, 1, 10.0, 0.9, 0.999, 1e-8, 0.01)[3]
    assert oracle.adam_larc_step(3 * w, g, z, z, 1, 10.0, 0.9, 0.999, 1e-8, 0.01)[3] == pytest.approx(3 * base)
    assert oracle.adam_larc_step(w, 4 * g, z, z, 1, 10.0, 0.9, 0.999, 1e-8, 0.01)[3] == pytest.approx(base / 4)


# ------------------------------------------------------------- batch norm
def test_batchnorm_matches_torch_float64():
    r = np.random.default_rng(5)
    x = r.standard_normal((2, 3, 4, 5, 6)) * 2.0 + 0.7
    gamma, beta = r.standard_normal(6), r.standard_normal(6)
    dy = r.standard_normal(x.shape)
    y, mean, invstd = oracle.batchnorm_fwd(x, gamma, beta, 1e-5)
    dx, dgamma, dbeta = oracle.batchnorm_bwd(x, dy, gamma, mean, invstd)
    xt = torch.from_numpy(x).permute(0, 4, 1, 2, 3).contiguous().requires_grad_()
    gt, bt = torch.from_numpy(gamma).requires_grad_(), torch.from_numpy(beta).requires_grad_()
    yt = torch.nn.functional.batch_norm(xt, None, None, gt, bt, training=True, eps=1e-5)
    yt.backward(torch.from_numpy(dy).permute(0, 4, 1, 2, 3))
    assert np.allclose(y, yt.detach().permute(0, 2, 3, 4, 1).numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dx, xt.grad.permute(0, 2, 3, 4, 1).numpy(), rtol=1e-11, atol=1e-12)
    assert np.allclose(dgamma, gt.grad.numpy(), rtol=1e-12) and np.allclose(dbeta, bt.grad.numpy(), rtol=1e-12)


def test_batchnorm_invariants():
    # eps = 0: every channel of xhat has mean 0 and mean square 1; the input
    # gradient sums to zero and is orthogonal to xhat per channel.
    r = np.random.default_rng(6)
    x = r.standard_normal((3, 2, 2, 2, 4)) * 3.0 - 1.0
    y, mean, invstd = oracle.batchnorm_fwd(x, np.ones(4), np.zeros(4), 0.0)
    f = y.reshape(-1, 4)
    assert np.allclose(f.mean(axis=0), 0, atol=1e-14) and np.allclose((f * f).mean(axis=0), 1, rtol=1e-13)
    dy = r.standard_normal(x.shape)
    dx, _, _ = oracle.batchnorm_bwd(x, dy, np.full(4, 2.0), mean, invstd)
    fd = dx.reshape(-1, 4)
    assert np.allclose(fd.sum(axis=0), 0, atol=1e-12)
    assert np.allclose((fd * f).sum(axis=0), 0, atol=1e-12)
    # a constant channel: xhat = 0, y = beta
    xc = np.full((1, 2, 2, 2, 1), 5.0)
    yc, mc, _ = oracle.batchnorm_fwd(xc, [2.0], [0.5], 1e-5)
    assert mc[0] == 5.0 and np.all(yc == 0.5)
