"""Pins of the oracle's leaky-ReLU + max-pool, dense, MSE and SGD operators:
closed forms (monotone ramp, constant windows), the monotone invariant
pool(lrelu(z)) == lrelu(pool(z)), gradient conservation, and library special
cases (torch max_pool3d / leaky_relu / linear in float64 with autograd)."""
import numpy as np
import pytest
import torch

import oracle

SLOPE = 0.3


def test_ramp_closed_form():
    N, D, H, W, C = 1, 4, 6, 2, 3
    z = np.arange(N * D * H * W * C, dtype=np.float64).reshape(N, D, H, W, C) - 40.0
    p, idx = oracle.lrelu_maxpool_fwd(z, SLOPE)
    assert np.all(idx == 7)   # the (1,1,1) corner of every window is largest
    top = z[:, 1::2, 1::2, 1::2, :]
    assert np.array_equal(p, np.where(top > 0, top, SLOPE * top))


def test_constant_windows_pick_first():
    z = np.full((2, 2, 4, 2, 5), -1.5)
    p, idx = oracle.lrelu_maxpool_fwd(z, SLOPE)
    assert np.all(idx == 0) and np.all(p == SLOPE * -1.5)


def test_pool_of_lrelu_equals_lrelu_of_pool():
    z = np.random.default_rng(1).standard_normal((2, 6, 4, 8, 3))
    p, _ = oracle.lrelu_maxpool_fwd(z, SLOPE)
    q, _ = oracle.lrelu_maxpool_fwd(z, 1.0)   # slope 1: plain max pool
    assert np.array_equal(p, oracle.lrelu_fwd(q, SLOPE))


def test_matches_torch_maxpool_float64():
    z = np.random.default_rng(2).standard_normal((2, 6, 4, 8, 5))  # tie-free
    p, idx = oracle.lrelu_maxpool_fwd(z, SLOPE)
    zt = torch.from_numpy(z).permute(0, 4, 1, 2, 3)
    pt, it = torch.nn.functional.max_pool3d(torch.nn.functional.leaky_relu(zt, SLOPE), 2, 2, return_indices=True)
    assert np.array_equal(p, pt.permute(0, 2, 3, 4, 1).numpy())
    # torch index is the flat d*H*W + h*W + w inside the (D,H,W) volume
    it = it.permute(0, 2, 3, 4, 1).numpy()
    N, D, H, W, C = z.shape
    d, rem = np.divmod(it, H * W)
    h, w = np.divmod(rem, W)
    Dp, Hp, Wp = D // 2, H // 2, W // 2
    gi = np.arange(Dp)[None, :, None, None, None]
    gj = np.arange(Hp)[None, None, :, None, None]
    gk = np.arange(Wp)[None, None, None, :, None]
    assert np.array_equal(idx, ((d - 2 * gi) * 4 + (h - 2 * gj) * 2 + (w - 2 * gk)).astype(np.uint8))


def test_backward_matches_torch_autograd_and_conserves():
    r = np.random.default_rng(3)
    z = r.standard_normal((2, 4, 6, 4, 3))
    dp = r.standard_normal((2, 2, 3, 2, 3))
    p, idx = oracle.lrelu_maxpool_fwd(z, SLOPE)
    dz = oracle.maxpool_lrelu_bwd(dp, p, idx, SLOPE)
    zt = torch.from_numpy(z).permute(0, 4, 1, 2, 3).requires_grad_()
    out = torch.nn.functional.max_pool3d(torch.nn.functional.leaky_relu(zt, SLOPE), 2, 2)
    out.backward(torch.from_numpy(dp).permute(0, 4, 1, 2, 3))
    assert np.allclose(dz, zt.grad.permute(0, 2, 3, 4, 1).numpy(), rtol=0, atol=1e-15)
    # one non-zero per window; total equals sum of dp * lrelu'(p)
    assert np.count_nonzero(dz) == dp.size
    assert np.isclose(dz.sum(), np.sum(np.where(p > 0, dp, SLOPE * dp)), rtol=1e-13)


def test_lrelu_pins():
    x = np.array([-2.0, -0.0, 0.0, 1e-300, 3.5])
    assert np.array_equal(oracle.lrelu_fwd(x, SLOPE), [-0.6, -0.0, 0.0, 1e-300, 3.5])
    assert np.array_equal(oracle.lrelu_bwd(x, np.ones(5), SLOPE), [SLOPE, SLOPE, SLOPE, 1.0, 1.0])


@pytest.mark.parametrize("slope", [SLOPE, -1.0])
def test_dense_matches_torch(slope):
    r = np.random.default_rng(4)
    B, In, Out = 3, 17, 5
    x = r.standard_normal((B, In))
    w = r.standard_normal((In, Out))
    b = r.standard_normal(Out)
    dy = r.standard_normal((B, Out))
    pre, y = oracle.dense_fwd(x, w, b, slope)
    assert np.allclose(pre, x @ w + b, rtol=1e-13, atol=1e-13)
    xt = torch.from_numpy(x).requires_grad_()
    wt = torch.from_numpy(w).requires_grad_()
    bt = torch.from_numpy(b).requires_grad_()
    pt = xt @ wt + bt
    yt = torch.nn.functional.leaky_relu(pt, slope) if slope >= 0 else pt
    assert np.allclose(y, yt.detach().numpy(), rtol=1e-13, atol=1e-13)
    yt.backward(torch.from_numpy(dy))
    dx, dw, db = oracle.dense_bwd(x, w, pre, dy, slope)
    assert np.allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(db, bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_mse_closed_form():
    yhat = np.array([[1.0, 2.0, 3.0], [0.0, -1.0, 0.5]])
    t = np.array([[0.0, 2.0, 1.0], [1.0, 1.0, 0.5]])
    loss, d = oracle.mse(yhat, t)
    assert loss == pytest.approx((1 + 0 + 4 + 1 + 4 + 0) / 6.0, rel=1e-15)
    assert np.allclose(d, 2 * (yhat - t) / 6.0, rtol=1e-15)


def test_sgd_closed_form():
    w = np.array([1.0, -2.0, 0.5])
    dw = np.array([10.0, 0.0, -4.0])
    assert np.allclose(oracle.sgd(w, dw, 1e-3), [0.99, -2.0, 0.504], rtol=1e-15)
