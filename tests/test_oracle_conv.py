"""Pins of the oracle's 3D convolution operators to facts fixed independently
of its own code: delta-kernel and delta-input identities (which fix the
cross-correlation orientation and the zero padding), the all-ones closed form,
linearity, the adjoint identities linking forward, backward-data and
backward-weight, and the library special case torch.nn.functional.conv3d in
float64 (NDHWC/DHWIO permuted to NCDHW/OIDHW)."""
import numpy as np
import pytest
import torch

import oracle


def rng(seed):
    return np.random.default_rng(seed)


def shift_fill(x, sd, sh, sw):
    """y[d,h,w] = x[d+sd, h+sh, w+sw], zero outside; built with numpy padding
    and slicing (independent of the oracle loops)."""
    N, D, H, W, C = x.shape
    xp = np.pad(x, ((0, 0), (1, 1), (1, 1), (1, 1), (0, 0)))
    return xp[:, 1 + sd:1 + sd + D, 1 + sh:1 + sh + H, 1 + sw:1 + sw + W, :]


def test_center_delta_kernel_is_identity():
    x = rng(1).standard_normal((2, 5, 4, 6, 3))
    w = np.zeros((3, 3, 3, 3, 3))
    for c in range(3):
        w[1, 1, 1, c, c] = 1.0
    assert np.array_equal(oracle.conv3d_fwd(x, w), x)


@pytest.mark.parametrize("tap", [(0, 0, 0), (2, 1, 0), (1, 2, 2), (0, 2, 1), (2, 2, 2)])
def test_shifted_delta_kernel(tap):
    kd, kh, kw = tap
    x = rng(2).standard_normal((1, 4, 5, 3, 2))
    w = np.zeros((3, 3, 3, 2, 2))
    w[kd, kh, kw, 0, 1] = 1.0   # channel 0 -> output channel 1
    y = oracle.conv3d_fwd(x, w)
    exp = shift_fill(x, kd - 1, kh - 1, kw - 1)
    assert np.array_equal(y[..., 1], exp[..., 0])
    assert np.array_equal(y[..., 0], np.zeros_like(y[..., 0]))


def test_delta_input_reproduces_kernel():
    D = H = W = 7
    w = rng(3).standard_normal((3, 3, 3, 2, 4))
    x = np.zeros((1, D, H, W, 2))
    p = (3, 2, 4)
    x[0, p[0], p[1], p[2], 1] = 1.0
    y = oracle.conv3d_fwd(x, w)
    for kd in range(3):
        for kh in range(3):
            for kw in range(3):
                o = (p[0] - kd + 1, p[1] - kh + 1, p[2] - kw + 1)
                assert np.array_equal(y[0, o[0], o[1], o[2]], w[kd, kh, kw, 1])
    assert np.count_nonzero(np.abs(y).sum(-1)) == 27


def test_all_ones_closed_form():
    D, H, W, Ci, Co = 5, 2, 4, 3, 2
    y = oracle.conv3d_fwd(np.ones((1, D, H, W, Ci)), np.ones((3, 3, 3, Ci, Co)))

    def cnt(i, n):  # in-range taps along one axis
        return 1 + (i > 0) + (i < n - 1)
    for d in range(D):
        for h in range(H):
            for w in range(W):
                assert np.all(y[0, d, h, w] == Ci * cnt(d, D) * cnt(h, H) * cnt(w, W))
    # interior 27*Ci, face 18*Ci, edge 12*Ci, corner 8*Ci on a 5^3 cube
    y5 = oracle.conv3d_fwd(np.ones((1, 5, 5, 5, 1)), np.ones((3, 3, 3, 1, 1)))[0, ..., 0]
    assert y5[2, 2, 2] == 27 and y5[0, 2, 2] == 18 and y5[0, 0, 2] == 12 and y5[0, 0, 0] == 8


def test_linearity():
    r = rng(4)
    x1, x2 = r.standard_normal((2, 2, 3, 4, 5, 3))
    w1, w2 = r.standard_normal((2, 3, 3, 3, 3, 4))
    a, b = 0.75, -1.25
    lhs = oracle.conv3d_fwd(a * x1 + b * x2, w1)
    rhs = a * oracle.conv3d_fwd(x1, w1) + b * oracle.conv3d_fwd(x2, w1)
    assert np.allclose(lhs, rhs, rtol=1e-13, atol=1e-13)
    lhs = oracle.conv3d_fwd(x1, a * w1 + b * w2)
    rhs = a * oracle.conv3d_fwd(x1, w1) + b * oracle.conv3d_fwd(x1, w2)
    assert np.allclose(lhs, rhs, rtol=1e-13, atol=1e-13)


def torch_conv(x, w):
    xt = torch.from_numpy(x).permute(0, 4, 1, 2, 3)           # NCDHW
    wt = torch.from_numpy(w).permute(4, 3, 0, 1, 2)           # OIDHW
    return torch.nn.functional.conv3d(xt, wt, padding=1).permute(0, 2, 3, 4, 1).numpy()


@pytest.mark.parametrize("shape", [(1, 3, 3, 3, 1, 1), (2, 4, 3, 5, 3, 5), (1, 6, 7, 5, 8, 4)])
def test_matches_torch_conv3d_float64(shape):
    N, D, H, W, Ci, Co = shape
    r = rng(5)
    x = r.standard_normal((N, D, H, W, Ci))
    w = r.standard_normal((3, 3, 3, Ci, Co))
    assert np.allclose(oracle.conv3d_fwd(x, w), torch_conv(x, w), rtol=1e-12, atol=1e-12)


def test_backward_matches_torch_autograd_float64():
    r = rng(6)
    N, D, H, W, Ci, Co = 2, 5, 4, 6, 3, 4
    x = r.standard_normal((N, D, H, W, Ci))
    w = r.standard_normal((3, 3, 3, Ci, Co))
    dy = r.standard_normal((N, D, H, W, Co))
    xt = torch.from_numpy(x).requires_grad_()
    wt = torch.from_numpy(w).requires_grad_()
    y = torch.nn.functional.conv3d(xt.permute(0, 4, 1, 2, 3), wt.permute(4, 3, 0, 1, 2), padding=1)
    y.permute(0, 2, 3, 4, 1).backward(torch.from_numpy(dy))
    assert np.allclose(oracle.conv3d_bwd_data(dy, w), xt.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(oracle.conv3d_bwd_weight(x, dy), wt.grad.numpy(), rtol=1e-12, atol=1e-11)


@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1, 1), (2, 3, 5, 4, 3, 2), (1, 7, 2, 9, 4, 6)])
def test_adjoint_identities(shape):
    N, D, H, W, Ci, Co = shape
    r = rng(7)
    x = r.standard_normal((N, D, H, W, Ci))
    w = r.standard_normal((3, 3, 3, Ci, Co))
    dy = r.standard_normal((N, D, H, W, Co))
    a = np.vdot(oracle.conv3d_fwd(x, w), dy)
    b = np.vdot(x, oracle.conv3d_bwd_data(dy, w))
    c = np.vdot(w, oracle.conv3d_bwd_weight(x, dy))
    s = max(abs(a), 1.0)
    assert abs(a - b) / s < 1e-12 and abs(a - c) / s < 1e-12


def test_point_variants_equal_full_operators():
    r = rng(8)
    N, D, H, W, Ci, Co = 2, 5, 6, 7, 4, 3
    # float32-representable inputs so both variants see identical values
    x = r.standard_normal((N, D, H, W, Ci)).astype(np.float32)
    w = r.standard_normal((3, 3, 3, Ci, Co)).astype(np.float32)
    dy = r.standard_normal((N, D, H, W, Co)).astype(np.float32)
    y = oracle.conv3d_fwd(x, w).ravel()
    p = r.choice(y.size, 50, replace=False)
    assert np.array_equal(oracle.conv3d_fwd_points(x, w, p), y[p])
    dx = oracle.conv3d_bwd_data(dy, w).ravel()
    p = r.choice(dx.size, 50, replace=False)
    assert np.array_equal(oracle.conv3d_bwd_data_points(dy, w, p), dx[p])
    dw = oracle.conv3d_bwd_weight(x, dy).ravel()
    p = r.choice(dw.size, 30, replace=False)
    assert np.allclose(oracle.conv3d_bwd_weight_points(x, dy, p), dw[p], rtol=1e-13, atol=1e-12)


def test_bwd_weight_single_voxel_closed_form():
    # one voxel, stride-1 pad-1: only the centre tap sees in-range input
    x = np.array([2.0, -3.0]).reshape(1, 1, 1, 1, 2)
    dy = np.array([5.0, 7.0, 11.0]).reshape(1, 1, 1, 1, 3)
    dw = oracle.conv3d_bwd_weight(x, dy)
    exp = np.zeros((3, 3, 3, 2, 3))
    exp[1, 1, 1] = np.outer([2.0, -3.0], [5.0, 7.0, 11.0])
    assert np.array_equal(dw, exp)
