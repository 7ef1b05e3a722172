"""Pins of the oracle's bf16 storage model and of the composed training step:
bf16 rounding against hand-worked values and two independent implementations
(torch's float32->bfloat16 cast and the input quantiser), finite differences
on a tiny network in fp64, and torch float64 autograd on the whole network."""
import numpy as np
import pytest
import torch

import oracle
import synthdata

SLOPE = 0.3


def test_round_bf16_worked_values():
    r = oracle.round_bf16
    one = 1.0
    assert r([one + 2.0 ** -8])[0] == one                      # tie -> even (down)
    assert r([one + 3 * 2.0 ** -8])[0] == one + 2.0 ** -6      # tie -> even (up)
    assert r([one + 2.0 ** -8 + 2.0 ** -30])[0] == one + 2.0 ** -7
    assert r([-(one + 2.0 ** -8 + 2.0 ** -30)])[0] == -(one + 2.0 ** -7)
    assert r([2.0 ** -133])[0] == 2.0 ** -133                  # smallest subnormal
    assert r([2.0 ** -135])[0] == 0.0                          # rounds to zero
    assert r([3 * 2.0 ** -134])[0] == 2.0 ** -132              # tie between 1 and 2 quanta -> even
    assert r([0.1])[0] == 0.10009765625
    assert r([1e39])[0] == np.inf


def test_round_bf16_agrees_with_two_independent_roundings():
    x = np.random.default_rng(1).standard_normal(200000).astype(np.float32) * 7.0
    x[:1000] = np.float32(1.0) + np.arange(1000, dtype=np.float32) * np.float32(2.0 ** -12)
    a = oracle.round_bf16(x.astype(np.float64))
    b = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    c = synthdata.bf16_round_f32(x).astype(np.float64)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def tiny_problem(seed, storage="f64"):
    r = np.random.default_rng(seed)
    x = r.standard_normal((2, 8, 8, 8, 2))
    conv = [r.standard_normal((3, 3, 3, 2, 4)) * 0.3, r.standard_normal((3, 3, 3, 4, 8)) * 0.2]
    flat = 2 ** 3 * 8
    dense = [(r.standard_normal((flat, 32)) * 0.2, r.standard_normal(32) * 0.1),
             (r.standard_normal((32, 8)) * 0.2, r.standard_normal(8) * 0.1),
             (r.standard_normal((8, 3)) * 0.3, r.standard_normal(3) * 0.1)]
    t = r.uniform(-1, 1, (2, 3))
    return x, conv, dense, t


def loss_of(x, conv, dense, t):
    yhat, _ = oracle.network_forward(x, conv, dense, SLOPE)
    return oracle.mse(yhat, t)[0]


def kinks_are_far(x, conv, dense, margin=1e-4):
    """True when every pool max is separated from the runner-up and no
    pre-activation sits near zero (finite differences stay off the kinks)."""
    a = x
    for w in conv:
        z = oracle.conv3d_fwd(a, w)
        if np.min(np.abs(z)) < margin:
            return False
        N, D, H, W, C = z.shape
        win = z.reshape(N, D // 2, 2, H // 2, 2, W // 2, 2, C).transpose(0, 1, 3, 5, 7, 2, 4, 6).reshape(-1, 8)
        s = np.sort(win, axis=1)
        if np.min(s[:, -1] - s[:, -2]) < margin:
            return False
        a, _ = oracle.lrelu_maxpool_fwd(z, SLOPE)
    return True


def test_network_finite_differences():
    seed = 0
    while True:
        x, conv, dense, t = tiny_problem(seed)
        if kinks_are_far(x, conv, dense):
            break
        seed += 1
    yhat, cache = oracle.network_forward(x, conv, dense, SLOPE)
    loss, dy = oracle.mse(yhat, t)
    conv_g, dense_g = oracle.network_backward(cache, conv, dense, dy, SLOPE)
    r = np.random.default_rng(100)
    h = 1e-6
    for li, w in enumerate(conv):
        for _ in range(3):
            v = r.standard_normal(w.shape)
            cp = [c.copy() for c in conv]
            cm = [c.copy() for c in conv]
            cp[li] += h * v
            cm[li] -= h * v
            fd = (loss_of(x, cp, dense, t) - loss_of(x, cm, dense, t)) / (2 * h)
            an = np.vdot(conv_g[li], v)
            assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3), (li, fd, an)
    for li in range(3):
        for k in range(2):
            v = r.standard_normal(dense[li][k].shape)
            dp = [list(p) for p in dense]
            dm = [list(p) for p in dense]
            dp[li][k] = dense[li][k] + h * v
            dm[li][k] = dense[li][k] - h * v
            fd = (loss_of(x, conv, dp, t) - loss_of(x, conv, dm, t)) / (2 * h)
            an = np.vdot(dense_g[li][k], v)
            assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3), (li, k, fd, an)


def test_network_matches_torch_autograd_float64():
    x, conv, dense, t = tiny_problem(7)
    out = oracle.train_step(x, t, conv, dense, 1e-3, SLOPE, storage="f64")
    F = torch.nn.functional
    ws = [torch.from_numpy(w).requires_grad_() for w in conv]
    ds = [(torch.from_numpy(W).requires_grad_(), torch.from_numpy(b).requires_grad_()) for W, b in dense]
    a = torch.from_numpy(x).permute(0, 4, 1, 2, 3)
    for w in ws:
        a = F.max_pool3d(F.leaky_relu(F.conv3d(a, w.permute(4, 3, 0, 1, 2), padding=1), SLOPE), 2, 2)
    h = a.permute(0, 2, 3, 4, 1).reshape(2, -1)
    for i, (W, b) in enumerate(ds):
        h = h @ W + b
        if i < 2:
            h = F.leaky_relu(h, SLOPE)
    loss = ((h - torch.from_numpy(t)) ** 2).mean()
    loss.backward()
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-12)
    for w, g, nw in zip(ws, out["conv_dw"], out["conv_w"]):
        assert np.allclose(g, w.grad.numpy(), rtol=1e-10, atol=1e-12)
        assert np.allclose(nw, w.detach().numpy() - 1e-3 * w.grad.numpy(), rtol=1e-12, atol=1e-14)
    for (W, b), (gW, gb) in zip(ds, out["dense_g"]):
        assert np.allclose(gW, W.grad.numpy(), rtol=1e-10, atol=1e-12)
        assert np.allclose(gb, b.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_bf16_storage_model_rounds_at_storage_points():
    x, conv, dense, t = tiny_problem(3)
    xb = oracle.round_bf16(x)
    yhat, cache = oracle.network_forward(xb, [oracle.round_bf16(w) for w in conv], dense, SLOPE, "bf16")
    for blk in cache["blocks"]:
        assert np.array_equal(blk["p"], oracle.round_bf16(blk["p"]))
    # with bf16 storage the result stays close to the exact fp64 evaluation
    y64, _ = oracle.network_forward(xb, [oracle.round_bf16(w) for w in conv], dense, SLOPE, "f64")
    assert np.max(np.abs(yhat - y64)) / np.sqrt(np.mean(y64 ** 2)) < 5e-2
