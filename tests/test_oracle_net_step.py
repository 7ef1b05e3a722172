"""Pins of the oracle's general network step (strided "same" convs,
batch norm, max / average / no pooling, dense layers without bias) against
torch float64 autograd on the same network, a library special case, and of
the SGD and Adam updates it applies."""
import numpy as np
import pytest
import torch

import oracle

F = torch.nn.functional
SLOPE = 0.3


def torch_same(a, w, stride):
    D = a.shape[2]
    out = -(-D // stride)
    total = max((out - 1) * stride + 3 - D, 0)
    lo, hi = total // 2, total - total // 2
    return F.conv3d(F.pad(a, (lo, hi, lo, hi, lo, hi)), w.permute(4, 3, 0, 1, 2), stride=stride)


def tiny(batch_norm, dense_bias, seed):
    r = np.random.default_rng(seed)
    # stride-2 layer, average pool, max pool, and a layer with no pool
    layers = [(4, 1, "avg"), (8, 2, "max"), (8, 1, "none")]
    dense = [16, 3]
    shapes = oracle.net_param_shapes(2, layers, dense, batch_norm, dense_bias, 16)
    params = []
    for sh in shapes:
        if len(sh) == 1:
            params.append(r.uniform(0.5, 1.5, sh) if len(params) % 3 == 1 and batch_norm else r.standard_normal(sh) * 0.1)
        else:
            params.append(r.standard_normal(sh) * (0.4 if len(sh) == 5 else 0.3))
    x = r.standard_normal((2, 16, 16, 16, 2))
    t = r.uniform(-1, 1, (2, 3))
    return x, t, layers, dense, params


@pytest.mark.parametrize("batch_norm,dense_bias", [(False, True), (True, False)])
def test_net_step_matches_torch_autograd_float64(batch_norm, dense_bias):
    x, t, layers, dense, params = tiny(batch_norm, dense_bias, 3 + batch_norm)
    out = oracle.net_train_step(x, t, params, layers, dense, SLOPE, batch_norm=batch_norm, dense_bias=dense_bias,
                                storage="f64", opt=("sgd", 1e-2))
    tp = [torch.from_numpy(p.copy()).requires_grad_() for p in params]
    per = 3 if batch_norm else 1
    a = torch.from_numpy(x).permute(0, 4, 1, 2, 3)
    for l, (f, s, pool) in enumerate(layers):
        a = torch_same(a, tp[l * per], s)
        if batch_norm:
            a = F.batch_norm(a, None, None, tp[l * per + 1], tp[l * per + 2], training=True, eps=1e-5)
        a = F.leaky_relu(a, SLOPE)
        if pool == "max":
            a = F.max_pool3d(a, 2, 2)
        elif pool == "avg":
            a = F.avg_pool3d(a, 2, 2)
    h = a.permute(0, 2, 3, 4, 1).reshape(2, -1)
    i = len(layers) * per
    for k in range(len(dense)):
        h = h @ tp[i]
        i += 1
        if dense_bias:
            h = h + tp[i]
            i += 1
        if k + 1 < len(dense):
            h = F.leaky_relu(h, SLOPE)
    loss = ((h - torch.from_numpy(t)) ** 2).mean()
    loss.backward()
    assert out["loss"] == pytest.approx(loss.item(), rel=1e-12)
    for g, p, nw in zip(out["grads"], tp, out["params"]):
        assert np.allclose(g, p.grad.numpy(), rtol=1e-9, atol=1e-12)
        assert np.allclose(nw, p.detach().numpy() - 1e-2 * p.grad.numpy(), rtol=1e-12, atol=1e-14)


def test_net_step_adam_update_is_the_per_tensor_adam_larc_step():
    x, t, layers, dense, params = tiny(False, True, 9)
    z = [np.zeros_like(p) for p in params]
    out = oracle.net_train_step(x, t, params, layers, dense, SLOPE, storage="f64",
                                opt=("adam", 0.01, 0.9, 0.999, 1e-8, 0.02, 1), adam_state=(z, z))
    for p, g, nw in zip(params, out["grads"], out["params"]):
        w1, _, _, _ = oracle.adam_larc_step(p, g, np.zeros_like(p), np.zeros_like(p), 1, 0.01, 0.9, 0.999, 1e-8, 0.02)
        assert np.array_equal(nw, w1)
