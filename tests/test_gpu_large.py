"""Parity at the 512^3 configurations (4 and 5).  The first block's conv
output has exactly 2^32 elements, so these cases exercise 64-bit addressing
in every kernel.  Inputs are drawn on the device by the seeded generators;
the oracle computes sampled outputs one by one from host copies of the same
inputs (pool slabs, conv output points, individual weight-gradient sums)."""
import numpy as np
import pytest
import torch

import oracle
import synthdata as sd
from cnn_cosmology_volumes_amd import cf
from cnn_cosmology_volumes_amd.configs import CONFIGS
from gpu_util import TOL_BF16, bf16_elementwise_ok, host64, rel_err, sample_points

pytestmark = pytest.mark.gpu
BF, F32 = torch.bfloat16, torch.float32
SLOPE = 0.3
DEV = "cuda"


def h32(t):
    return t.float().cpu().numpy()


def conv_weights(seed, cin, cout):
    w = sd.bf16_round_f32(sd.he_normal_conv(np.random.default_rng(seed), cin, cout))
    return w, torch.from_numpy(w).to(DEV).to(BF)


def fwd_points(x_dev, w32, y_dev, rng, n):
    pts = sample_points(rng, tuple(y_dev.shape), n)
    o = oracle.conv3d_fwd_points(h32(x_dev), w32, pts)
    g = host64(y_dev.reshape(-1)[torch.from_numpy(pts).to(DEV)])
    assert rel_err(g, o) <= TOL_BF16
    assert bf16_elementwise_ok(g, o) == 0


def dgrad_points(dz_dev, w32, dx_dev, rng, n):
    pts = sample_points(rng, tuple(dx_dev.shape), n)
    o = oracle.conv3d_bwd_data_points(h32(dz_dev), w32, pts)
    g = host64(dx_dev.reshape(-1)[torch.from_numpy(pts).to(DEV)])
    assert rel_err(g, o) <= TOL_BF16
    assert bf16_elementwise_ok(g, o) == 0


def wgrad_points(x_dev, dz_dev, dw_dev, rng, n):
    ci, co = x_dev.shape[4], dz_dev.shape[4]
    pts = set(int(p) for p in rng.integers(0, 27 * ci * co, n))
    pts.add(0)
    pts.add(27 * ci * co - 1)
    pts = np.array(sorted(pts), np.int64)
    o = oracle.conv3d_bwd_weight_points(h32(x_dev), h32(dz_dev), pts)
    g = host64(dw_dev.reshape(-1)[torch.from_numpy(pts).to(DEV)])
    assert np.max(np.abs(g - o)) <= 1e-3 * max(np.max(np.abs(o)), 1e-30)


def pool_slabs(z_dev, p_dev, idx_dev, dp_dev, dz_dev, rng, nslab=2):
    D = z_dev.shape[1]
    planes = [0, D // 2 - 1] + [int(rng.integers(0, D // 2)) for _ in range(nslab)]
    for a in planes:
        zs = h32(z_dev[:, 2 * a:2 * a + 2])
        po, io = oracle.lrelu_maxpool_fwd(zs, SLOPE)
        assert np.array_equal(idx_dev[:, a:a + 1].cpu().numpy(), io)
        assert np.all(np.abs(host64(p_dev[:, a:a + 1]) - po) <= 2.0 ** -8 * np.abs(po))
        dzo = oracle.maxpool_lrelu_bwd(h32(dp_dev[:, a:a + 1]), po, io, SLOPE)
        gz = host64(dz_dev[:, 2 * a:2 * a + 2])
        assert np.all(np.abs(gz - dzo) <= 2.0 ** -8 * np.abs(dzo))


def test_partial512_block1_full():
    """512^3 x 4 -> 32: layer-1 forward, pooling, backward-weight."""
    c = CONFIGS["partial_bf16_512c4_b1"]
    S, Co = c.in_size, c.filters[0]
    g = sd.torch_generator(4001, DEV)
    rng = np.random.default_rng(41)
    x = sd.lognormal_poisson_input_torch(g, (1, S, S, S), 4, DEV)
    w32, w = conv_weights(42, 4, Co)
    z = cf.cf_conv3d_fwd(x, w)
    torch.cuda.synchronize()
    assert z.numel() == 2 ** 32
    fwd_points(x, w32, z, rng, 2000)
    # pooling on synthetic N(0,1) activations of the same 2^32-element shape
    zs = sd.normal_torch(g, z.shape, DEV)
    del z
    P, idx = cf.cf_pool3d_fwd(zs, SLOPE)
    dp = sd.normal_torch(g, P.shape, DEV)
    dZ = cf.cf_pool3d_bwd(dp, P, idx, SLOPE)
    torch.cuda.synchronize()
    pool_slabs(zs, P, idx, dp, dZ, rng)
    del P, idx, dp, dZ
    # backward-weight over all 2^27 voxels
    dw = cf.cf_conv3d_bwd_weight(x, zs)
    torch.cuda.synchronize()
    wgrad_points(x, zs, dw, rng, 6)


def test_partial512_block2_full():
    """256^3 x 32 -> 64: forward, backward-data, backward-weight."""
    c = CONFIGS["partial_bf16_512c4_b1"]
    S, Ci, Co = c.in_size // 2, c.filters[0], c.filters[1]
    g = sd.torch_generator(4002, DEV)
    rng = np.random.default_rng(43)
    x = sd.normal_torch(g, (1, S, S, S, Ci), DEV).abs_()
    w32, w = conv_weights(44, Ci, Co)
    dz = sd.normal_torch(g, (1, S, S, S, Co), DEV)
    y = cf.cf_conv3d_fwd(x, w)
    dx = cf.cf_conv3d_bwd_data(dz, w)
    dw = cf.cf_conv3d_bwd_weight(x, dz)
    torch.cuda.synchronize()
    fwd_points(x, w32, y, rng, 2000)
    del y
    dgrad_points(dz, w32, dx, rng, 2000)
    wgrad_points(x, dz, dw, rng, 10)


TRAIN512 = CONFIGS["train_bf16_512c4_b1"]
C5_LAYERS = []
_s, _c = TRAIN512.in_size, TRAIN512.in_channels
for _f in TRAIN512.filters:
    C5_LAYERS.append((_s, _c, _f))
    _s, _c = _s // 2, _f


# layers 1 and 2 of the 7-block 512^3 network have the shapes of the two-block 512^3 workload's blocks
@pytest.mark.parametrize("layer", range(2, len(C5_LAYERS)))
def test_train512_layer_full(layer):
    S, Ci, Co = C5_LAYERS[layer]
    g = sd.torch_generator(5000 + layer, DEV)
    rng = np.random.default_rng(50 + layer)
    x = sd.normal_torch(g, (1, S, S, S, Ci), DEV).abs_()
    w32, w = conv_weights(60 + layer, Ci, Co)
    dz = sd.normal_torch(g, (1, S, S, S, Co), DEV)
    y = cf.cf_conv3d_fwd(x, w)
    dx = cf.cf_conv3d_bwd_data(dz, w)
    dw = cf.cf_conv3d_bwd_weight(x, dz)
    P, idx = cf.cf_pool3d_fwd(dz, SLOPE)
    dp = sd.normal_torch(g, P.shape, DEV)
    dZ = cf.cf_pool3d_bwd(dp, P, idx, SLOPE)
    torch.cuda.synchronize()
    fwd_points(x, w32, y, rng, 1500)
    dgrad_points(dz, w32, dx, rng, 1500)
    wgrad_points(x, dz, dw, rng, 16)
    pool_slabs(dz, P, idx, dp, dZ, rng)


def test_train512_train_step_full_consistency():
    """Full 7-block step at 512^3: finite loss, bitwise deterministic, equal
    to the composition of the individual entry points."""
    from test_gpu_train import composed_step
    c = TRAIN512
    g = sd.torch_generator(5100, DEV)
    x = sd.lognormal_poisson_input_torch(g, (1, c.in_size, c.in_size, c.in_size), 4, DEV)
    st = sd.streams(TRAIN512.seed_id)
    conv, cin = [], 4
    for f in c.filters:
        conv.append(sd.he_normal_conv(st["convw"], cin, f))
        cin = f
    dense, fan = [], 4 ** 3 * 256
    for o in c.dense:
        dense.append(sd.he_normal_dense(st["densew"], fan, o))
        fan = o
    t = torch.from_numpy(sd.targets(st["targets"], 1)).to(DEV)

    def params():
        ps = [torch.from_numpy(w).to(DEV) for w in conv]
        for W, b in dense:
            ps += [torch.from_numpy(W).to(DEV), torch.from_numpy(b).to(DEV)]
        return ps

    m = cf.model_desc(4, c.in_size, c.filters, c.dense, SLOPE)
    ws = torch.empty(cf.cf_train_step_workspace_size(m, cf.CF_BF16, 1), dtype=torch.uint8, device=DEV)
    p1, p2 = params(), params()
    l1, _ = cf.cf_train_step(m, x, t, p1, c.lr, ws=ws)
    l2, _ = cf.cf_train_step(m, x, t, p2, c.lr, ws=ws)
    torch.cuda.synchronize()
    assert np.isfinite(l1.item()) and torch.equal(l1, l2)
    for a, b in zip(p1, p2):
        assert torch.equal(a, b)
    del ws
    torch.cuda.empty_cache()
    p3 = params()
    l3 = composed_step(x, p3[:7], p3[7:], t, c.lr)
    torch.cuda.synchronize()
    assert torch.equal(l1, l3)
    for a, b in zip(p1, p3):
        assert torch.equal(a, b)
