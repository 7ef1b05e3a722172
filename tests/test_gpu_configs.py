"""Parity at the full sizes of the five benchmark configurations, in the
launch configurations the benchmark uses.  Outputs too large for the oracle
are checked on samples it computes one by one: random output points plus the
volume corners for the convolutions, whole slabs for the pooling kernels
(pooling is window-local, so a slab of the input determines the matching
slab of the output), and individual weight-gradient entries (each a full sum
over every voxel).  Inputs are the seeded generators' synthetic volumes."""
import numpy as np
import pytest
import torch

import oracle
import synthdata as sd
from cnn_cosmology_volumes_amd import cf
from cnn_cosmology_volumes_amd.configs import CONFIGS
from gpu_util import TOL_BF16, TOL_F32, bf16_elementwise_ok, host32, host64, rel_err, sample_points, to_dev

pytestmark = pytest.mark.gpu
BF, F32 = torch.bfloat16, torch.float32
SLOPE = 0.3


def check_conv_fwd(x32, w32, y_dev, rng, npts=3000):
    pts = sample_points(rng, tuple(y_dev.shape), npts)
    o = oracle.conv3d_fwd_points(x32, w32, pts)
    g = host64(y_dev.reshape(-1)[torch.from_numpy(pts).to(y_dev.device)])
    assert rel_err(g, o) <= TOL_BF16
    assert bf16_elementwise_ok(g, o) == 0


def check_conv_dgrad(dy32, w32, dx_dev, rng, npts=3000):
    pts = sample_points(rng, tuple(dx_dev.shape), npts)
    o = oracle.conv3d_bwd_data_points(dy32, w32, pts)
    g = host64(dx_dev.reshape(-1)[torch.from_numpy(pts).to(dx_dev.device)])
    assert rel_err(g, o) <= TOL_BF16
    assert bf16_elementwise_ok(g, o) == 0


def check_conv_wgrad(x32, dy32, dw_dev, rng, npts=24):
    ci, co = x32.shape[4], dy32.shape[4]
    total = 27 * ci * co
    pts = set(int(p) for p in rng.integers(0, total, npts))
    for t in (0, 13, 26):                      # corner and centre taps
        pts.add((t * ci + ci - 1) * co + co - 1)
        pts.add((t * ci) * co)
    pts = np.array(sorted(pts), np.int64)
    o = oracle.conv3d_bwd_weight_points(x32, dy32, pts)
    g = host64(dw_dev.reshape(-1)[torch.from_numpy(pts).to(dw_dev.device)])
    # exact bf16 inputs: only the fp32 accumulation order differs
    assert rel_err(g, o) <= 1e-3
    assert np.max(np.abs(g - o)) <= 1e-3 * max(np.max(np.abs(o)), 1e-30)


def check_pool_slabs(z32, p_dev, idx_dev, dp32, dz_dev, rng, nslab=2):
    """Compare a few depth slabs [n, 2a:2a+2] of the pooled outputs."""
    N, D = z32.shape[0], z32.shape[1]
    for _ in range(nslab):
        n = int(rng.integers(0, N))
        a = int(rng.integers(0, D // 2))
        zs = z32[n:n + 1, 2 * a:2 * a + 2]
        po, io = oracle.lrelu_maxpool_fwd(zs, SLOPE)
        gp = host64(p_dev[n:n + 1, a:a + 1])
        gi = idx_dev[n:n + 1, a:a + 1].cpu().numpy()
        assert np.array_equal(gi, io)
        assert np.all(np.abs(gp - po) <= 2.0 ** -8 * np.abs(po))
        dzo = oracle.maxpool_lrelu_bwd(dp32[n:n + 1, a:a + 1], po, io, SLOPE)
        gz = host64(dz_dev[n:n + 1, 2 * a:2 * a + 2])
        assert np.all(np.abs(gz - dzo) <= 2.0 ** -8 * np.abs(dzo))


# ------------------------------------- one conv forward, fp32, 1 x 32^3 x 4 -> 16
def test_conv_fwd_f32_32c4_full():
    c = CONFIGS["conv3d_fwd_f32_32c4"]
    st = sd.streams(c.seed_id)
    x = sd.lognormal_field_input(st["field"], (c.batch, c.in_size, c.in_size, c.in_size), c.in_channels)
    w = sd.he_normal_conv(st["convw"], c.in_channels, c.filters[0])
    y = cf.cf_conv3d_fwd(to_dev(x, F32), to_dev(w, F32))
    torch.cuda.synchronize()
    assert rel_err(host64(y), oracle.conv3d_fwd(x, w)) <= TOL_F32


# ----------------------------------- one block, bf16, 4 x 128^3 x 4 -> 32
def test_block_128c4_b4_full():
    c = CONFIGS["block_bf16_128c4_b4"]
    st = sd.streams(c.seed_id)
    S, B, Cin, Co = c.in_size, c.batch, c.in_channels, c.filters[0]
    x = sd.lognormal_poisson_input(st["field"], st["poisson"], (B, S, S, S), Cin)
    w = sd.bf16_round_f32(sd.he_normal_conv(st["convw"], Cin, Co))
    rng = np.random.default_rng(2)
    xd, wd = to_dev(x, BF), to_dev(w, BF)
    # forward conv
    y = cf.cf_conv3d_fwd(xd, wd)
    torch.cuda.synchronize()
    check_conv_fwd(x, w, y, rng)
    del y
    # pooling forward/backward on synthetic full-size activations
    z = sd.normal(st["upstream"], (B, S, S, S, Co))
    dp = sd.normal(st["upstream"], (B, S // 2, S // 2, S // 2, Co))
    zd = to_dev(z, BF)
    P, idx = cf.cf_pool3d_fwd(zd, SLOPE)
    dZ = cf.cf_pool3d_bwd(to_dev(dp, BF), P, idx, SLOPE)
    torch.cuda.synchronize()
    check_pool_slabs(z, P, idx, dp, dZ, rng)
    del zd, P, idx
    # backward-data and backward-weight of the block's conv with a full-size dZ
    dzd = to_dev(z, BF)   # N(0,1) upstream gradient of the conv output
    dx = cf.cf_conv3d_bwd_data(dzd, wd)
    dw = cf.cf_conv3d_bwd_weight(xd, dzd)
    torch.cuda.synchronize()
    check_conv_dgrad(z, w, dx, rng)
    check_conv_wgrad(x, z, dw, rng)


# ---------------------------- 5-block network training step, bf16, 8 x 128^3 x 4
TRAIN128 = CONFIGS["train_bf16_128c4_b8"]
C3_LAYERS = []
_s, _c = TRAIN128.in_size, TRAIN128.in_channels
for _f in TRAIN128.filters:
    C3_LAYERS.append((_s, _c, _f))
    _s, _c = _s // 2, _f


@pytest.mark.parametrize("layer", range(len(C3_LAYERS)))
def test_train128_conv_layer_full(layer):
    S, Cin, Co = C3_LAYERS[layer]
    B = TRAIN128.batch
    st = sd.streams(TRAIN128.seed_id)
    rng = np.random.default_rng(30 + layer)
    if layer == 0:
        x = sd.lognormal_poisson_input(st["field"], st["poisson"], (B, S, S, S), Cin)
    else:
        # pooled leaky-ReLU activations are mostly positive with a negative tail
        x = np.abs(sd.normal(st["field"], (B, S, S, S, Cin))) * np.float32(1.0)
        x[..., ::3] *= np.float32(-0.3)
        x = sd.bf16_round_f32(x)
    w = sd.bf16_round_f32(sd.he_normal_conv(st["convw"], Cin, Co))
    dz = sd.normal(st["upstream"], (B, S, S, S, Co))
    xd, wd, dzd = to_dev(x, BF), to_dev(w, BF), to_dev(dz, BF)
    y = cf.cf_conv3d_fwd(xd, wd)
    dw = cf.cf_conv3d_bwd_weight(xd, dzd)
    dx = cf.cf_conv3d_bwd_data(dzd, wd) if layer > 0 else None
    torch.cuda.synchronize()
    check_conv_fwd(x, w, y, rng)
    check_conv_wgrad(x, dz, dw, rng)
    if dx is not None:
        check_conv_dgrad(dz, w, dx, rng)


@pytest.mark.parametrize("layer", range(len(C3_LAYERS)))
def test_train128_pool_level_full(layer):
    S, _, Co = C3_LAYERS[layer]
    B = TRAIN128.batch
    st = sd.streams(TRAIN128.seed_id)
    rng = np.random.default_rng(40 + layer)
    z = sd.normal(st["upstream"], (B, S, S, S, Co))
    dp = sd.normal(st["upstream"], (B, S // 2, S // 2, S // 2, Co))
    P, idx = cf.cf_pool3d_fwd(to_dev(z, BF), SLOPE)
    dZ = cf.cf_pool3d_bwd(to_dev(dp, BF), P, idx, SLOPE)
    torch.cuda.synchronize()
    check_pool_slabs(z, P, idx, dp, dZ, rng)


def test_train128_dense_head_full():
    """Dense head at the headline shape; the oracle runs its own chain from
    the same synthetic input and weights."""
    st = sd.streams(TRAIN128.seed_id)
    B = TRAIN128.batch
    widths = [4 ** 3 * 256] + TRAIN128.dense
    x = sd.normal(st["field"], (B, widths[0]), bf16=True)
    h = x.astype(np.float64)
    hd = to_dev(x, F32)
    for k in range(3):
        W, _ = sd.he_normal_dense(st["densew"], widths[k], widths[k + 1])
        b = (st["densew"].standard_normal(widths[k + 1]) * 0.05).astype(np.float32)
        s = SLOPE if k < 2 else -1.0
        dy = st["upstream"].standard_normal((B, widths[k + 1])).astype(np.float32)
        pre, y = cf.cf_dense_fwd(hd, to_dev(W, F32), to_dev(b, F32), s)
        dx, dw, db = cf.cf_dense_bwd(hd, to_dev(W, F32), pre, to_dev(dy, F32), s)
        torch.cuda.synchronize()
        pre_o, y_o = oracle.dense_fwd(h, W, b, s)
        assert rel_err(host64(pre), pre_o) <= TOL_F32
        assert rel_err(host64(y), y_o) <= TOL_F32
        dx_o, dw_o, db_o = oracle.dense_bwd(h, W, pre_o, dy, s)
        assert rel_err(host64(dx), dx_o) <= TOL_F32
        assert rel_err(host64(dw), dw_o) <= TOL_F32
        assert rel_err(host64(db), db_o) <= TOL_F32
        hd, h = y, y_o


def test_train128_train_step_full_consistency():
    """Full-size headline step: finite loss, bitwise deterministic, and equal
    to the composition of the individual entry points."""
    from test_gpu_train import composed_step, device_params
    c = TRAIN128
    st = sd.streams(TRAIN128.seed_id)
    x = sd.lognormal_poisson_input(st["field"], st["poisson"], (c.batch, c.in_size, c.in_size, c.in_size), 4)
    conv, cin = [], 4
    for f in c.filters:
        conv.append(sd.he_normal_conv(st["convw"], cin, f))
        cin = f
    dense, fan = [], 4 ** 3 * 256
    for o in c.dense:
        dense.append(sd.he_normal_dense(st["densew"], fan, o))
        fan = o
    t = sd.targets(st["targets"], c.batch)
    m = cf.model_desc(4, c.in_size, c.filters, c.dense, SLOPE)
    xd, td = to_dev(x, BF), to_dev(t, F32)
    p1, p2, p3 = device_params(conv, dense), device_params(conv, dense), device_params(conv, dense)
    l1, _ = cf.cf_train_step(m, xd, td, p1, c.lr)
    l2, _ = cf.cf_train_step(m, xd, td, p2, c.lr)
    l3 = composed_step(xd, p3[:5], p3[5:], td, c.lr)
    torch.cuda.synchronize()
    assert np.isfinite(l1.item())
    assert torch.equal(l1, l2) and torch.equal(l1, l3)
    for a, b, cc in zip(p1, p2, p3):
        assert torch.equal(a, b) and torch.equal(a, cc)


def test_train128_training_lowers_loss():
    """Repeated steps on one fixed batch of the 128^3 x 4 workload: every
    loss is finite, the loss falls over the first steps (gradient descent on
    a smooth loss with a small step), and after 20 steps it is below a tenth
    of the first one."""
    from test_gpu_train import device_params
    c = TRAIN128
    st = sd.streams(TRAIN128.seed_id)
    x = sd.lognormal_poisson_input(st["field"], st["poisson"], (c.batch, c.in_size, c.in_size, c.in_size), 4)
    conv, cin = [], 4
    for f in c.filters:
        conv.append(sd.he_normal_conv(st["convw"], cin, f))
        cin = f
    dense, fan = [], 4 ** 3 * 256
    for o in c.dense:
        dense.append(sd.he_normal_dense(st["densew"], fan, o))
        fan = o
    t = sd.targets(st["targets"], c.batch)
    m = cf.model_desc(4, c.in_size, c.filters, c.dense, SLOPE)
    xd, td = to_dev(x, BF), to_dev(t, F32)
    params = device_params(conv, dense)
    ws = torch.empty(cf.cf_train_step_workspace_size(m, cf.CF_BF16, c.batch), dtype=torch.uint8, device="cuda")
    losses = []
    for _ in range(20):
        l, _ = cf.cf_train_step(m, xd, td, params, c.lr, ws=ws)
        losses.append(float(l.item()))
    assert all(np.isfinite(losses)), losses
    assert all(b < a for a, b in zip(losses[:10], losses[1:11])), losses
    assert losses[-1] < 0.1 * losses[0], losses


# ------------------------- weight-ring convolutions with many ragged tiles
# More tiles than one round of resident blocks, ragged against the tiles:
# backward-data into 32 channels (the 32-channel ring block, two input
# chunks); the pooled block forward of 64 -> 128 channels (the 64-channel
# ring block on 4 x 4 x 16 tiles); and a 64 -> 64 forward on a volume 8 wide
# (the 64-channel ring block on 4 x 8 x 8 tiles).
@pytest.mark.parametrize("shape", [(5, 18, 34, 66, 64, 32), (4, 16, 34, 66, 64, 128), (40, 16, 30, 8, 64, 64)])
def test_ring_conv_many_ragged_tiles(shape):
    N, D, H, W, Ci, Co = shape
    rng = np.random.default_rng(sum(shape) + 41)
    x = sd.normal(rng, (N, D, H, W, Ci), bf16=True)
    w = sd.bf16_round_f32(sd.he_normal_conv(rng, Ci, Co))
    xd, wd = to_dev(x, torch.bfloat16), to_dev(w, torch.bfloat16)
    if Co == 32:
        # backward-data of a Co-input conv: dY has Ci channels, dX has Co
        wt = sd.bf16_round_f32(sd.he_normal_conv(rng, Co, Ci))
        dx = cf.cf_conv3d_bwd_data(xd, to_dev(wt, torch.bfloat16))
        torch.cuda.synchronize()
        check_conv_dgrad(x, wt, dx, rng)
        return
    y = cf.cf_conv3d_fwd(xd, wd)
    torch.cuda.synchronize()
    check_conv_fwd(x, w, y, rng)
    if D % 2 == 0 and H % 2 == 0 and W % 2 == 0:
        P, idx = cf.cf_conv3d_pool_fwd(xd, wd, SLOPE)
        P2, idx2 = cf.cf_pool3d_fwd(y, SLOPE)
        torch.cuda.synchronize()
        assert torch.equal(P.view(torch.int16), P2.view(torch.int16)) and torch.equal(idx, idx2)
