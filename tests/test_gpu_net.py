"""GPU parity of the extended-network pieces against the fp64 oracle:

- the stride-2 "same" convolution (cf_conv3d_fwd / _bwd_data / _bwd_weight
  with stride 2; Oyama et al., Table I, c4) at even and odd sizes;
- 2^3 average pooling with leaky ReLU (cf_avgpool3d_fwd / _bwd; CosmoFlow
  Sec. III-A / III-C);
- cf_net_train_step: the Table I network at 128^3 (stride-2 c4, average
  pooling, no pool after c6 / c7, fc 2048-256-4 without bias), a network
  with batch norm and Adam + LARC, and the benchmark network, which must
  equal cf_train_step bit for bit.

Tolerances as elsewhere: fp32 1e-5, bf16 2e-2 of RMS (beyond one bf16
quantum for tensors both sides store in bf16)."""
import numpy as np
import pytest
import torch

import oracle
import synthdata as sd
from cnn_cosmology_volumes_amd import cf
from cnn_cosmology_volumes_amd.configs import oyama_table1_net
from gpu_util import TOL_BF16, TOL_F32, host64, rel_err, rel_err_bf16, to_dev

pytestmark = pytest.mark.gpu
BF, F32 = torch.bfloat16, torch.float32
SLOPE = 0.3
LR_RECOVER = 2.0 ** 20
POOL = {"max": cf.CF_POOL_MAX, "avg": cf.CF_POOL_AVG, "none": cf.CF_POOL_NONE}


# ------------------------------------------------------------ stride 2
@pytest.mark.parametrize("dtype", [BF, F32])
@pytest.mark.parametrize("shape", [(2, 16, 16, 16, 64, 128), (1, 9, 7, 11, 32, 32), (2, 6, 10, 8, 4, 16),
                                   (1, 5, 5, 5, 8, 12)])
def test_stride2_conv_matches_oracle(shape, dtype):
    N, D, H, W, Ci, Co = shape
    rng = np.random.default_rng(sum(shape))
    x = sd.normal(rng, (N, D, H, W, Ci), bf16=(dtype == BF))
    w = sd.he_normal_conv(rng, Ci, Co)
    w = sd.bf16_round_f32(w) if dtype == BF else w
    xd, wd = to_dev(x, dtype), to_dev(w, dtype)
    y = cf.cf_conv3d_fwd(xd, wd, stride=2)
    Do, Ho, Wo = (D + 1) // 2, (H + 1) // 2, (W + 1) // 2
    assert tuple(y.shape) == (N, Do, Ho, Wo, Co)
    dy = sd.normal(rng, (N, Do, Ho, Wo, Co), bf16=(dtype == BF))
    dyd = to_dev(dy, dtype)
    dx = cf.cf_conv3d_bwd_data(dyd, wd, xshape=x.shape, stride=2)
    dw = cf.cf_conv3d_bwd_weight(xd, dyd, stride=2)
    torch.cuda.synchronize()
    # the oracle's rule for non-cubic volumes: its same_geometry per dimension
    p = (D & 1)
    yo = np.empty((N, Do, Ho, Wo, Co))
    lib = oracle.lib()
    f = lambda a: np.ascontiguousarray(a, np.float64)
    lib.or_conv3d_fwd_s(N, D, H, W, Ci, Co, 2, p, Do, Ho, Wo, oracle._ptr(f(x)), oracle._ptr(f(w)), oracle._ptr(yo))
    dxo = np.empty((N, D, H, W, Ci))
    lib.or_conv3d_bwd_data_s(N, D, H, W, Ci, Co, 2, p, Do, Ho, Wo, oracle._ptr(f(dy)), oracle._ptr(f(w)),
                             oracle._ptr(dxo))
    dwo = np.empty((3, 3, 3, Ci, Co))
    lib.or_conv3d_bwd_weight_s(N, D, H, W, Ci, Co, 2, p, Do, Ho, Wo, oracle._ptr(f(x)), oracle._ptr(f(dy)),
                               oracle._ptr(dwo))
    if dtype == F32:
        assert rel_err(host64(y), yo) <= TOL_F32
        assert rel_err(host64(dx), dxo) <= TOL_F32
        assert rel_err(host64(dw), dwo) <= TOL_F32
    else:
        assert rel_err(host64(y), yo) <= TOL_BF16
        assert rel_err(host64(dx), dxo) <= TOL_BF16
        assert rel_err(host64(dw), dwo) <= 1e-4      # fp32 sums of exact bf16 products


def test_stride2_rejects_wrong_padding():
    x = torch.zeros((1, 8, 8, 8, 32), dtype=BF, device="cuda")
    w = torch.zeros((3, 3, 3, 32, 32), dtype=BF, device="cuda")
    y = torch.empty((1, 4, 4, 4, 32), dtype=BF, device="cuda")
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    st = cf.lib().cf_conv3d_fwd(cf.CF_BF16, cf.dims(x.shape), cf._ptr(x), cf._ptr(w), 32, cf.cf_conv(3, 2, 1),
                                cf._ptr(y), cf._ptr(ws), 1 << 24, cf._stream())
    assert st == cf.CF_ERR_UNSUPPORTED   # even sizes take pad 0


# ------------------------------------------------------------ average pool
@pytest.mark.parametrize("dtype", [BF, F32])
@pytest.mark.parametrize("shape", [(2, 6, 10, 8, 16), (1, 4, 4, 4, 4), (2, 8, 8, 8, 256)])
def test_avgpool_matches_oracle(shape, dtype):
    rng = np.random.default_rng(sum(shape) + 1)
    z = sd.normal(rng, shape, bf16=(dtype == BF))
    Np, Dp, Hp, Wp = shape[0], shape[1] // 2, shape[2] // 2, shape[3] // 2
    dp = sd.normal(rng, (Np, Dp, Hp, Wp, shape[4]), bf16=(dtype == BF))
    zd, dpd = to_dev(z, dtype), to_dev(dp, dtype)
    P = cf.cf_avgpool3d_fwd(zd, SLOPE)
    dZ = cf.cf_avgpool3d_bwd(dpd, zd, SLOPE)
    torch.cuda.synchronize()
    po = oracle.avgpool_fwd(oracle.lrelu_fwd(z, SLOPE))
    dzo = oracle.lrelu_bwd(z, oracle.avgpool_bwd(dp), SLOPE)
    if dtype == F32:
        assert rel_err(host64(P), po) <= TOL_F32 and rel_err(host64(dZ), dzo) <= TOL_F32
    else:
        assert rel_err_bf16(host64(P), oracle.round_bf16(po)) <= TOL_BF16
        assert rel_err_bf16(host64(dZ), oracle.round_bf16(dzo)) <= TOL_BF16


# ------------------------------------------------------------ network step
def make_net(layers, dense, in_ch, size, batch_norm, dense_bias):
    return cf.net_desc(in_ch, size, [l[0] for l in layers], [l[1] for l in layers], [POOL[l[2]] for l in layers],
                       dense=dense, dense_bias=dense_bias, batch_norm=batch_norm, slope=SLOPE)


def init_params(rng, shapes, batch_norm):
    ps = []
    for i, sh in enumerate(shapes):
        if len(sh) == 5:
            ps.append(sd.he_normal_conv(rng, sh[3], sh[4]))
        elif len(sh) == 2:
            ps.append(sd.he_normal_dense(rng, sh[0], sh[1])[0])
        else:
            ps.append(rng.uniform(0.5, 1.5, sh).astype(np.float32) if batch_norm and len(shapes[i - 1]) == 5
                      else (rng.standard_normal(sh) * 0.05).astype(np.float32))
    return ps


def net_problem(layers, dense, size, B, dtype, batch_norm, dense_bias, seed):
    rng = np.random.default_rng(seed)
    x = sd.lognormal_poisson_input(rng, rng, (B, size, size, size), 4, bf16=(dtype == BF))
    t = sd.targets(rng, B, dense[-1])
    m = make_net(layers, dense, 4, size, batch_norm, dense_bias)
    shapes = oracle.net_param_shapes(4, layers, dense, batch_norm, dense_bias, size)
    assert [int(np.prod(s)) for s in shapes] == cf.cf_net_param_count(m)
    return x, t, m, init_params(rng, shapes, batch_norm)


# Relative size of the conditioning perturbation of the oracle's conv sums
# (about the fp32 accumulation error of the GPU's sums), the number of
# perturbed oracle runs, and the margin over their largest deviation.  The
# largest deviation of a gradient is set by its single largest flipped
# decision, so it varies from run to run: three runs and a factor 3.
PERTURB = 2.0 ** -22
SPREAD_SEEDS = (1, 2, 3)
SPREAD_FACTOR = 3.0


def oracle_spread(x, t, params, layers, dense, batch_norm, dense_bias, storage, ref_grads):
    """How far the step's gradients are determined by the arithmetic: the
    largest rel_err between the oracle's gradients and those of two oracle
    runs whose conv sums are perturbed by PERTURB before rounding.  Leaky-ReLU
    kinks (either slope is accepted there), near-tied max-pool windows, and
    at small batches the few terms of the deep layers' and the head's
    gradients make single decisions weigh heavily."""
    spread = [0.0] * len(ref_grads)
    for seed in SPREAD_SEEDS:
        print("oracle step with perturbed conv sums, seed %d ..." % seed, flush=True)
        alt = oracle.net_train_step(x, t, params, layers, dense, SLOPE, batch_norm=batch_norm, dense_bias=dense_bias,
                                    storage=storage, opt=("sgd", LR_RECOVER),
                                    perturb=(np.random.default_rng(seed), PERTURB))
        spread = [max(sp, rel_err(a, r)) for sp, a, r in zip(spread, alt["grads"], ref_grads)]
    return spread


def check_net_step(layers, dense, size, B, dtype, batch_norm, dense_bias, seed, label):
    """SGD step with a power-of-two rate (gradients recovered from the
    update): loss and predictions gated at the path's tolerance, each
    gradient at max(tolerance, SPREAD_FACTOR x the oracle's own spread)."""
    x, t, m, params = net_problem(layers, dense, size, B, dtype, batch_norm, dense_bias, seed)
    pd = [to_dev(p, F32) for p in params]
    old = [host64(p) for p in pd]
    pred = torch.empty((B, dense[-1]), dtype=F32, device="cuda")
    loss, _ = cf.cf_net_train_step(m, to_dev(x, dtype), to_dev(t, F32), pd, cf.sgd_optimizer(LR_RECOVER), pred=pred)
    torch.cuda.synchronize()
    grads = [(o_ - host64(p)) / LR_RECOVER for o_, p in zip(old, pd)]
    storage = "bf16" if dtype == BF else "f32"
    print("GPU step done; oracle step ...", flush=True)
    ref = oracle.net_train_step(x, t, params, layers, dense, SLOPE, batch_norm=batch_norm, dense_bias=dense_bias,
                                storage=storage, opt=("sgd", LR_RECOVER))
    spread = oracle_spread(x, t, params, layers, dense, batch_norm, dense_bias, storage, ref["grads"])
    tol = TOL_BF16 if dtype == BF else TOL_F32
    e_loss = abs(loss.item() - ref["loss"]) / ref["loss"]
    e_pred = rel_err(host64(pred), ref["yhat"])
    errs = [rel_err(g, r) for g, r in zip(grads, ref["grads"])]
    print("%s (%s) vs oracle: loss %.2e, pred %.2e; gradients %s" % (
        label, dtype, e_loss, e_pred, ", ".join("%.2e (spread %.2e)" % es for es in zip(errs, spread))), flush=True)
    assert e_loss <= tol and e_pred <= tol
    bad = [(i, e, sp) for i, (e, sp) in enumerate(zip(errs, spread)) if not e <= max(tol, SPREAD_FACTOR * sp)]
    assert not bad, bad


TABLE1_128 = [(16, 1, "avg"), (32, 1, "avg"), (64, 1, "avg"), (128, 2, "avg"), (256, 1, "avg"), (256, 1, "none"),
              (256, 1, "none")]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype", [BF, F32])
def test_table1_network_step_matches_oracle(dtype):
    """The extended network of Oyama et al., Table I, at 128^3 (batch 2)."""
    net = oyama_table1_net(128)
    assert [(L.cout, L.stride, "avg" if L.pool else "none") for L in net.convs] == TABLE1_128
    check_net_step(TABLE1_128, [2048, 256, 4], 128, 2, dtype, False, False, 41, "Table I 128^3 network step")


SMALL_BN = [(16, 1, "avg"), (32, 1, "max"), (64, 2, "avg"), (64, 1, "none")]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("dtype", [BF, F32])
def test_bn_network_step_matches_oracle(dtype):
    """Batch norm after every conv, average / max / no pooling, a stride-2
    layer, no dense bias."""
    check_net_step(SMALL_BN, [64, 16, 4], 32, 2, dtype, True, False, 42, "BN network step")


@pytest.mark.parametrize("dtype", [BF, F32])
def test_bn_network_adam_step_matches_oracle(dtype):
    """Adam + LARC inside cf_net_train_step (update 3, decayed rate, nonzero
    moments).  The update must be the oracle's per-tensor Adam + LARC step
    applied to the gradient this same network step computes: that gradient
    is read back from an SGD run of the identical step (forward and backward
    do not depend on the optimizer; the equal loss and predictions of the two
    runs confirm it).  The gradient itself is compared with the oracle's in
    test_bn_network_step_matches_oracle; the update's arithmetic is fp32, so
    it is held to the fp32 tolerance whatever the network's dtype."""
    layers, dense = SMALL_BN, [64, 16, 4]
    B, t_upd = 2, 3
    x, t, m, params = net_problem(layers, dense, 32, B, dtype, True, False, 43)
    rng = np.random.default_rng(44)
    m0 = [(rng.standard_normal(p.shape) * 1e-3).astype(np.float32) for p in params]
    v0 = [(rng.uniform(0.0, 1e-5, p.shape)).astype(np.float32) for p in params]
    xd, td = to_dev(x, dtype), to_dev(t, F32)

    # the step's own gradient, from an SGD run with a power-of-two rate
    ps = [to_dev(p, F32) for p in params]
    pred_s = torch.empty((B, dense[-1]), dtype=F32, device="cuda")
    loss_s, _ = cf.cf_net_train_step(m, xd, td, ps, cf.sgd_optimizer(LR_RECOVER), pred=pred_s)

    pa = [to_dev(p, F32) for p in params]
    mom = ([to_dev(a, F32) for a in m0], [to_dev(a, F32) for a in v0])
    hp = cf.adam_larc_params(0.01, lr_end=0.001, decay_steps=10, trust=0.02)
    pred_a = torch.empty((B, dense[-1]), dtype=F32, device="cuda")
    loss_a, _ = cf.cf_net_train_step(m, xd, td, pa, cf.adam_optimizer(hp, t_upd), moments=mom, pred=pred_a)
    torch.cuda.synchronize()
    assert torch.equal(loss_s, loss_a) and torch.equal(pred_s, pred_a)

    storage = "bf16" if dtype == BF else "f32"
    ref = oracle.net_train_step(x, t, params, layers, dense, SLOPE, batch_norm=True, dense_bias=False, storage=storage,
                                opt=("sgd", LR_RECOVER))
    tol = TOL_BF16 if dtype == BF else TOL_F32
    assert abs(loss_a.item() - ref["loss"]) <= tol * ref["loss"]
    assert rel_err(host64(pred_a), ref["yhat"]) <= tol

    f = lambda v: float(np.float32(v))
    lr_t = oracle.poly_decay(f(0.01), f(0.001), 10, 1.0, t_upd - 1)
    for i, p0 in enumerate(params):
        g = (np.float64(p0) - host64(ps[i])) / LR_RECOVER
        w_o, m_o, v_o, _ = oracle.adam_larc_step(p0, g, m0[i], v0[i], t_upd, lr_t, f(0.9), f(0.999), f(1e-8), f(0.02))
        # beyond the one fp32 rounding of the stored weight, relative to the step
        got = host64(pa[i])
        beyond = np.maximum(np.abs(got - w_o) - 0.5 * np.spacing(np.abs(w_o).astype(np.float32)), 0.0)
        d_want = w_o - np.float64(p0)
        e = float(beyond.max() / np.sqrt(np.mean(d_want * d_want)))
        assert e <= TOL_F32, (i, e)
        assert rel_err(host64(mom[0][i]), m_o) <= TOL_F32, i
        assert rel_err(host64(mom[1][i]), v_o) <= TOL_F32, i


def test_benchmark_network_through_net_step_equals_train_step():
    """The 5-block benchmark network run by cf_net_train_step (unfused
    kernels, single stream) equals cf_train_step (fused kernels, second
    stream) bit for bit."""
    from test_gpu_train import device_params, make_problem
    B, size, filters, dense_w = 2, 32, [32, 64, 128], [64, 32, 3]
    x, conv, dense, t = make_problem(7, B, size, filters, dense_w, BF)
    xd, td = to_dev(x, BF), to_dev(t, F32)
    p1, p2 = device_params(conv, dense), device_params(conv, dense)
    m = cf.model_desc(4, size, filters, dense_w, SLOPE)
    aux = cf.StepAux()
    l1, _ = cf.cf_train_step(m, xd, td, p1, 1e-3, aux=aux)
    mn = cf.net_desc(4, size, filters, dense=dense_w, slope=SLOPE)
    l2, _ = cf.cf_net_train_step(mn, xd, td, p2, cf.sgd_optimizer(1e-3))
    torch.cuda.synchronize()
    assert torch.equal(l1, l2)
    for a, b in zip(p1, p2):
        assert torch.equal(a, b)
