"""GPU parity of the optimizer (cf_adam_larc: Adam + LARC + polynomial decay)
and of training-mode batch normalisation (cf_batchnorm_fwd / _bwd) against
the fp64 oracle, from the same seeded fp32 / bf16 inputs.

Tolerances: max |gpu - oracle| / RMS(oracle) <= 1e-5 for fp32 results; bf16
outputs (both sides rounded to bf16) <= 2e-2 beyond one bf16 quantum."""
import numpy as np
import pytest
import torch

import oracle
import synthdata as sd
from cnn_cosmology_volumes_amd import cf
from gpu_util import TOL_BF16, TOL_F32, host64, rel_err, rel_err_bf16, to_dev

pytestmark = pytest.mark.gpu
BF, F32 = torch.bfloat16, torch.float32


# ---------------------------------------------------------------- optimizer
# tensor sizes: one element, a ragged tail, exactly one chunk, several
# chunks with a tail (the dense layer-1 weight of the 128^3 network)
SIZES = [1, 37, 4096, 27 * 32 * 64, 16384 * 128 + 3]


@pytest.mark.parametrize("trust", [0.0, 0.02, 1e3])
def test_adam_larc_matches_oracle_over_steps(trust):
    rng = np.random.default_rng(11 + int(trust * 100))
    ws = [(rng.standard_normal(n) * rng.uniform(0.05, 2.0)).astype(np.float32) for n in SIZES]
    hp = cf.adam_larc_params(0.05, lr_end=0.0005, decay_steps=4, power=1.0, trust=trust)
    # the oracle gets the hyperparameters as the GPU receives them (fp32)
    f = lambda v: float(np.float32(v))
    b1, b2, eps, tr = f(0.9), f(0.999), f(1e-8), f(trust)
    wd = [torch.from_numpy(w.copy()).cuda() for w in ws]
    md = [torch.zeros_like(w) for w in wd]
    vd = [torch.zeros_like(w) for w in wd]
    lr_out = torch.zeros(len(SIZES), dtype=F32, device="cuda")
    wo = [w.astype(np.float64) for w in ws]
    mo = [np.zeros(n) for n in SIZES]
    vo = [np.zeros(n) for n in SIZES]
    for t in range(1, 7):     # past the end of the decay (held at lr_end)
        gs = [(rng.standard_normal(n) * rng.uniform(0.1, 10.0)).astype(np.float32) for n in SIZES]
        gd = [torch.from_numpy(g).cuda() for g in gs]
        cf.cf_adam_larc(hp, t, wd, gd, md, vd, lr_out=lr_out)
        torch.cuda.synchronize()
        lr_t = oracle.poly_decay(f(0.05), f(0.0005), 4, 1.0, t - 1)
        lrs = []
        for i in range(len(SIZES)):
            # the oracle continues from the GPU's fp32 state, so each update
            # is compared on its own (no drift between fp32 and fp64 state)
            w_prev = wo[i]
            wo[i], mo[i], vo[i], lr_l = oracle.adam_larc_step(w_prev, gs[i], mo[i], vo[i], t, lr_t, b1, b2, eps, tr)
            lrs.append(lr_l)
            assert rel_err(host64(md[i]), mo[i]) <= TOL_F32, (t, i)
            assert rel_err(host64(vd[i]), vo[i]) <= TOL_F32, (t, i)
            # the step itself, relative to its own size, beyond the fp32
            # rounding of the updated weight
            dg, do = host64(wd[i]) - w_prev, wo[i] - w_prev
            bound = TOL_F32 * np.sqrt(np.mean(do * do)) + 2.0 ** -23 * np.abs(wo[i])
            assert np.all(np.abs(dg - do) <= bound), (t, i)
            assert rel_err(host64(wd[i]), wo[i]) <= TOL_F32, (t, i)
            wo[i], mo[i], vo[i] = host64(wd[i]), host64(md[i]), host64(vd[i])
        assert np.allclose(host64(lr_out), lrs, rtol=1e-6, atol=0), (t, host64(lr_out), lrs)
        if trust == 0.02:
            # the trust ratio is active on some tensors and not on others
            assert min(lrs) < lr_t * 0.999 or t > 4


def test_adam_larc_is_deterministic_and_validates():
    rng = np.random.default_rng(3)
    n = 16384 * 128
    w0 = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
    g = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).cuda()
    hp = cf.adam_larc_params(0.01, trust=0.01)
    outs = []
    for _ in range(2):
        w, m, v = w0.clone(), torch.zeros_like(w0), torch.zeros_like(w0)
        cf.cf_adam_larc(hp, 1, [w], [g], [m], [v])
        outs.append(w)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    with pytest.raises(cf.CfError) as e:
        cf.cf_adam_larc(hp, 0, [w], [g], [m], [v])      # t starts at 1
    assert e.value.status == cf.CF_ERR_INVALID


# --------------------------------------------------------------- batch norm
BN_CASES = [(2, 5, 6, 7, 16), (1, 8, 8, 8, 64), (2, 3, 3, 3, 256), (3, 4, 4, 6, 12), (1, 2, 2, 2, 4)]


@pytest.mark.parametrize("dtype", [F32, BF])
@pytest.mark.parametrize("shape", BN_CASES)
def test_batchnorm_matches_oracle(shape, dtype):
    rng = np.random.default_rng(sum(shape))
    C = shape[4]
    # a channel mean away from zero, as after a convolution of positive inputs
    x = sd.normal(rng, shape, bf16=(dtype == BF), scale=1.5) + np.float32(0.75)
    x = sd.bf16_round_f32(x) if dtype == BF else x
    dy = sd.normal(rng, shape, bf16=(dtype == BF))
    gamma = rng.uniform(-1.5, 1.5, C).astype(np.float32)
    beta = rng.uniform(-0.5, 0.5, C).astype(np.float32)
    eps = 1e-5
    xd, dyd = to_dev(x, dtype), to_dev(dy, dtype)
    gd, bd = to_dev(gamma, F32), to_dev(beta, F32)
    Y, mean, invstd = cf.cf_batchnorm_fwd(xd, gd, bd, eps)
    dX, dgamma, dbeta = cf.cf_batchnorm_bwd(xd, dyd, gd, mean, invstd)
    torch.cuda.synchronize()
    yo, mo, iso = oracle.batchnorm_fwd(x, gamma, beta, eps)
    dxo, dgo, dbo = oracle.batchnorm_bwd(x, dy, gamma, mo, iso)
    assert rel_err(host64(mean), mo) <= TOL_F32
    assert rel_err(host64(invstd), iso) <= TOL_F32
    assert rel_err(host64(dgamma), dgo) <= TOL_F32
    assert rel_err(host64(dbeta), dbo) <= TOL_F32
    if dtype == F32:
        assert rel_err(host64(Y), yo) <= TOL_F32
        assert rel_err(host64(dX), dxo) <= TOL_F32
    else:
        assert rel_err_bf16(host64(Y), oracle.round_bf16(yo)) <= TOL_BF16
        assert rel_err_bf16(host64(dX), oracle.round_bf16(dxo)) <= TOL_BF16


def test_batchnorm_full_size_layer():
    """The second block's conv output of the 128^3 network (8 x 64^3 x 64,
    bf16): 512 reduction blocks per channel."""
    rng = np.random.default_rng(64)
    shape = (8, 64, 64, 64, 64)
    x = sd.normal(rng, shape, bf16=True, scale=2.0)
    dy = sd.normal(rng, shape, bf16=True)
    gamma = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    beta = rng.uniform(-0.5, 0.5, 64).astype(np.float32)
    xd, dyd = to_dev(x, BF), to_dev(dy, BF)
    gd, bd = to_dev(gamma, F32), to_dev(beta, F32)
    Y, mean, invstd = cf.cf_batchnorm_fwd(xd, gd, bd, 1e-5)
    dX, dgamma, dbeta = cf.cf_batchnorm_bwd(xd, dyd, gd, mean, invstd)
    torch.cuda.synchronize()
    yo, mo, iso = oracle.batchnorm_fwd(x, gamma, beta, 1e-5)
    dxo, dgo, dbo = oracle.batchnorm_bwd(x, dy, gamma, mo, iso)
    assert rel_err(host64(mean), mo) <= TOL_F32
    assert rel_err(host64(invstd), iso) <= TOL_F32
    assert rel_err(host64(dgamma), dgo) <= TOL_F32
    assert rel_err(host64(dbeta), dbo) <= TOL_F32
    assert rel_err_bf16(host64(Y[0]), oracle.round_bf16(yo[0])) <= TOL_BF16
    assert rel_err_bf16(host64(dX[7]), oracle.round_bf16(dxo[7])) <= TOL_BF16
