"""fp64 CPU oracle for the CosmoFlow-style 3D-CNN training step.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product package.  It shares no
code with the HIP path.

Each numpy-level function wraps one definition in ``oracle.c``; the network
functions at the bottom compose them in the order the method runs a step:
forward through every block [conv -> leaky ReLU -> 2^3 max pool], flatten,
three dense layers, mean squared error, then the backward pass in reverse and
one SGD update (CosmoFlow, Sec. III-A and III-B; Oyama et al., Sec. II-A SGD
equation and Sec. IV).

Storage model.  The bf16 path stores activations and activation gradients in
bfloat16 and keeps weight gradients, master weights and the dense head in
fp32.  ``storage='bf16'`` rounds the oracle's own fp64 values at those same
storage points (round to nearest, ties to even); ``'f32'`` rounds to fp32;
``'f64'`` keeps full precision.  Arithmetic between storage points is fp64.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_P = ctypes.c_void_p

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = build_oracle(force=False)
        L = ctypes.CDLL(path)
        sig = {
            "or_round_bf16": ([_dbl], _dbl),
            "or_round_bf16_array": ([_i64, _P], None),
            "or_round_f32_array": ([_i64, _P], None),
            "or_num_threads": ([], ctypes.c_int),
            "or_set_num_threads": ([ctypes.c_int], None),
            "or_conv3d_fwd": ([_i64] * 6 + [_P, _P, _P], None),
            "or_conv3d_bwd_data": ([_i64] * 6 + [_P, _P, _P], None),
            "or_conv3d_bwd_weight": ([_i64] * 6 + [_P, _P, _P], None),
            "or_conv3d_fwd_points": ([_i64] * 6 + [_P, _P, _i64, _P, _P], None),
            "or_conv3d_bwd_data_points": ([_i64] * 6 + [_P, _P, _i64, _P, _P], None),
            "or_conv3d_bwd_weight_points": ([_i64] * 6 + [_P, _P, _i64, _P, _P], None),
            "or_lrelu_fwd": ([_i64, _dbl, _P, _P], None),
            "or_lrelu_bwd": ([_i64, _dbl, _P, _P, _P], None),
            "or_lrelu_maxpool_fwd": ([_i64] * 5 + [_dbl, _P, _P, _P], None),
            "or_maxpool_lrelu_bwd": ([_i64] * 5 + [_dbl, _P, _P, _P, _P], None),
            "or_dense_fwd": ([_i64] * 3 + [_P, _P, _P, _dbl, _P, _P], None),
            "or_dense_bwd": ([_i64] * 3 + [_P, _P, _P, _P, _dbl, _P, _P, _P], None),
            "or_mse": ([_i64, _i64, _P, _P, _P], _dbl),
            "or_sgd": ([_i64, _dbl, _P, _P], None),
            "or_conv3d_fwd_s": ([_i64] * 11 + [_P, _P, _P], None),
            "or_conv3d_bwd_data_s": ([_i64] * 11 + [_P, _P, _P], None),
            "or_conv3d_bwd_weight_s": ([_i64] * 11 + [_P, _P, _P], None),
            "or_avgpool_fwd": ([_i64] * 5 + [_P, _P], None),
            "or_avgpool_bwd": ([_i64] * 5 + [_P, _P], None),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def num_threads() -> int:
    return int(lib().or_num_threads())


def set_num_threads(n: int) -> None:
    lib().or_set_num_threads(int(n))


# ----------------------------------------------------------------- rounding
def round_bf16(x):
    """Round every element to the nearest bfloat16 value, ties to even."""
    y = np.array(x, dtype=np.float64, copy=True, order="C")
    lib().or_round_bf16_array(y.size, _ptr(y))
    return y


def round_f32(x):
    y = np.array(x, dtype=np.float64, copy=True, order="C")
    lib().or_round_f32_array(y.size, _ptr(y))
    return y


def store(x, storage: str):
    """Model a storage point of the given precision ('f64', 'f32', 'bf16')."""
    if storage == "bf16":
        return round_bf16(x)
    if storage == "f32":
        return round_f32(x)
    if storage == "f64":
        return _f64(x)
    raise ValueError(storage)


# --------------------------------------------------------------------- conv
def conv3d_fwd(x, w):
    """x [N,D,H,W,Ci], w [3,3,3,Ci,Co] -> y [N,D,H,W,Co] (3^3, stride 1, pad 1)."""
    x, w = _f64(x), _f64(w)
    N, D, H, W, Ci = x.shape
    assert w.shape[:4] == (3, 3, 3, Ci), w.shape
    Co = w.shape[4]
    y = np.empty((N, D, H, W, Co), np.float64)
    lib().or_conv3d_fwd(N, D, H, W, Ci, Co, _ptr(x), _ptr(w), _ptr(y))
    return y


def conv3d_bwd_data(dy, w):
    """dy [N,D,H,W,Co], w [3,3,3,Ci,Co] -> dx [N,D,H,W,Ci]."""
    dy, w = _f64(dy), _f64(w)
    N, D, H, W, Co = dy.shape
    Ci = w.shape[3]
    assert w.shape == (3, 3, 3, Ci, Co), w.shape
    dx = np.empty((N, D, H, W, Ci), np.float64)
    lib().or_conv3d_bwd_data(N, D, H, W, Ci, Co, _ptr(dy), _ptr(w), _ptr(dx))
    return dx


def conv3d_bwd_weight(x, dy):
    """x [N,D,H,W,Ci], dy [N,D,H,W,Co] -> dw [3,3,3,Ci,Co]."""
    x, dy = _f64(x), _f64(dy)
    N, D, H, W, Ci = x.shape
    Co = dy.shape[4]
    assert dy.shape[:4] == x.shape[:4]
    dw = np.empty((3, 3, 3, Ci, Co), np.float64)
    lib().or_conv3d_bwd_weight(N, D, H, W, Ci, Co, _ptr(x), _ptr(dy), _ptr(dw))
    return dw


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def conv3d_fwd_points(x32, w32, pts):
    """Forward conv evaluated at flat output indices ``pts`` of y [N,D,H,W,Co].

    x32 and w32 are float32 arrays of exactly representable inputs; the sums
    are fp64."""
    x32, w32 = _f32(x32), _f32(w32)
    pts = np.ascontiguousarray(pts, dtype=np.int64)
    N, D, H, W, Ci = x32.shape
    Co = w32.shape[4]
    out = np.empty(pts.size, np.float64)
    lib().or_conv3d_fwd_points(N, D, H, W, Ci, Co, _ptr(x32), _ptr(w32), pts.size, _ptr(pts), _ptr(out))
    return out


def conv3d_bwd_data_points(dy32, w32, pts):
    """Backward-data evaluated at flat indices ``pts`` of dx [N,D,H,W,Ci]."""
    dy32, w32 = _f32(dy32), _f32(w32)
    pts = np.ascontiguousarray(pts, dtype=np.int64)
    N, D, H, W, Co = dy32.shape
    Ci = w32.shape[3]
    out = np.empty(pts.size, np.float64)
    lib().or_conv3d_bwd_data_points(N, D, H, W, Ci, Co, _ptr(dy32), _ptr(w32), pts.size, _ptr(pts), _ptr(out))
    return out


def conv3d_bwd_weight_points(x32, dy32, pts):
    """Backward-weight evaluated at flat indices ``pts`` of dw [3,3,3,Ci,Co]."""
    x32, dy32 = _f32(x32), _f32(dy32)
    pts = np.ascontiguousarray(pts, dtype=np.int64)
    N, D, H, W, Ci = x32.shape
    Co = dy32.shape[4]
    out = np.empty(pts.size, np.float64)
    lib().or_conv3d_bwd_weight_points(N, D, H, W, Ci, Co, _ptr(x32), _ptr(dy32), pts.size, _ptr(pts), _ptr(out))
    return out


# ------------------------------------------------ strided "same" conv
def same_geometry(size, stride, k=3):
    """TensorFlow's "same" padding (the padding of every layer in Oyama et
    al., Table I) for one dimension: output ceil(size / stride), total
    padding max((out - 1) * stride + k - size, 0), of which the low side
    gets the floor of half.  Returns (out, pad_low)."""
    out = -(-size // stride)
    total = max((out - 1) * stride + k - size, 0)
    return out, total // 2


def conv3d_fwd_s(x, w, stride):
    """x [N,D,H,W,Ci], w [3,3,3,Ci,Co] -> y [N,Do,Ho,Wo,Co], 3^3 kernel,
    given stride, "same" padding (same_geometry; cubic volumes)."""
    x, w = _f64(x), _f64(w)
    N, D, H, W, Ci = x.shape
    assert D == H == W
    Co = w.shape[4]
    o, p = same_geometry(D, stride)
    y = np.empty((N, o, o, o, Co), np.float64)
    lib().or_conv3d_fwd_s(N, D, H, W, Ci, Co, stride, p, o, o, o, _ptr(x), _ptr(w), _ptr(y))
    return y


def conv3d_bwd_data_s(dy, w, stride, in_size):
    dy, w = _f64(dy), _f64(w)
    N, o, _, _, Co = dy.shape
    Ci = w.shape[3]
    o2, p = same_geometry(in_size, stride)
    assert o2 == o
    dx = np.empty((N, in_size, in_size, in_size, Ci), np.float64)
    lib().or_conv3d_bwd_data_s(N, in_size, in_size, in_size, Ci, Co, stride, p, o, o, o, _ptr(dy), _ptr(w), _ptr(dx))
    return dx


def conv3d_bwd_weight_s(x, dy, stride):
    x, dy = _f64(x), _f64(dy)
    N, D, H, W, Ci = x.shape
    Co = dy.shape[4]
    o, p = same_geometry(D, stride)
    assert dy.shape[1:4] == (o, o, o)
    dw = np.empty((3, 3, 3, Ci, Co), np.float64)
    lib().or_conv3d_bwd_weight_s(N, D, H, W, Ci, Co, stride, p, o, o, o, _ptr(x), _ptr(dy), _ptr(dw))
    return dw


# ------------------------------------------------------------ average pool
def avgpool_fwd(z):
    """2^3 stride-2 average pool, weights 1/8: z [N,D,H,W,C] -> [N,D/2,H/2,W/2,C]."""
    z = _f64(z)
    N, D, H, W, C = z.shape
    assert D % 2 == 0 and H % 2 == 0 and W % 2 == 0
    p = np.empty((N, D // 2, H // 2, W // 2, C), np.float64)
    lib().or_avgpool_fwd(N, D, H, W, C, _ptr(z), _ptr(p))
    return p


def avgpool_bwd(dp):
    dp = _f64(dp)
    N, Dp, Hp, Wp, C = dp.shape
    dz = np.empty((N, 2 * Dp, 2 * Hp, 2 * Wp, C), np.float64)
    lib().or_avgpool_bwd(N, 2 * Dp, 2 * Hp, 2 * Wp, C, _ptr(dp), _ptr(dz))
    return dz


# ------------------------------------------------------------- activations
def lrelu_fwd(x, slope):
    x = _f64(x)
    y = np.empty_like(x)
    lib().or_lrelu_fwd(x.size, float(slope), _ptr(x), _ptr(y))
    return y


def lrelu_bwd(x, dy, slope):
    x, dy = _f64(x), _f64(dy)
    dx = np.empty_like(x)
    lib().or_lrelu_bwd(x.size, float(slope), _ptr(x), _ptr(dy), _ptr(dx))
    return dx


def lrelu_maxpool_fwd(z, slope):
    """z [N,D,H,W,C] (D,H,W even) -> (p [N,D/2,H/2,W/2,C], idx uint8 same shape)."""
    z = _f64(z)
    N, D, H, W, C = z.shape
    assert D % 2 == 0 and H % 2 == 0 and W % 2 == 0
    p = np.empty((N, D // 2, H // 2, W // 2, C), np.float64)
    idx = np.empty(p.shape, np.uint8)
    lib().or_lrelu_maxpool_fwd(N, D, H, W, C, float(slope), _ptr(z), _ptr(p), _ptr(idx))
    return p, idx


def maxpool_lrelu_bwd(dp, p, idx, slope):
    """-> dz [N,2Dp,2Hp,2Wp,C]."""
    dp, p = _f64(dp), _f64(p)
    idx = np.ascontiguousarray(idx, dtype=np.uint8)
    N, Dp, Hp, Wp, C = dp.shape
    dz = np.empty((N, 2 * Dp, 2 * Hp, 2 * Wp, C), np.float64)
    lib().or_maxpool_lrelu_bwd(N, 2 * Dp, 2 * Hp, 2 * Wp, C, float(slope), _ptr(dp), _ptr(p), _ptr(idx), _ptr(dz))
    return dz


# -------------------------------------------------------------------- dense
def dense_fwd(x, w, b, slope):
    """x [B,In], w [In,Out], b [Out]; slope < 0 means a linear layer."""
    x, w = _f64(x), _f64(w)
    b = _f64(b) if b is not None else None
    B, In = x.shape
    Out = w.shape[1]
    pre = np.empty((B, Out), np.float64)
    y = np.empty((B, Out), np.float64)
    lib().or_dense_fwd(B, In, Out, _ptr(x), _ptr(w), _ptr(b), float(slope), _ptr(pre), _ptr(y))
    return pre, y


def dense_bwd(x, w, pre, dy, slope, need_dx=True):
    x, w, pre, dy = _f64(x), _f64(w), _f64(pre), _f64(dy)
    B, In = x.shape
    Out = w.shape[1]
    dx = np.empty((B, In), np.float64) if need_dx else None
    dw = np.empty((In, Out), np.float64)
    db = np.empty((Out,), np.float64)
    lib().or_dense_bwd(B, In, Out, _ptr(x), _ptr(w), _ptr(pre), _ptr(dy), float(slope), _ptr(dx), _ptr(dw), _ptr(db))
    return dx, dw, db


def mse(yhat, t):
    """-> (loss, dyhat) with loss = mean over all B*K entries."""
    yhat, t = _f64(yhat), _f64(t)
    B, K = yhat.shape
    d = np.empty_like(yhat)
    loss = lib().or_mse(B, K, _ptr(yhat), _ptr(t), _ptr(d))
    return float(loss), d


def sgd(w, dw, lr):
    """Returns W - lr * dW (a new array)."""
    w2 = np.array(w, dtype=np.float64, copy=True, order="C")
    dw = _f64(dw)
    lib().or_sgd(w2.size, float(lr), _ptr(w2), _ptr(dw))
    return w2


# ------------------------------------------------------------------ network
def _perturbed(a, perturb):
    """The conditioning probe: a * (1 + r u), u ~ U(-1, 1) from the probe's
    generator (perturb = (Generator, r)); a unchanged when perturb is None."""
    if perturb is None:
        return a
    g, r = perturb
    return a * (1.0 + r * g.uniform(-1.0, 1.0, np.shape(a)))


def network_forward(x, conv_w, dense_w, slope, storage="f64", trace=None, perturb=None):
    """Forward pass of the conv stack and the dense head.

    x [B,D,H,W,Cin]; conv_w list of [3,3,3,Ci,Co]; dense_w list of three
    (W [In,Out], b [Out]).  Returns (yhat, cache).  If ``trace`` is a dict,
    each block's stored conv output is appended to trace["z"].

    ``perturb`` = (numpy Generator, r) is a conditioning probe, not part of
    the method: every matrix-product result (conv sums, dense pre-activations;
    in network_backward the dense and conv input gradients) is multiplied by
    (1 + r u), u ~ U(-1, 1), before its storage rounding, as an fp32
    accumulation error of relative size r would move it.  Comparing a
    perturbed run with an unperturbed one shows how far the step's results
    are determined by the arithmetic at all."""
    a = store(x, storage)
    blocks = []
    for w in conv_w:
        z = store(_perturbed(conv3d_fwd(a, w), perturb), storage)
        if trace is not None:
            trace.setdefault("z", []).append(z)
        p, idx = lrelu_maxpool_fwd(z, slope)
        p = store(p, storage)
        blocks.append(dict(x=a, p=p, idx=idx))
        a = p
    B = a.shape[0]
    h = a.reshape(B, -1)
    dense = []
    for li, (W, b) in enumerate(dense_w):
        s = slope if li < len(dense_w) - 1 else -1.0
        pre, _ = dense_fwd(h, W, b, s)
        pre = _perturbed(pre, perturb)
        y = lrelu_fwd(pre, s) if s >= 0 else pre
        dense.append(dict(x=h, pre=pre, slope=s))
        h = y
    return h, dict(blocks=blocks, dense=dense, last_shape=a.shape)


def network_backward(cache, conv_w, dense_w, dyhat, slope, storage="f64", first_dgrad=False, trace=None,
                     perturb=None):
    """Backward pass; returns (conv_dw list, dense grads list of (dW, db)).
    If ``trace`` is a dict, the stored pooled gradient and conv-output
    gradient of each block are recorded in trace["dp"][l] and trace["dz"][l].
    ``perturb``: the conditioning probe of network_forward."""
    g = dyhat
    dense_g = [None] * len(dense_w)
    for li in reversed(range(len(dense_w))):
        c = cache["dense"][li]
        dx, dw, db = dense_bwd(c["x"], dense_w[li][0], c["pre"], g, c["slope"], need_dx=True)
        dense_g[li] = (dw, db)
        g = _perturbed(dx, perturb)
    dp = store(g.reshape(cache["last_shape"]), storage)
    conv_g = [None] * len(conv_w)
    if trace is not None:
        trace["dp"] = [None] * len(conv_w)
        trace["dz"] = [None] * len(conv_w)
    for l in reversed(range(len(conv_w))):
        blk = cache["blocks"][l]
        dz = store(maxpool_lrelu_bwd(dp, blk["p"], blk["idx"], slope), storage)
        if trace is not None:
            trace["dp"][l] = dp
            trace["dz"][l] = dz
        conv_g[l] = conv3d_bwd_weight(blk["x"], dz)
        if l > 0 or first_dgrad:
            dp = store(_perturbed(conv3d_bwd_data(dz, conv_w[l]), perturb), storage)
    return conv_g, dense_g


def train_step(x, targets, conv_w32, dense_w32, lr, slope, storage="f64", trace=None, perturb=None):
    """One full step.  Weights used in the passes are the masters rounded to
    the storage precision (bf16 for the conv weights of the bf16 path); the
    update is applied to the fp32/fp64 masters.  ``trace``: as for
    network_forward / network_backward, plus trace["conv_w"], the conv
    weights the passes used.  ``perturb``: as for network_forward.

    Returns dict(loss, yhat, conv_w, dense_w, conv_dw, dense_g)."""
    conv_use = [store(w, storage) for w in conv_w32]
    if trace is not None:
        trace["conv_w"] = conv_use
    dense_use = [(_f64(W), _f64(b)) for W, b in dense_w32]
    yhat, cache = network_forward(x, conv_use, dense_use, slope, storage, trace=trace, perturb=perturb)
    loss, dy = mse(yhat, targets)
    conv_g, dense_g = network_backward(cache, conv_use, dense_use, dy, slope, storage, trace=trace, perturb=perturb)
    master = "f64" if storage == "f64" else "f32"
    new_conv = [store(sgd(w, g, lr), master) for w, g in zip(conv_w32, conv_g)]
    new_dense = [(store(sgd(W, dW, lr), master), store(sgd(b, db, lr), master))
                 for (W, b), (dW, db) in zip(dense_w32, dense_g)]
    return dict(loss=loss, yhat=yhat, conv_w=new_conv, dense_w=new_dense,
                conv_dw=conv_g, dense_g=dense_g)


# ------------------------------------------------------ Adam + LARC + decay
def poly_decay(lr0, lr_end, decay_steps, power, step):
    """Polynomial learning-rate decay (CosmoFlow, Sec. III-B: power 1, i.e.
    linear; Oyama et al., Sec. IV: linear decay to 0.01x of the initial
    rate): the rate after ``step`` completed updates,
        (lr0 - lr_end) * (1 - min(step, T) / T) ** power + lr_end."""
    s = min(float(step), float(decay_steps))
    return (lr0 - lr_end) * (1.0 - s / float(decay_steps)) ** power + lr_end


def adam_larc_step(w, g, m, v, t, lr, beta1, beta2, eps, trust):
    """One Adam update with LARC's layer-wise clipping, for one parameter
    tensor (one "layer"), in fp64.

    Adam (Kingma and Ba; the optimizer of CosmoFlow Sec. III-B and Oyama et
    al. Sec. IV, beta1 0.9, beta2 0.999, eps 1e-8):
        m <- beta1 m + (1 - beta1) g;   v <- beta2 v + (1 - beta2) g^2
        u = (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
    LARC (CosmoFlow Sec. III-B: the rate is scaled by the layer's weight
    norm and clipped at Adam's nominal rate): the tensor's rate is
        lr_l = min(lr, trust * ||w|| / ||g||),
    or lr itself when trust <= 0 or either norm is zero.  Then w <- w - lr_l u.
    t is the 1-based update count.  Returns (w, m, v, lr_l) as new arrays."""
    w, g, m, v = _f64(w), _f64(g), _f64(m), _f64(v)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    u = mhat / (np.sqrt(vhat) + eps)
    wn = float(np.sqrt(np.sum(w * w)))
    gn = float(np.sqrt(np.sum(g * g)))
    lr_l = lr
    if trust > 0.0 and wn > 0.0 and gn > 0.0:
        lr_l = min(lr, trust * wn / gn)
    return w - lr_l * u, m, v, lr_l


# --------------------------------------------------------------- batch norm
def batchnorm_fwd(x, gamma, beta, eps):
    """Training-mode batch normalisation of NDHWC x over (N, D, H, W) per
    channel (Oyama et al., Sec. IV: a batch-normalisation layer after every
    convolution; Sec. III: its statistics are each channel's sum and sum of
    squares): mean = sum / M, var = sumsq / M - mean^2 (biased),
    xhat = (x - mean) / sqrt(var + eps), y = gamma xhat + beta.
    Returns (y, mean, invstd)."""
    x = _f64(x)
    C = x.shape[-1]
    flat = x.reshape(-1, C)
    M = flat.shape[0]
    mean = np.sum(flat, axis=0) / M
    var = np.sum(flat * flat, axis=0) / M - mean * mean
    invstd = 1.0 / np.sqrt(var + eps)
    y = (flat - mean) * invstd * _f64(gamma) + _f64(beta)
    return y.reshape(x.shape), mean, invstd


def batchnorm_bwd(x, dy, gamma, mean, invstd):
    """Backward of batchnorm_fwd (chain rule through the batch statistics):
        dbeta = sum dy;  dgamma = sum dy xhat
        dx = gamma invstd (dy - dbeta / M - xhat dgamma / M).
    Returns (dx, dgamma, dbeta)."""
    x, dy = _f64(x), _f64(dy)
    C = x.shape[-1]
    fx, fd = x.reshape(-1, C), dy.reshape(-1, C)
    M = fx.shape[0]
    xhat = (fx - mean) * invstd
    dbeta = np.sum(fd, axis=0)
    dgamma = np.sum(fd * xhat, axis=0)
    dx = _f64(gamma) * invstd * (fd - dbeta / M - xhat * dgamma / M)
    return dx.reshape(x.shape), dgamma, dbeta


# ------------------------------------------------- general network step
def net_param_shapes(cin, layers, dense, batch_norm, dense_bias, in_size):
    """Parameter shapes in the order the step takes them: per conv layer W
    [3,3,3,cin,f] (then gamma [f], beta [f] with batch norm); per dense layer
    W [in,out] (then b [out] with biases).  layers: (filters, stride, pool)
    with pool in {"max", "avg", "none"}; cubic input of width in_size."""
    shapes, c, s = [], cin, in_size
    for f, stride, pool in layers:
        shapes.append((3, 3, 3, c, f))
        if batch_norm:
            shapes += [(f,), (f,)]
        s = same_geometry(s, stride)[0]
        if pool != "none":
            s //= 2
        c = f
    fan = s ** 3 * c
    for o in dense:
        shapes.append((fan, o))
        if dense_bias:
            shapes.append((o,))
        fan = o
    return shapes


def net_train_step(x, targets, params, layers, dense, slope, batch_norm=False, bn_eps=1e-5, dense_bias=True,
                   storage="f64", opt=("sgd", 1e-3), adam_state=None, perturb=None):
    """One training step of a general conv network (the extended CosmoFlow
    network of Oyama et al., Table I and Sec. IV, and the benchmark network
    alike): per layer a 3^3 "same" conv of the given stride without bias,
    batch normalisation (optional), leaky ReLU and max / average / no
    pooling; flatten; dense layers (leaky ReLU but on the last; optional
    biases); MSE; backward; the update.

    Storage points (rounded to ``storage``): the input, each conv output,
    batch-norm output, layer output and their gradients; conv weights are
    the masters rounded to ``storage``.  opt: ("sgd", lr) or ("adam", lr_t,
    beta1, beta2, eps, trust, t) with adam_state = (m list, v list).
    perturb: the conditioning probe of network_forward (every matrix-product
    result scaled by 1 + r u before its storage rounding).
    Returns dict(loss, yhat, grads, params, adam_state)."""
    L = len(layers)
    per = 3 if batch_norm else 1
    conv_w = [params[l * per] for l in range(L)]
    gam = [params[l * per + 1] for l in range(L)] if batch_norm else None
    bet = [params[l * per + 2] for l in range(L)] if batch_norm else None
    dp_ = 2 if dense_bias else 1
    dw0 = L * per
    dW = [_f64(params[dw0 + k * dp_]) for k in range(len(dense))]
    db = [_f64(params[dw0 + k * dp_ + 1]) if dense_bias else np.zeros(dense[k]) for k in range(len(dense))]
    wuse = [store(w, storage) for w in conv_w]

    def conv(a, w, s):
        return conv3d_fwd(a, w) if s == 1 else conv3d_fwd_s(a, w, s)

    a = store(x, storage)
    cache = []
    for l, (f, s, pool) in enumerate(layers):
        z = store(_perturbed(conv(a, wuse[l], s), perturb), storage)
        y, mean, invstd = z, None, None
        if batch_norm:
            y, mean, invstd = batchnorm_fwd(z, gam[l], bet[l], bn_eps)
            y = store(y, storage)
        idx = None
        if pool == "max":
            out, idx = lrelu_maxpool_fwd(y, slope)
        elif pool == "avg":
            out = avgpool_fwd(lrelu_fwd(y, slope))
        else:
            out = lrelu_fwd(y, slope)
        out = store(out, storage)
        cache.append(dict(x=a, z=z, y=y, out=out, idx=idx, mean=mean, invstd=invstd, s=s))
        a = out
    B = a.shape[0]
    h = a.reshape(B, -1)
    dcache = []
    for k in range(len(dense)):
        sk = slope if k + 1 < len(dense) else -1.0
        pre, _ = dense_fwd(h, dW[k], db[k], sk)
        pre = _perturbed(pre, perturb)
        yk = lrelu_fwd(pre, sk) if sk >= 0 else pre
        dcache.append((h, pre, sk))
        h = yk
    loss, g = mse(h, targets)
    grads = [None] * len(params)
    for k in reversed(range(len(dense))):
        hin, pre, sk = dcache[k]
        g, gw, gb = dense_bwd(hin, dW[k], pre, g, sk, need_dx=True)
        g = _perturbed(g, perturb)
        grads[dw0 + k * dp_] = gw
        if dense_bias:
            grads[dw0 + k * dp_ + 1] = gb
    dA = store(g.reshape(a.shape), storage)
    for l in reversed(range(L)):
        c = cache[l]
        pool = layers[l][2]
        if pool == "max":
            dy = maxpool_lrelu_bwd(dA, c["out"], c["idx"], slope)
        elif pool == "avg":
            dy = lrelu_bwd(c["y"], avgpool_bwd(dA), slope)
        else:
            dy = lrelu_bwd(c["y"], dA, slope)
        dy = store(dy, storage)
        dz = dy
        if batch_norm:
            dz, gg, gb = batchnorm_bwd(c["z"], dy, gam[l], c["mean"], c["invstd"])
            dz = store(dz, storage)
            grads[l * per + 1], grads[l * per + 2] = gg, gb
        s = c["s"]
        grads[l * per] = conv3d_bwd_weight(c["x"], dz) if s == 1 else conv3d_bwd_weight_s(c["x"], dz, s)
        if l > 0:
            size = c["x"].shape[1]
            dA = conv3d_bwd_data(dz, wuse[l]) if s == 1 else conv3d_bwd_data_s(dz, wuse[l], s, size)
            dA = store(_perturbed(dA, perturb), storage)
    master = "f64" if storage == "f64" else "f32"
    if opt[0] == "sgd":
        new = [store(sgd(p, gr, opt[1]), master) for p, gr in zip(params, grads)]
        state = None
    else:
        _, lr_t, b1, b2, eps, trust, t = opt
        ms, vs = adam_state
        new, nm, nv = [], [], []
        for p, gr, m_, v_ in zip(params, grads, ms, vs):
            w_, m2, v2, _ = adam_larc_step(p, gr, m_, v_, t, lr_t, b1, b2, eps, trust)
            new.append(store(w_, master))
            nm.append(m2)
            nv.append(v2)
        state = (nm, nv)
    return dict(loss=loss, yhat=h, grads=grads, params=new, adam_state=state)
