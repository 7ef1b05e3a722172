"""ctypes binding of libcf.so (include/cf.h), one Python function per C entry
point with the same name.  Argument marshalling only: shapes are read from
torch tensors, outputs and workspaces are allocated with torch on the
tensors' device, the call goes to the library on torch's current stream, and
a non-zero status raises CfError.  Every step of the computation runs in the
library's HIP kernels; there is no other code path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcf.so")

CF_OK, CF_ERR_INVALID, CF_ERR_UNSUPPORTED, CF_ERR_WORKSPACE, CF_ERR_HIP = 0, -1, -2, -3, -4
CF_F32, CF_BF16 = 0, 1
CF_CONV_FWD, CF_CONV_BWD_DATA, CF_CONV_BWD_WEIGHT, CF_CONV_POOL_FWD, CF_POOL_CONV_BWD_WEIGHT = 0, 1, 2, 3, 4
CF_MAX_BLOCKS = 8
CF_MAX_OPT_TENSORS = 32


class CfError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s (status %d): %s" % (_status_name(status), status, msg))
        self.status = status


class cf_dims(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("d", ctypes.c_int64), ("h", ctypes.c_int64),
                ("w", ctypes.c_int64), ("c", ctypes.c_int64)]


class cf_conv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("stride", ctypes.c_int32), ("pad", ctypes.c_int32)]


class cf_model_desc(ctypes.Structure):
    _fields_ = [("nblocks", ctypes.c_int32), ("cin", ctypes.c_int32), ("d", ctypes.c_int32),
                ("h", ctypes.c_int32), ("w", ctypes.c_int32),
                ("filters", ctypes.c_int32 * CF_MAX_BLOCKS), ("dense", ctypes.c_int32 * 3),
                ("slope", ctypes.c_float)]


class cf_step_aux(ctypes.Structure):
    _fields_ = [("stream", ctypes.c_void_p), ("fork", ctypes.c_void_p * CF_MAX_BLOCKS), ("join", ctypes.c_void_p)]


class cf_adam_larc_params(ctypes.Structure):
    _fields_ = [("lr0", ctypes.c_float), ("lr_end", ctypes.c_float), ("decay_steps", ctypes.c_int64),
                ("power", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("trust", ctypes.c_float)]


CF_MAX_DENSE = 4
CF_POOL_MAX, CF_POOL_AVG, CF_POOL_NONE = 0, 1, 2
CF_OPT_SGD, CF_OPT_ADAM_LARC = 0, 1


class cf_net_desc(ctypes.Structure):
    _fields_ = [("nlayers", ctypes.c_int32), ("cin", ctypes.c_int32), ("d", ctypes.c_int32), ("h", ctypes.c_int32),
                ("w", ctypes.c_int32), ("filters", ctypes.c_int32 * CF_MAX_BLOCKS),
                ("stride", ctypes.c_int32 * CF_MAX_BLOCKS), ("pool", ctypes.c_int32 * CF_MAX_BLOCKS),
                ("batch_norm", ctypes.c_int32), ("bn_eps", ctypes.c_float), ("ndense", ctypes.c_int32),
                ("dense", ctypes.c_int32 * CF_MAX_DENSE), ("dense_bias", ctypes.c_int32), ("slope", ctypes.c_float)]


class cf_optimizer(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("lr", ctypes.c_float), ("adam", cf_adam_larc_params),
                ("t", ctypes.c_int64)]


_P = ctypes.c_void_p
_SIG = {
    "cf_abi_version": ([], ctypes.c_int32),
    "cf_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "cf_last_error": ([], ctypes.c_char_p),
    "cf_conv3d_workspace_size": ([ctypes.c_int, cf_dims, ctypes.c_int32, cf_conv, ctypes.c_int], ctypes.c_size_t),
    "cf_conv3d_fwd": ([ctypes.c_int, cf_dims, _P, _P, ctypes.c_int32, cf_conv, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "cf_conv3d_bwd_data": ([ctypes.c_int, cf_dims, _P, _P, ctypes.c_int32, cf_conv, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "cf_conv3d_bwd_weight": ([ctypes.c_int, cf_dims, _P, _P, ctypes.c_int32, cf_conv, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "cf_conv3d_bwd_weight_noalloc": ([ctypes.c_int, cf_dims, _P, _P, ctypes.c_int32, cf_conv, _P, _P], ctypes.c_int),
    "cf_conv3d_pool_fwd": ([ctypes.c_int, cf_dims, _P, _P, ctypes.c_int32, cf_conv, ctypes.c_float, _P, _P, _P,
                            ctypes.c_size_t, _P], ctypes.c_int),
    "cf_pool_conv3d_bwd_weight": ([ctypes.c_int, cf_dims, _P, _P, _P, _P, ctypes.c_int32, cf_conv, ctypes.c_float, _P,
                                   _P, ctypes.c_size_t, _P], ctypes.c_int),
    "cf_pool3d_fwd": ([ctypes.c_int, cf_dims, _P, ctypes.c_float, _P, _P, _P], ctypes.c_int),
    "cf_pool3d_bwd": ([ctypes.c_int, cf_dims, _P, _P, _P, ctypes.c_float, _P, _P], ctypes.c_int),
    "cf_avgpool3d_fwd": ([ctypes.c_int, cf_dims, _P, ctypes.c_float, _P, _P], ctypes.c_int),
    "cf_avgpool3d_bwd": ([ctypes.c_int, cf_dims, _P, _P, ctypes.c_float, _P, _P], ctypes.c_int),
    "cf_lrelu": ([ctypes.c_int, ctypes.c_int64, _P, _P, ctypes.c_float, _P, _P], ctypes.c_int),
    "cf_dense_workspace_size": ([ctypes.c_int32] * 3, ctypes.c_size_t),
    "cf_dense_fwd": ([ctypes.c_int32] * 3 + [_P, _P, _P, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "cf_dense_bwd": ([ctypes.c_int32] * 3 + [_P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P], ctypes.c_int),
    "cf_mse": ([ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P], ctypes.c_int),
    "cf_sgd": ([ctypes.c_int64, ctypes.c_float, _P, _P, _P], ctypes.c_int),
    "cf_adam_larc_workspace_size": ([ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)], ctypes.c_size_t),
    "cf_adam_larc": ([ctypes.POINTER(cf_adam_larc_params), ctypes.c_int64, ctypes.c_int32,
                      ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P),
                      ctypes.POINTER(_P), _P, _P, ctypes.c_size_t, _P], ctypes.c_int),
    "cf_batchnorm_workspace_size": ([ctypes.c_int, cf_dims], ctypes.c_size_t),
    "cf_batchnorm_fwd": ([ctypes.c_int, cf_dims, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, ctypes.c_size_t, _P],
                         ctypes.c_int),
    "cf_batchnorm_bwd": ([ctypes.c_int, cf_dims, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
                         ctypes.c_int),
    "cf_net_param_count": ([ctypes.POINTER(cf_net_desc), ctypes.POINTER(ctypes.c_int64)], ctypes.c_int32),
    "cf_net_train_step_workspace_size": ([ctypes.POINTER(cf_net_desc), ctypes.c_int, ctypes.c_int32], ctypes.c_size_t),
    "cf_net_train_step": ([ctypes.POINTER(cf_net_desc), ctypes.c_int, ctypes.c_int32, _P, _P, ctypes.POINTER(_P),
                           ctypes.POINTER(cf_optimizer), ctypes.POINTER(_P), ctypes.POINTER(_P), _P, _P, _P,
                           ctypes.c_size_t, _P], ctypes.c_int),
    "cf_train_step_workspace_size": ([ctypes.POINTER(cf_model_desc), ctypes.c_int, ctypes.c_int32], ctypes.c_size_t),
    "cf_step_aux_create": ([ctypes.POINTER(cf_step_aux)], ctypes.c_int),
    "cf_step_aux_destroy": ([ctypes.POINTER(cf_step_aux)], ctypes.c_int),
    "cf_train_step": ([ctypes.POINTER(cf_model_desc), ctypes.c_int, ctypes.c_int32, _P, _P, ctypes.POINTER(_P),
                       ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P, ctypes.POINTER(cf_step_aux)], ctypes.c_int),
}

_lib = None


def lib():
    """The loaded libcf.so.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libcf.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIG.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _status_name(s):
    return {0: "CF_OK", -1: "CF_ERR_INVALID", -2: "CF_ERR_UNSUPPORTED", -3: "CF_ERR_WORKSPACE",
            -4: "CF_ERR_HIP"}.get(s, "?")


def check(status):
    if status != CF_OK:
        raise CfError(status, lib().cf_last_error().decode())


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return CF_F32
    if t == torch.bfloat16:
        return CF_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def dims(shape) -> cf_dims:
    n, d, h, w, c = (int(v) for v in shape)
    return cf_dims(n, d, h, w, c)


CONV3 = cf_conv(3, 1, 1)


def conv_geometry(stride, size):
    """cf_conv for a 3^3 convolution of the given stride with "same" padding
    on a volume whose sizes have the parity of `size`."""
    if stride == 1:
        return CONV3
    return cf_conv(3, 2, int(size) & 1)


def out_shape(shape, cout, stride):
    n, d, h, w, _ = (int(v) for v in shape)
    if stride == 1:
        return (n, d, h, w, cout)
    return (n, (d + 1) // 2, (h + 1) // 2, (w + 1) // 2, cout)


def _ws(nbytes, device, ws=None):
    if nbytes == 0:
        return ws
    if ws is not None and ws.numel() * ws.element_size() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _wsbytes(ws):
    return 0 if ws is None else ws.numel() * ws.element_size()


# --------------------------------------------------------------------- conv
def cf_conv3d_workspace_size(dtype, xshape, cout, pass_, stride=1):
    geom = conv_geometry(stride, xshape[1])
    return int(lib().cf_conv3d_workspace_size(dtype, dims(xshape), int(cout), geom, int(pass_)))


def cf_conv3d_fwd(X, W, Y=None, ws=None, stream=None, stride=1):
    """X [N,D,H,W,Cin], W [3,3,3,Cin,Cout] (same dtype) -> Y [N,D,H,W,Cout]
    (stride 2: "same" padding, output ceil(D/2) etc.)."""
    dt = dtype_code(X.dtype)
    cout = int(W.shape[4])
    if Y is None:
        Y = torch.empty(out_shape(X.shape, cout, stride), dtype=X.dtype, device=X.device)
    ws = _ws(cf_conv3d_workspace_size(dt, X.shape, cout, CF_CONV_FWD, stride), X.device, ws)
    check(lib().cf_conv3d_fwd(dt, dims(X.shape), _ptr(X), _ptr(W), cout, conv_geometry(stride, X.shape[1]), _ptr(Y),
                              _ptr(ws), _wsbytes(ws), _stream(stream)))
    return Y


def cf_conv3d_bwd_data(dY, W, dX=None, ws=None, stream=None, xshape=None, stride=1):
    """dY [N,D,H,W,Cout], W [3,3,3,Cin,Cout] -> dX [N,D,H,W,Cin]; with
    stride 2, xshape is the forward input's shape."""
    dt = dtype_code(dY.dtype)
    cin, cout = int(W.shape[3]), int(W.shape[4])
    if xshape is None:
        xshape = tuple(dY.shape[:4]) + (cin,)
    xshape = tuple(int(v) for v in xshape)
    if dX is None:
        dX = torch.empty(xshape, dtype=dY.dtype, device=dY.device)
    ws = _ws(cf_conv3d_workspace_size(dt, xshape, cout, CF_CONV_BWD_DATA, stride), dY.device, ws)
    check(lib().cf_conv3d_bwd_data(dt, dims(xshape), _ptr(dY), _ptr(W), cout, conv_geometry(stride, xshape[1]),
                                   _ptr(dX), _ptr(ws), _wsbytes(ws), _stream(stream)))
    return dX


def cf_conv3d_bwd_weight(X, dY, dW=None, ws=None, stream=None, stride=1):
    """X [N,D,H,W,Cin], dY [N,Do,Ho,Wo,Cout] -> dW [3,3,3,Cin,Cout] fp32."""
    dt = dtype_code(X.dtype)
    cout = int(dY.shape[4])
    if dW is None:
        dW = torch.empty((3, 3, 3, int(X.shape[4]), cout), dtype=torch.float32, device=X.device)
    ws = _ws(cf_conv3d_workspace_size(dt, X.shape, cout, CF_CONV_BWD_WEIGHT, stride), X.device, ws)
    check(lib().cf_conv3d_bwd_weight(dt, dims(X.shape), _ptr(X), _ptr(dY), cout, conv_geometry(stride, X.shape[1]),
                                     _ptr(dW), _ptr(ws), _wsbytes(ws), _stream(stream)))
    return dW


def cf_conv3d_bwd_weight_noalloc(X, dY, dW, stream=None):
    """As cf_conv3d_bwd_weight, with no workspace: the library's static
    per-device scratch holds the partial sums.  dW must be given (the call
    allocates nothing)."""
    dt = dtype_code(X.dtype)
    cout = int(dY.shape[4])
    check(lib().cf_conv3d_bwd_weight_noalloc(dt, dims(X.shape), _ptr(X), _ptr(dY), cout, CONV3, _ptr(dW),
                                             _stream(stream)))
    return dW


def cf_conv3d_pool_fwd(X, W, slope, P=None, idx=None, ws=None, stream=None):
    """Fused block forward: pool(lrelu(conv(X, W))) -> (P, idx)."""
    dt = dtype_code(X.dtype)
    cout = int(W.shape[4])
    N, D, H, Wd = (int(v) for v in X.shape[:4])
    pshape = (N, D // 2, H // 2, Wd // 2, cout)
    if P is None:
        P = torch.empty(pshape, dtype=X.dtype, device=X.device)
    if idx is None:
        idx = torch.empty(pshape, dtype=torch.uint8, device=X.device)
    ws = _ws(cf_conv3d_workspace_size(dt, X.shape, cout, CF_CONV_POOL_FWD), X.device, ws)
    check(lib().cf_conv3d_pool_fwd(dt, dims(X.shape), _ptr(X), _ptr(W), cout, CONV3, float(slope), _ptr(P), _ptr(idx),
                                   _ptr(ws), _wsbytes(ws), _stream(stream)))
    return P, idx


def cf_pool_conv3d_bwd_weight(X, dP, P, idx, slope, dW=None, ws=None, stream=None):
    """Fused block weight gradient: wgrad(X, pool_bwd(dP, P, idx)) -> dW fp32."""
    dt = dtype_code(X.dtype)
    cout = int(dP.shape[4])
    if dW is None:
        dW = torch.empty((3, 3, 3, int(X.shape[4]), cout), dtype=torch.float32, device=X.device)
    ws = _ws(cf_conv3d_workspace_size(dt, X.shape, cout, CF_POOL_CONV_BWD_WEIGHT), X.device, ws)
    check(lib().cf_pool_conv3d_bwd_weight(dt, dims(X.shape), _ptr(X), _ptr(dP), _ptr(P), _ptr(idx), cout, CONV3,
                                          float(slope), _ptr(dW), _ptr(ws), _wsbytes(ws), _stream(stream)))
    return dW


# --------------------------------------------------------------------- pool
def cf_pool3d_fwd(Z, slope, P=None, idx=None, stream=None):
    """Z [N,D,H,W,C] -> (P [N,D/2,H/2,W/2,C], idx uint8)."""
    dt = dtype_code(Z.dtype)
    N, D, H, W, C = (int(v) for v in Z.shape)
    pshape = (N, D // 2, H // 2, W // 2, C)
    if P is None:
        P = torch.empty(pshape, dtype=Z.dtype, device=Z.device)
    if idx is None:
        idx = torch.empty(pshape, dtype=torch.uint8, device=Z.device)
    check(lib().cf_pool3d_fwd(dt, dims(Z.shape), _ptr(Z), float(slope), _ptr(P), _ptr(idx), _stream(stream)))
    return P, idx


def cf_pool3d_bwd(dP, P, idx, slope, dZ=None, stream=None):
    dt = dtype_code(dP.dtype)
    N, Dp, Hp, Wp, C = (int(v) for v in dP.shape)
    zshape = (N, 2 * Dp, 2 * Hp, 2 * Wp, C)
    if dZ is None:
        dZ = torch.empty(zshape, dtype=dP.dtype, device=dP.device)
    check(lib().cf_pool3d_bwd(dt, dims(zshape), _ptr(dP), _ptr(P), _ptr(idx), float(slope), _ptr(dZ),
                              _stream(stream)))
    return dZ


def cf_avgpool3d_fwd(Z, slope, P=None, stream=None):
    """Z [N,D,H,W,C] -> P [N,D/2,H/2,W/2,C] = mean over 2^3 of lrelu(Z)."""
    dt = dtype_code(Z.dtype)
    N, D, H, W, C = (int(v) for v in Z.shape)
    if P is None:
        P = torch.empty((N, D // 2, H // 2, W // 2, C), dtype=Z.dtype, device=Z.device)
    check(lib().cf_avgpool3d_fwd(dt, dims(Z.shape), _ptr(Z), float(slope), _ptr(P), _stream(stream)))
    return P


def cf_avgpool3d_bwd(dP, Z, slope, dZ=None, stream=None):
    dt = dtype_code(Z.dtype)
    if dZ is None:
        dZ = torch.empty_like(Z)
    check(lib().cf_avgpool3d_bwd(dt, dims(Z.shape), _ptr(dP), _ptr(Z), float(slope), _ptr(dZ), _stream(stream)))
    return dZ


def cf_lrelu(x, slope, dy=None, out=None, stream=None):
    dt = dtype_code(x.dtype)
    if out is None:
        out = torch.empty_like(x)
    check(lib().cf_lrelu(dt, x.numel(), _ptr(x), _ptr(dy), float(slope), _ptr(out), _stream(stream)))
    return out


# -------------------------------------------------------------------- dense
def cf_dense_fwd(X, W, b, slope, pre=None, Y=None, ws=None, stream=None):
    """X [B,in] fp32, W [in,out], b [out] or None -> (pre, Y)."""
    B, fin = (int(v) for v in X.shape)
    fout = int(W.shape[1])
    if pre is None:
        pre = torch.empty((B, fout), dtype=torch.float32, device=X.device)
    if Y is None:
        Y = torch.empty((B, fout), dtype=torch.float32, device=X.device)
    ws = _ws(int(lib().cf_dense_workspace_size(B, fin, fout)), X.device, ws)
    check(lib().cf_dense_fwd(B, fin, fout, _ptr(X), _ptr(W), _ptr(b), float(slope), _ptr(pre), _ptr(Y), _ptr(ws),
                             _wsbytes(ws), _stream(stream)))
    return pre, Y


def cf_dense_bwd(X, W, pre, dY, slope, need_dx=True, stream=None):
    B, fin = (int(v) for v in X.shape)
    fout = int(W.shape[1])
    dX = torch.empty((B, fin), dtype=torch.float32, device=X.device) if need_dx else None
    dW = torch.empty((fin, fout), dtype=torch.float32, device=X.device)
    db = torch.empty((fout,), dtype=torch.float32, device=X.device)
    check(lib().cf_dense_bwd(B, fin, fout, _ptr(X), _ptr(W), _ptr(pre), _ptr(dY), float(slope), _ptr(dX), _ptr(dW),
                             _ptr(db), _stream(stream)))
    return dX, dW, db


def cf_mse(yhat, t, stream=None):
    """-> (loss [1] device tensor, dyhat)."""
    B, K = (int(v) for v in yhat.shape)
    loss = torch.empty((1,), dtype=torch.float32, device=yhat.device)
    dy = torch.empty_like(yhat)
    check(lib().cf_mse(B, K, _ptr(yhat), _ptr(t), _ptr(loss), _ptr(dy), _stream(stream)))
    return loss, dy


def cf_sgd(W, dW, lr, stream=None):
    """In place: W -= lr * dW (fp32)."""
    check(lib().cf_sgd(W.numel(), float(lr), _ptr(W), _ptr(dW), _stream(stream)))
    return W


# -------------------------------------------------------------- train step
def model_desc(in_channels, size, filters, dense=(128, 64, 3), slope=0.3):
    """cf_model_desc for a cubic input (or size = (d, h, w))."""
    m = cf_model_desc()
    d, h, w = (size, size, size) if isinstance(size, int) else size
    m.nblocks, m.cin, m.d, m.h, m.w = len(filters), in_channels, d, h, w
    for i, f in enumerate(filters):
        m.filters[i] = f
    for i, f in enumerate(dense):
        m.dense[i] = f
    m.slope = slope
    return m


def cf_train_step_workspace_size(m, dtype, B):
    return int(lib().cf_train_step_workspace_size(ctypes.byref(m), dtype, int(B)))


class StepAux:
    """A cf_step_aux (second stream and events for cf_train_step) created on
    the current device; destroyed with the object or by close()."""

    def __init__(self):
        self.aux = cf_step_aux()
        check(lib().cf_step_aux_create(ctypes.byref(self.aux)))

    def close(self):
        if self.aux is not None:
            torch.cuda.synchronize()
            check(lib().cf_step_aux_destroy(ctypes.byref(self.aux)))
            self.aux = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def cf_train_step(m, X, targets, params, lr, ws=None, loss=None, pred=None, stream=None, aux=None):
    """One training step; `params` (fp32 masters: conv W per block, then W1,
    b1, W2, b2, W3, b3) are updated in place.  `aux`: a StepAux whose stream
    runs the weight gradients beside the rest of the backward pass, or None
    (everything on one stream).  Returns (loss, pred)."""
    dt = dtype_code(X.dtype)
    B = int(X.shape[0])
    ws = _ws(cf_train_step_workspace_size(m, dt, B), X.device, ws)
    if loss is None:
        loss = torch.empty((1,), dtype=torch.float32, device=X.device)
    arr = (_P * len(params))(*[p.data_ptr() for p in params])
    auxp = None if aux is None else ctypes.byref(aux.aux)
    check(lib().cf_train_step(ctypes.byref(m), dt, B, _ptr(X), _ptr(targets), arr, float(lr), _ptr(loss), _ptr(pred),
                              _ptr(ws), _wsbytes(ws), _stream(stream), auxp))
    return loss, pred


# ---------------------------------------------------------------- optimizer
def adam_larc_params(lr0, lr_end=None, decay_steps=1, power=1.0, beta1=0.9, beta2=0.999, eps=1e-8, trust=0.0):
    """cf_adam_larc_params; lr_end defaults to lr0 (no decay)."""
    return cf_adam_larc_params(float(lr0), float(lr0 if lr_end is None else lr_end), int(decay_steps), float(power),
                               float(beta1), float(beta2), float(eps), float(trust))


def cf_adam_larc(hp, t, params, grads, m, v, lr_out=None, ws=None, stream=None):
    """Update t (1-based) of the fp32 tensors `params` in place from `grads`,
    with Adam moments m, v (same shapes, updated in place)."""
    k = len(params)
    n = (ctypes.c_int64 * k)(*[p.numel() for p in params])
    arr = lambda ts: (_P * k)(*[q.data_ptr() for q in ts])
    ws = _ws(int(lib().cf_adam_larc_workspace_size(k, n)), params[0].device, ws)
    check(lib().cf_adam_larc(ctypes.byref(hp), int(t), k, n, arr(params), arr(grads), arr(m), arr(v), _ptr(lr_out),
                             _ptr(ws), _wsbytes(ws), _stream(stream)))


# --------------------------------------------------------------- batch norm
def cf_batchnorm_fwd(X, gamma, beta, eps, Y=None, mean=None, invstd=None, ws=None, stream=None):
    """Training-mode batch norm of NDHWC X per channel -> (Y, mean, invstd)."""
    dt = dtype_code(X.dtype)
    C = int(X.shape[4])
    Y = torch.empty_like(X) if Y is None else Y
    mean = torch.empty((C,), dtype=torch.float32, device=X.device) if mean is None else mean
    invstd = torch.empty((C,), dtype=torch.float32, device=X.device) if invstd is None else invstd
    ws = _ws(int(lib().cf_batchnorm_workspace_size(dt, dims(X.shape))), X.device, ws)
    check(lib().cf_batchnorm_fwd(dt, dims(X.shape), _ptr(X), _ptr(gamma), _ptr(beta), float(eps), _ptr(Y), _ptr(mean),
                                 _ptr(invstd), _ptr(ws), _wsbytes(ws), _stream(stream)))
    return Y, mean, invstd


def cf_batchnorm_bwd(X, dY, gamma, mean, invstd, dX=None, ws=None, stream=None):
    """-> (dX, dgamma, dbeta)."""
    dt = dtype_code(X.dtype)
    C = int(X.shape[4])
    dX = torch.empty_like(X) if dX is None else dX
    dgamma = torch.empty((C,), dtype=torch.float32, device=X.device)
    dbeta = torch.empty((C,), dtype=torch.float32, device=X.device)
    ws = _ws(int(lib().cf_batchnorm_workspace_size(dt, dims(X.shape))), X.device, ws)
    check(lib().cf_batchnorm_bwd(dt, dims(X.shape), _ptr(X), _ptr(dY), _ptr(gamma), _ptr(mean), _ptr(invstd),
                                 _ptr(dX), _ptr(dgamma), _ptr(dbeta), _ptr(ws), _wsbytes(ws), _stream(stream)))
    return dX, dgamma, dbeta


# ------------------------------------------------------ general network step
def net_desc(in_channels, size, filters, strides=None, pools=None, dense=(128, 64, 3), dense_bias=True,
             batch_norm=False, bn_eps=1e-5, slope=0.3):
    """cf_net_desc for a cubic input (or size = (d, h, w)); pools are
    CF_POOL_* values (default max after every layer)."""
    m = cf_net_desc()
    d, h, w = (size, size, size) if isinstance(size, int) else size
    m.nlayers, m.cin, m.d, m.h, m.w = len(filters), in_channels, d, h, w
    strides = strides or [1] * len(filters)
    pools = pools if pools is not None else [CF_POOL_MAX] * len(filters)
    for i, f in enumerate(filters):
        m.filters[i], m.stride[i], m.pool[i] = f, strides[i], pools[i]
    m.batch_norm, m.bn_eps = int(bool(batch_norm)), bn_eps
    m.ndense = len(dense)
    for i, f in enumerate(dense):
        m.dense[i] = f
    m.dense_bias, m.slope = int(bool(dense_bias)), slope
    return m


def cf_net_param_count(m):
    n = (ctypes.c_int64 * CF_MAX_OPT_TENSORS)()
    k = int(lib().cf_net_param_count(ctypes.byref(m), n))
    if k < 0:
        raise CfError(CF_ERR_INVALID, lib().cf_last_error().decode())
    return [int(n[i]) for i in range(k)]


def sgd_optimizer(lr):
    o = cf_optimizer()
    o.kind, o.lr = CF_OPT_SGD, float(lr)
    return o


def adam_optimizer(hp, t):
    o = cf_optimizer()
    o.kind, o.adam, o.t = CF_OPT_ADAM_LARC, hp, int(t)
    return o


def cf_net_train_step(m, X, targets, params, opt, moments=None, ws=None, loss=None, pred=None, stream=None):
    """One step of the general network; params (and Adam moments (m, v)) in
    cf_net_param_count's order, updated in place.  Returns (loss, pred)."""
    dt = dtype_code(X.dtype)
    B = int(X.shape[0])
    ws = _ws(int(lib().cf_net_train_step_workspace_size(ctypes.byref(m), dt, B)), X.device, ws)
    if loss is None:
        loss = torch.empty((1,), dtype=torch.float32, device=X.device)
    k = len(params)
    arr = lambda ts: (_P * k)(*[q.data_ptr() for q in ts])
    mp = vp = None
    if moments is not None:
        mp, vp = arr(moments[0]), arr(moments[1])
    check(lib().cf_net_train_step(ctypes.byref(m), dt, B, _ptr(X), _ptr(targets), arr(params), ctypes.byref(opt), mp,
                                  vp, _ptr(loss), _ptr(pred), _ptr(ws), _wsbytes(ws), _stream(stream)))
    return loss, pred
