"""C-ABI contract on the CPU: the library loads, exports every function that
include/cf.h declares, validates arguments before enqueuing anything (so no
GPU is needed to see the error statuses), and sizes its workspaces as
documented.  Pointers passed here are never dereferenced: every call fails
validation first."""
import ctypes
import os
import re

import pytest

from cnn_cosmology_volumes_amd import cf

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "cf.h")
FAKE = ctypes.c_void_p(0x100000)       # aligned, never dereferenced
MIS = ctypes.c_void_p(0x100008)        # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cf_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    L = cf.lib()
    names = declared_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(L, n), n
    assert L.cf_abi_version() == 2


def test_status_strings():
    L = cf.lib()
    assert L.cf_status_string(0) == b"ok"
    assert L.cf_status_string(-3) == b"workspace too small"
    assert L.cf_status_string(-4) == b"HIP error"


def conv(dt, shape, cout, X, W, Y, ws=None, wsb=0, geom=cf.CONV3, fn="cf_conv3d_fwd"):
    return getattr(cf.lib(), fn)(dt, cf.dims(shape), X, W, cout, geom, Y, ws, wsb, None)


def test_conv_validation():
    s = (1, 8, 8, 8, 32)
    assert conv(cf.CF_BF16, s, 32, None, FAKE, FAKE) == cf.CF_ERR_INVALID
    assert conv(cf.CF_BF16, s, 32, MIS, FAKE, FAKE) == cf.CF_ERR_INVALID
    assert conv(cf.CF_BF16, (1, 0, 8, 8, 32), 32, FAKE, FAKE, FAKE) == cf.CF_ERR_INVALID
    assert conv(cf.CF_BF16, s, 0, FAKE, FAKE, FAKE) == cf.CF_ERR_INVALID
    assert conv(7, s, 32, FAKE, FAKE, FAKE) == cf.CF_ERR_INVALID
    assert conv(cf.CF_BF16, s, 32, FAKE, FAKE, FAKE, geom=cf.cf_conv(5, 1, 2)) == cf.CF_ERR_UNSUPPORTED
    assert conv(cf.CF_BF16, s, 32, FAKE, FAKE, FAKE, geom=cf.cf_conv(3, 2, 1)) == cf.CF_ERR_UNSUPPORTED
    assert conv(cf.CF_BF16, s, 32, FAKE, FAKE, FAKE, FAKE, 16) == cf.CF_ERR_WORKSPACE
    assert b"workspace" in cf.lib().cf_last_error()
    for fn in ("cf_conv3d_bwd_data", "cf_conv3d_bwd_weight"):
        assert conv(cf.CF_BF16, s, 32, FAKE, FAKE, FAKE, FAKE, 16, fn=fn) == cf.CF_ERR_WORKSPACE
        assert conv(cf.CF_BF16, s, 32, FAKE, None, FAKE, fn=fn) == cf.CF_ERR_INVALID
    assert b"null" in cf.lib().cf_last_error()


def test_conv_workspace_sizes():
    # forward on MFMA: bf16 weights [27][roundup(cout,128)][cin], 256-byte aligned
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (8, 64, 64, 64, 32), 64, cf.CF_CONV_FWD) == 27 * 128 * 32 * 2
    # first layer (4 channels): [roundup(cout,128)][128]
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (8, 128, 128, 128, 4), 32, cf.CF_CONV_FWD) == 128 * 128 * 2
    # fp32 forward on the matrix cores: fp32 weights [27][roundup(cout,64)][roundup(cin,16)]
    assert cf.cf_conv3d_workspace_size(cf.CF_F32, (1, 32, 32, 32, 4), 16, cf.CF_CONV_FWD) == 27 * 64 * 16 * 4
    # the direct fp32 kernel (channels not multiples of 4) needs nothing
    assert cf.cf_conv3d_workspace_size(cf.CF_F32, (1, 32, 32, 32, 3), 16, cf.CF_CONV_FWD) == 0
    # small volume, many channels: split over in-channel chunks adds fp32 partials
    ws = cf.cf_conv3d_workspace_size(cf.CF_BF16, (8, 8, 8, 8, 256), 256, cf.CF_CONV_FWD)
    assert ws > 27 * 256 * 256 * 2 and (ws - 27 * 256 * 256 * 2) % (4096 * 256 * 4) == 0
    # backward-weight: fp32 partials, a whole number of dW copies
    ws = cf.cf_conv3d_workspace_size(cf.CF_BF16, (8, 64, 64, 64, 32), 64, cf.CF_CONV_BWD_WEIGHT)
    assert ws % (27 * 32 * 64 * 4) == 0 and ws > 0
    # the bf16 MFMA kernels address a tile's six input planes with 32-bit
    # byte offsets: planes of 4096 x 4096 x 32 bf16 (6 planes = 6.4 GB) take
    # the fp32 matrix-core kernels on bf16 data (64-bit addressing), with
    # fp32 weights [27][roundup(cout,64)][roundup(cin,16)]
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (1, 8, 4096, 4096, 32), 64, cf.CF_CONV_FWD) == 27 * 64 * 32 * 4
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (1, 8, 2048, 2048, 32), 64, cf.CF_CONV_FWD) == 27 * 128 * 32 * 2
    # backward-data: the bf16 MFMA path keeps [27][roundup(cin,128)][cout];
    # the fp32 matrix-core path [27][roundup(cin,64)][roundup(cout,16)] fp32
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (1, 8, 4096, 4096, 32), 64, cf.CF_CONV_BWD_DATA) == \
        27 * 64 * 64 * 4
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (1, 8, 1024, 1024, 32), 64, cf.CF_CONV_BWD_DATA) == \
        27 * 128 * 64 * 2
    # backward-weight addresses a box's six input planes (and four planes of
    # the output gradient) with 32-bit byte offsets too: beyond that it takes
    # the fp32 matrix-core kernel, whose partials a fp32 layer of the same
    # shape uses as well
    big = (1, 8, 2048, 2048, 32)
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, big, 64, cf.CF_CONV_BWD_WEIGHT) == \
        cf.cf_conv3d_workspace_size(cf.CF_F32, big, 64, cf.CF_CONV_BWD_WEIGHT)
    ok = (1, 8, 1024, 1024, 32)
    ws = cf.cf_conv3d_workspace_size(cf.CF_BF16, ok, 64, cf.CF_CONV_BWD_WEIGHT)
    assert ws % (27 * 32 * 64 * 4) == 0 and ws != cf.cf_conv3d_workspace_size(cf.CF_F32, ok, 64, cf.CF_CONV_BWD_WEIGHT)
    # bf16 layers with input channels a multiple of 8 but not of 32 (the
    # 16-channel layer of the Table I network) run the bf16 kernels on a copy
    # of the input padded to 32 channels: padded weights, the padded copy
    xp = 8 * 64 ** 3 * 32 * 2
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (8, 64, 64, 64, 16), 32, cf.CF_CONV_FWD) == 27 * 128 * 32 * 2 + xp
    ws = cf.cf_conv3d_workspace_size(cf.CF_BF16, (8, 64, 64, 64, 16), 32, cf.CF_CONV_BWD_WEIGHT)
    assert (ws - xp - 27 * 32 * 32 * 4) % (27 * 32 * 32 * 4) == 0 and ws > xp
    # other multiples of 4 (here 12) use the fp32 matrix cores on bf16 data
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (2, 8, 8, 8, 12), 32, cf.CF_CONV_FWD) == 27 * 64 * 16 * 4
    # bf16 channels not multiples of 4 keep the direct kernel (bf16 DHWIO as given)
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (1, 8, 8, 8, 3), 6, cf.CF_CONV_FWD) == 0
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (1, 8, 8, 8, 32), 32, cf.CF_CONV_FWD + 9) == 0
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (1, 8, 8, 8, 32), -1, cf.CF_CONV_FWD) == 0


def test_pool_and_elementwise_validation():
    L = cf.lib()
    assert L.cf_pool3d_fwd(cf.CF_BF16, cf.dims((1, 3, 4, 4, 8)), FAKE, 0.3, FAKE, FAKE, None) == cf.CF_ERR_UNSUPPORTED
    assert L.cf_pool3d_fwd(cf.CF_BF16, cf.dims((1, 4, 4, 4, 8)), None, 0.3, FAKE, FAKE, None) == cf.CF_ERR_INVALID
    assert L.cf_pool3d_fwd(cf.CF_BF16, cf.dims((1, 4, 4, 4, 8)), FAKE, float("nan"), FAKE, FAKE, None) == cf.CF_ERR_INVALID
    assert L.cf_pool3d_bwd(cf.CF_F32, cf.dims((1, 4, 4, 6, 8)), FAKE, FAKE, MIS, 0.3, FAKE, None) == cf.CF_ERR_INVALID
    assert L.cf_lrelu(cf.CF_F32, 0, FAKE, None, 0.3, FAKE, None) == cf.CF_ERR_INVALID
    assert L.cf_dense_fwd(0, 4, 4, FAKE, FAKE, None, 0.3, FAKE, FAKE, FAKE, 1 << 20, None) == cf.CF_ERR_INVALID
    assert L.cf_dense_fwd(8, 16384, 128, FAKE, FAKE, None, 0.3, FAKE, FAKE, FAKE, 0, None) == cf.CF_ERR_WORKSPACE
    assert L.cf_dense_workspace_size(8, 16384, 128) == 128 * 8 * 128 * 4
    # dense pointers must be 16-byte aligned (the kernels use 16-byte stores)
    assert L.cf_dense_fwd(8, 64, 16, FAKE, MIS, None, 0.3, FAKE, FAKE, FAKE, 1 << 20, None) == cf.CF_ERR_INVALID
    assert L.cf_dense_bwd(8, 64, 16, FAKE, FAKE, FAKE, FAKE, 0.3, None, MIS, FAKE, None) == cf.CF_ERR_INVALID
    assert L.cf_mse(0, 3, FAKE, FAKE, FAKE, None, None) == cf.CF_ERR_INVALID
    assert L.cf_sgd(10, 1e-3, None, FAKE, None) == cf.CF_ERR_INVALID


def test_train_step_validation_and_workspace():
    m = cf.model_desc(4, 128, [32, 64, 128, 256, 256])
    ws = cf.cf_train_step_workspace_size(m, cf.CF_BF16, 8)
    # the first block is fused (its 8x128^3x32 conv output is never stored);
    # the second block's conv output (bf16 8x64^3x64) is the largest buffer
    assert 8 * 64 ** 3 * 64 * 2 < ws < 8 * 128 ** 3 * 32 * 2
    # the fused first-block entry points need only weights / partial sums
    fx = (8, 128, 128, 128, 4)
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, fx, 32, cf.CF_CONV_POOL_FWD) == 128 * 128 * 2
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, fx, 32, cf.CF_POOL_CONV_BWD_WEIGHT) % (27 * 4 * 32 * 4) == 0
    # the fused kernel addresses a box by 32-bit offsets (H * W <= 2^23); a larger plane
    # takes the unfused path, which carries the full-resolution conv gradient
    big = (1, 2, 4096, 4096, 4)
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, big, 32, cf.CF_POOL_CONV_BWD_WEIGHT) >= 2 * 4096 * 4096 * 32 * 2
    edge = (1, 2, 2048, 4096, 4)
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, edge, 32, cf.CF_POOL_CONV_BWD_WEIGHT) < 2 * 2048 * 4096 * 32 * 2
    # MFMA shapes whose plan has 64/128-channel blocks on 4x4x16 tiles and no
    # channel split run fused: weights only (27 taps x 128 padded co x Cin)
    mx = (2, 16, 16, 16, 32)
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, mx, 64, cf.CF_CONV_POOL_FWD) == 27 * 128 * 32 * 2
    # a plan with a channel split pools in the reduction of its partials:
    # weights and the fp32 partials (2 splits of 2048 voxels x 64), no conv output
    sx = (1, 8, 8, 32, 64)
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, sx, 64, cf.CF_CONV_POOL_FWD) == 27 * 128 * 64 * 2 + 2 * 2048 * 64 * 4
    # unfused shapes carry the conv output through the workspace: 32 output
    # channels (512-voxel tiles), an fp32 conv
    for ux, co, dt in [((2, 16, 16, 16, 32), 32, cf.CF_BF16), ((2, 16, 16, 16, 32), 64, cf.CF_F32)]:
        zb = ux[0] * ux[1] * ux[2] * ux[3] * co * (4 if dt == cf.CF_F32 else 2)
        assert cf.cf_conv3d_workspace_size(dt, ux, co, cf.CF_CONV_POOL_FWD) >= zb
    assert cf.cf_conv3d_workspace_size(cf.CF_BF16, (1, 3, 4, 4, 4), 32, cf.CF_CONV_POOL_FWD) == 0   # odd D
    bad = cf.model_desc(4, 100, [32, 64, 128])      # 100 not divisible by 8
    assert cf.cf_train_step_workspace_size(bad, cf.CF_BF16, 8) == 0
    L = cf.lib()
    arr = (ctypes.c_void_p * 11)(*([0x100000] * 11))
    st = L.cf_train_step(ctypes.byref(bad), cf.CF_BF16, 8, FAKE, FAKE, arr, 1e-3, FAKE, None, FAKE, 1 << 40, None, None)
    assert st == cf.CF_ERR_UNSUPPORTED
    st = L.cf_train_step(ctypes.byref(m), cf.CF_BF16, 8, FAKE, FAKE, arr, 1e-3, FAKE, None, FAKE, 16, None, None)
    assert st == cf.CF_ERR_WORKSPACE
    arr[3] = None
    st = L.cf_train_step(ctypes.byref(m), cf.CF_BF16, 8, FAKE, FAKE, arr, 1e-3, FAKE, None, FAKE, 1 << 40, None, None)
    assert st == cf.CF_ERR_INVALID
    m.nblocks = 9
    assert cf.cf_train_step_workspace_size(m, cf.CF_BF16, 8) == 0


def test_negative_or_nan_slope_rejected():
    """Leaky ReLU with slope >= 0 is non-decreasing, which the pooling rule
    (lrelu of the window maximum) and its backward (sign taken from P)
    rely on; other slopes are rejected before anything is enqueued."""
    L = cf.lib()
    z = cf.dims((1, 4, 4, 4, 32))
    for slope in (-0.3, float("nan")):
        assert L.cf_pool3d_fwd(cf.CF_BF16, z, FAKE, slope, FAKE, FAKE, None) == cf.CF_ERR_INVALID
        assert L.cf_pool3d_bwd(cf.CF_BF16, z, FAKE, FAKE, FAKE, slope, FAKE, None) == cf.CF_ERR_INVALID
        assert L.cf_conv3d_pool_fwd(cf.CF_BF16, z, FAKE, FAKE, 32, cf.CONV3, slope, FAKE, FAKE, FAKE, 1 << 30,
                                    None) == cf.CF_ERR_INVALID
        assert L.cf_pool_conv3d_bwd_weight(cf.CF_BF16, cf.dims((1, 4, 4, 4, 4)), FAKE, FAKE, FAKE, FAKE, 32,
                                           cf.CONV3, slope, FAKE, FAKE, 1 << 30, None) == cf.CF_ERR_INVALID
        assert b"slope" in L.cf_last_error()
        m = cf.model_desc(4, 16, [32, 64], (32, 16, 3), slope)
        assert cf.cf_train_step_workspace_size(m, cf.CF_BF16, 2) == 0
    # slope 0 (plain ReLU) and 1 (plain max pooling) are valid
    m = cf.model_desc(4, 16, [32, 64], (32, 16, 3), 0.0)
    assert cf.cf_train_step_workspace_size(m, cf.CF_BF16, 2) > 0


def test_noalloc_rejects_oversized_partials_before_any_gpu_call():
    """cf_conv3d_bwd_weight_noalloc checks its partial sums against the
    static scratch before touching the device: a 1024 -> 1024 layer's dW
    alone (113 MB of fp32) exceeds CF_NOALLOC_SCRATCH_BYTES (64 MiB)."""
    L = cf.lib()
    st = L.cf_conv3d_bwd_weight_noalloc(cf.CF_F32, cf.dims((1, 2, 2, 2, 1024)), FAKE, FAKE, 1024, cf.CONV3, FAKE, None)
    assert st == cf.CF_ERR_WORKSPACE and b"static scratch" in L.cf_last_error()
    st = L.cf_conv3d_bwd_weight_noalloc(cf.CF_BF16, cf.dims((1, 8, 8, 8, 32)), MIS, FAKE, 32, cf.CONV3, FAKE, None)
    assert st == cf.CF_ERR_INVALID
    st = L.cf_conv3d_bwd_weight_noalloc(cf.CF_BF16, cf.dims((1, 8, 8, 8, 32)), FAKE, FAKE, 32, cf.cf_conv(3, 2, 0),
                                        FAKE, None)
    assert st == cf.CF_ERR_UNSUPPORTED


def test_train_step_aux_validation():
    """A caller-owned second stream must carry every handle; a half-filled
    cf_step_aux is rejected before anything is enqueued."""
    L = cf.lib()
    m = cf.model_desc(4, 16, [32, 64], (32, 16, 3))
    arr = (ctypes.c_void_p * 8)(*([0x100000] * 8))
    aux = cf.cf_step_aux()
    aux.stream = 0x200000
    aux.join = 0x300000
    st = L.cf_train_step(ctypes.byref(m), cf.CF_BF16, 2, FAKE, FAKE, arr, 1e-3, FAKE, None, FAKE, 1 << 40, None,
                         ctypes.byref(aux))
    assert st == cf.CF_ERR_INVALID and b"fork" in L.cf_last_error()
    for i in range(cf.CF_MAX_BLOCKS):
        aux.fork[i] = 0x400000 + 16 * i
    aux.stream = None
    st = L.cf_train_step(ctypes.byref(m), cf.CF_BF16, 2, FAKE, FAKE, arr, 1e-3, FAKE, None, FAKE, 1 << 40, None,
                         ctypes.byref(aux))
    assert st == cf.CF_ERR_INVALID
    assert L.cf_step_aux_create(None) == cf.CF_ERR_INVALID
    assert L.cf_step_aux_destroy(None) == cf.CF_OK


def test_batchnorm_rejects_nonpositive_eps():
    """A zero (or negative, NaN, infinite) epsilon is rejected before any
    GPU work: with eps = 0 a constant channel would divide by zero."""
    L = cf.lib()
    x = cf.dims((1, 4, 4, 4, 8))
    for eps in (0.0, -1e-5, float("nan"), float("inf")):
        st = L.cf_batchnorm_fwd(cf.CF_BF16, x, FAKE, FAKE, FAKE, eps, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
        assert st == cf.CF_ERR_INVALID, eps
        assert b"eps" in L.cf_last_error()
    m = cf.net_desc(4, 16, [16, 32], [1, 1], [cf.CF_POOL_MAX, cf.CF_POOL_MAX], dense=[8, 4], batch_norm=True,
                    bn_eps=0.0)
    assert L.cf_net_train_step_workspace_size(ctypes.byref(m), cf.CF_BF16, 2) == 0
    assert b"bn_eps" in L.cf_last_error()
