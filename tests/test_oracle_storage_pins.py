"""Pins of the oracle's storage model: where the bf16 path rounds.

The bf16 path stores the conv weights, each block's conv output Z, pooled
output P, pooled gradient dP and conv-output gradient dZ in bfloat16 (round
to nearest, ties to even).  Each hand case below is built so that the exact
fp64 value at one storage point is not a bf16 number and moving (or
dropping) that one rounding changes a result the test states by hand; the
expected numbers are worked out in the comments, not computed by the oracle.
The fp32 rounding used by the fp32 path's storage model is pinned against
numpy's float64 -> float32 conversion (round to nearest even)."""
import numpy as np

import oracle

SLOPE = 0.3
CENTER = (1, 1, 1)


def delta_weights(taps, cin=1, cout=1):
    """DHWIO weights, zero except the listed {(kd,kh,kw): value} taps (ci = co = 0)."""
    w = np.zeros((3, 3, 3, cin, cout))
    for t, v in taps.items():
        w[t + (0, 0)] = v
    return w


def linear_head():
    """Three 1 -> 1 dense layers with unit weight and zero bias."""
    return [(np.ones((1, 1)), np.zeros(1)) for _ in range(3)]


def linear_cache(blocks, last_shape):
    """A forward cache whose dense head passes the output gradient through
    unchanged: unit weights, no activation (slope < 0 means linear)."""
    dense = [dict(x=np.ones((1, 1)), pre=np.ones((1, 1)), slope=-1.0) for _ in range(3)]
    return dict(blocks=blocks, dense=dense, last_shape=last_shape)


def test_conv_output_rounding_decides_the_pool_index():
    # Z[d,h,w] = X[d,h,w] + X[d,h,w-1] (centre tap and the kw = 0 tap, both 1).
    # X[0,0,0] = 1, X[0,0,1] = 2^-10: window position 0 holds Z = 1, position 1
    # holds Z = 1 + 2^-10, the other six hold 0.  Rounded to bf16 (8
    # significant bits) 1 + 2^-10 becomes 1, so the two tie and the first
    # position wins: idx 0, P = 1.  Unrounded, position 1 is the maximum.
    x = np.zeros((1, 2, 2, 2, 1))
    x[0, 0, 0, 0, 0] = 1.0
    x[0, 0, 0, 1, 0] = 2.0 ** -10
    w = delta_weights({CENTER: 1.0, (1, 1, 0): 1.0})
    _, cache = oracle.network_forward(x, [w], linear_head(), SLOPE, "bf16")
    assert cache["blocks"][0]["idx"].ravel().tolist() == [0]
    assert cache["blocks"][0]["p"].ravel().tolist() == [1.0]
    _, cache64 = oracle.network_forward(x, [w], linear_head(), SLOPE, "f64")
    assert cache64["blocks"][0]["idx"].ravel().tolist() == [1]
    assert cache64["blocks"][0]["p"].ravel().tolist() == [1.0 + 2.0 ** -10]
    # The weight gradient follows the window position: with dP = 1 and P > 0,
    # dZ = 1 at (0,0,0), so dW[t] = X[(0,0,0) + t - 1]: the centre tap sees
    # X[0,0,0] = 1 and the kw = 2 tap sees X[0,0,1] = 2^-10.
    dyhat = np.ones((1, 1))
    gw, _ = oracle.network_backward(cache, [w], linear_head(), dyhat, SLOPE, "bf16")
    expect = np.zeros((3, 3, 3, 1, 1))
    expect[1, 1, 1, 0, 0] = 1.0
    expect[1, 1, 2, 0, 0] = 2.0 ** -10
    assert np.array_equal(gw[0], expect)
    gw64, _ = oracle.network_backward(cache64, [w], linear_head(), dyhat, SLOPE, "f64")
    expect64 = np.zeros((3, 3, 3, 1, 1))
    expect64[1, 1, 1, 0, 0] = 2.0 ** -10     # dZ at (0,0,1) sees X[0,0,1]
    expect64[1, 1, 0, 0, 0] = 1.0            # and X[0,0,0] through the kw = 0 tap
    assert np.array_equal(gw64[0], expect64)


def test_conv_output_gradient_is_rounded_after_the_slope():
    # P < 0, so the pooled gradient 1 is scaled by the slope 0.3 before it is
    # stored as dZ.  0.3 = 1.2 * 2^-2 has the 8-bit significand 1.2 * 128 =
    # 153.6 -> 154, so bf16 dZ = 154/128 * 2^-2 = 0.30078125.  With X[0,0,0]
    # = 1 and dZ non-zero only at (0,0,0), dW at the centre tap is dZ itself.
    x = np.zeros((1, 2, 2, 2, 1))
    x[0, 0, 0, 0, 0] = 1.0
    blk = dict(x=x, p=np.full((1, 1, 1, 1, 1), -0.5), idx=np.zeros((1, 1, 1, 1, 1), np.uint8))
    cache = linear_cache([blk], (1, 1, 1, 1, 1))
    w = delta_weights({CENTER: 1.0})
    trace = {}
    gw, _ = oracle.network_backward(cache, [w], linear_head(), np.ones((1, 1)), SLOPE, "bf16", trace=trace)
    assert gw[0][1, 1, 1, 0, 0] == 0.30078125
    assert trace["dz"][0][0, 0, 0, 0, 0] == 0.30078125
    gw64, _ = oracle.network_backward(cache, [w], linear_head(), np.ones((1, 1)), SLOPE, "f64")
    assert gw64[0][1, 1, 1, 0, 0] == 0.3


def test_head_gradient_is_rounded_into_the_last_pooled_gradient():
    # The dense head's input gradient becomes the last block's pooled
    # gradient dP, a bf16 storage point: 1 + 2^-10 is stored as 1.  With
    # P > 0 and X[0,0,0] = 1, dW at the centre tap is that dP.
    x = np.zeros((1, 2, 2, 2, 1))
    x[0, 0, 0, 0, 0] = 1.0
    blk = dict(x=x, p=np.ones((1, 1, 1, 1, 1)), idx=np.zeros((1, 1, 1, 1, 1), np.uint8))
    cache = linear_cache([blk], (1, 1, 1, 1, 1))
    w = delta_weights({CENTER: 1.0})
    dyhat = np.full((1, 1), 1.0 + 2.0 ** -10)
    gw, _ = oracle.network_backward(cache, [w], linear_head(), dyhat, SLOPE, "bf16")
    assert gw[0][1, 1, 1, 0, 0] == 1.0
    gw64, _ = oracle.network_backward(cache, [w], linear_head(), dyhat, SLOPE, "f64")
    assert gw64[0][1, 1, 1, 0, 0] == 1.0 + 2.0 ** -10


def test_backward_data_output_is_rounded_into_the_previous_pooled_gradient():
    # Two blocks.  Block 2's conv weight is 1 + 2^-10 at the centre tap (given
    # to the backward pass as is).  dP2 = 1 and P2 > 0 put dZ2 = 1 at (0,0,0);
    # backward-data gives block 1's pooled gradient dP1 = 1 + 2^-10 there (0
    # elsewhere), stored in bf16 as 1.  P1 > 0, idx1 = 0 and X1[0,0,0] = 1 then
    # give block 1's centre-tap weight gradient dP1[0,0,0] = 1.  Block 2's own
    # centre-tap gradient is P1[0,0,0] * dZ2[0,0,0] = 1.
    x1 = np.zeros((1, 4, 4, 4, 1))
    x1[0, 0, 0, 0, 0] = 1.0
    p1 = np.ones((1, 2, 2, 2, 1))
    blocks = [dict(x=x1, p=p1, idx=np.zeros((1, 2, 2, 2, 1), np.uint8)),
              dict(x=p1, p=np.ones((1, 1, 1, 1, 1)), idx=np.zeros((1, 1, 1, 1, 1), np.uint8))]
    cache = linear_cache(blocks, (1, 1, 1, 1, 1))
    w1 = delta_weights({CENTER: 1.0})
    w2 = delta_weights({CENTER: 1.0 + 2.0 ** -10})
    trace = {}
    gw, _ = oracle.network_backward(cache, [w1, w2], linear_head(), np.ones((1, 1)), SLOPE, "bf16", trace=trace)
    assert trace["dp"][0][0, 0, 0, 0, 0] == 1.0
    assert np.count_nonzero(trace["dp"][0]) == 1
    assert gw[0][1, 1, 1, 0, 0] == 1.0
    assert gw[1][1, 1, 1, 0, 0] == 1.0
    gw64, _ = oracle.network_backward(cache, [w1, w2], linear_head(), np.ones((1, 1)), SLOPE, "f64")
    assert gw64[0][1, 1, 1, 0, 0] == 1.0 + 2.0 ** -10


def test_conv_weights_are_rounded_before_the_forward_pass():
    # Master weight 1 + 2^-8 + 2^-10 at the centre tap lies above the midpoint
    # 1 + 2^-8 between the bf16 neighbours 1 and 1 + 2^-7, so the pass uses
    # 1 + 2^-7.  With X[0,0,0] = 3: (1 + 2^-7) * 3 = 3.0234375, which sits
    # halfway between the bf16 numbers 3.015625 and 3.03125 (spacing 2^-6 at
    # 3); ties to even give 3.03125 (significand 194).  Rounding only the
    # product instead would give 3 * (1 + 2^-8 + 2^-10) = 3.0146484375 ->
    # 3.015625.
    x = np.zeros((1, 2, 2, 2, 1))
    x[0, 0, 0, 0, 0] = 3.0
    w = delta_weights({CENTER: 1.0 + 2.0 ** -8 + 2.0 ** -10})
    trace = {}
    out = oracle.train_step(x, np.zeros((1, 1)), [w], linear_head(), 0.0, SLOPE, "bf16", trace=trace)
    assert trace["conv_w"][0][1, 1, 1, 0, 0] == 1.0 + 2.0 ** -7
    assert trace["z"][0][0, 0, 0, 0, 0] == 3.03125
    assert out["yhat"][0, 0] == 3.03125       # P passes the identity head unchanged
    # the update is applied to the master, not to its bf16 copy (lr 0 keeps it)
    assert out["conv_w"][0][1, 1, 1, 0, 0] == np.float32(1.0 + 2.0 ** -8 + 2.0 ** -10)


def test_every_storage_point_is_on_its_grid():
    """On a random two-block problem every traced storage point of the bf16
    model is a bf16 number and every one of the fp32 model an fp32 number;
    the fp32 model's values are mostly not bf16 numbers (so the bf16 check
    is not vacuous)."""
    r = np.random.default_rng(5)
    x = oracle.round_bf16(r.standard_normal((2, 8, 8, 8, 2)))
    conv = [r.standard_normal((3, 3, 3, 2, 4)) * 0.3, r.standard_normal((3, 3, 3, 4, 8)) * 0.2]
    dense = [(r.standard_normal((64, 16)) * 0.2, r.standard_normal(16) * 0.1),
             (r.standard_normal((16, 8)) * 0.2, r.standard_normal(8) * 0.1),
             (r.standard_normal((8, 3)) * 0.3, r.standard_normal(3) * 0.1)]
    t = r.uniform(-1, 1, (2, 3))
    for storage, rnd in (("bf16", oracle.round_bf16), ("f32", oracle.round_f32)):
        trace = {}
        oracle.train_step(x, t, conv, dense, 1e-3, SLOPE, storage, trace=trace)
        arrays = trace["conv_w"] + trace["z"] + trace["dp"] + trace["dz"]
        assert len(arrays) == 8
        for a in arrays:
            assert np.array_equal(a, rnd(a))
        if storage == "f32":
            off_bf16 = np.mean(np.concatenate([(a != oracle.round_bf16(a)).ravel() for a in arrays]))
            assert off_bf16 > 0.5


def test_round_f32_matches_numpy_float32_conversion():
    r = np.random.default_rng(11)
    x = np.concatenate([
        r.standard_normal(100000) * 10.0 ** r.integers(-40, 40, 100000),
        1.0 + np.arange(-2000, 2000) * 2.0 ** -26,                        # near ties around 1
        np.array([2.0 ** -149, 2.0 ** -150, 3 * 2.0 ** -150, 2.0 ** -151, 3.5e38, -3.5e38, 0.0, -0.0]),
    ])
    with np.errstate(over="ignore"):
        expect = x.astype(np.float32).astype(np.float64)
    got = oracle.round_f32(x)
    assert np.array_equal(got, expect)
    # worked values: ties go to the even significand
    assert oracle.round_f32([1.0 + 2.0 ** -24])[0] == 1.0
    assert oracle.round_f32([1.0 + 3 * 2.0 ** -24])[0] == 1.0 + 2.0 ** -22
    assert oracle.round_f32([2.0 ** -150])[0] == 0.0                 # half the smallest subnormal -> 0 (even)
    assert oracle.round_f32([3 * 2.0 ** -150])[0] == 2.0 ** -148     # 1.5 quanta -> 2 quanta
