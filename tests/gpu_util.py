"""Helpers shared by the GPU parity tests (host-side only)."""
import numpy as np
import torch

DEV = "cuda"

# Tolerances: max_i |gpu_i - oracle_i| / RMS(oracle) per output tensor.
TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def to_dev(a, dtype):
    """numpy float array (values already on the target grid) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(DEV).to(dtype)


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def host32(t):
    return t.detach().float().cpu().numpy()


def rel_err(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    rms = np.sqrt(np.mean(o * o))
    if rms == 0.0:
        return float(np.max(np.abs(g - o)))
    return float(np.max(np.abs(g - o)) / rms)


def bf16_ulp(o):
    """One bf16 quantum at each value of o: 2^(e - 7) for |o| in [2^e, 2^(e+1))
    (8 significant bits), the subnormal spacing 2^-133 below 2^-126."""
    a = np.abs(np.asarray(o, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def rel_err_bf16(g, o):
    """rel_err for a tensor that both sides store in bf16: the part of each
    difference beyond one bf16 quantum at the oracle's value, over RMS(o).
    Two correct roundings of sums that differ only in their last fp32 bits
    land one quantum apart; that is not counted as error."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    rms = np.sqrt(np.mean(o * o))
    excess = np.maximum(np.abs(g - o) - bf16_ulp(o), 0.0)
    if rms == 0.0:
        return float(np.max(excess))
    return float(np.max(excess) / rms)


def bf16_elementwise_ok(g, o, rms_frac=2e-3):
    """Each bf16 output within its own rounding (2^-8 relative) plus a small
    accumulation allowance relative to the tensor's RMS."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    rms = np.sqrt(np.mean(o * o))
    bad = np.abs(g - o) > (2.0 ** -8) * np.abs(o) + rms_frac * rms
    return int(np.count_nonzero(bad))


def sample_points(rng, shape, n, include_corners=True):
    """Flat indices into a tensor of `shape` (NDHWC): random points plus the
    volume's corner voxels (all channels), where padding matters most."""
    N, D, H, W, C = shape
    total = N * D * H * W * C
    pts = set(int(p) for p in rng.integers(0, total, size=n))
    if include_corners:
        for n_ in (0, N - 1):
            for d in (0, D - 1):
                for h in (0, H - 1):
                    for w in (0, W - 1):
                        base = (((n_ * D + d) * H + h) * W + w) * C
                        for c in (0, C - 1):
                            pts.add(base + c)
    return np.array(sorted(pts), dtype=np.int64)


def windows(z):
    """[N,D,H,W,C] -> [N,D/2,H/2,W/2,C,8] with the last axis in window order
    a*4 + b*2 + e (depth, height, width offsets)."""
    N, D, H, W, C = z.shape
    return z.reshape(N, D // 2, 2, H // 2, 2, W // 2, 2, C).transpose(0, 1, 3, 5, 7, 2, 4, 6).reshape(
        N, D // 2, H // 2, W // 2, C, 8)


def window_values(z, where):
    """Window values [K, 8] (window order) of z [N,D,H,W,C] at the K pooled
    positions of the boolean mask ``where`` [N,D/2,H/2,W/2,C]."""
    n, i, j, k, c = np.nonzero(where)
    out = np.empty((n.size, 8), np.float64)
    for pos in range(8):
        a, b, e = pos >> 2, (pos >> 1) & 1, pos & 1
        out[:, pos] = z[n, 2 * i + a, 2 * j + b, 2 * k + e, c]
    return out


def check_pool_indices(z_oracle, idx_gpu, idx_oracle, p_gpu, p_oracle, rel=2.0 ** -7):
    """The pooling rule where several answers are correct: a GPU window index
    may differ from the oracle's only where the oracle's two largest window
    values are a near tie, |v1 - v2| <= rel * max(|v1|, RMS(z)); there the
    two pooled values must agree to within that gap plus one bf16 rounding.
    Everywhere else the index must be the oracle's and P must match to
    within what the two roundings allow: each side's conv output is a bf16
    rounding of nearly the same sum (fp32 accumulation on the GPU, exact in
    the oracle), so the two can sit one bf16 ulp apart (up to 2^-7
    relative), and P = lrelu(Z) is rounded once more on each side (2^-9
    each); hence 2^-6 relative, plus 1e-3 of RMS(P) for outputs near zero.
    Returns the boolean mask of windows (shape of P) whose index differs,
    for masking the gradients that depend on them."""
    z = np.asarray(z_oracle, np.float64)
    idx_gpu = np.asarray(idx_gpu)
    idx_oracle = np.asarray(idx_oracle)
    rms = float(np.sqrt(np.mean(np.square(z))))
    diff = idx_gpu != idx_oracle
    if np.any(diff):
        top2 = np.sort(window_values(z, diff), axis=1)[:, -2:]
        near = (top2[:, 1] - top2[:, 0]) <= rel * np.maximum(np.abs(top2[:, 1]), rms)
        assert np.all(near), "index differs from the oracle's in %d windows without a near tie" % int(
            np.count_nonzero(~near))
    pg = np.asarray(p_gpu, np.float64)
    po = np.asarray(p_oracle, np.float64)
    prms = float(np.sqrt(np.mean(np.square(po))))
    tol = (2.0 ** -6) * np.abs(po) + 1e-3 * prms
    tol = np.where(diff, tol + rel * np.maximum(np.abs(po), prms), tol)
    assert np.all(np.abs(pg - po) <= tol), "pooled values differ beyond rounding"
    return diff


def kink_mask(z_oracle, p_oracle, slope, rel=2.0 ** -8):
    """Pooled positions whose window maximum z sits at the leaky-ReLU kink,
    |z| <= rel * RMS(z): there either slope of the derivative is accepted."""
    z = np.asarray(z_oracle, np.float64)
    po = np.asarray(p_oracle, np.float64)
    zmax = np.where(po > 0, po, po / slope)
    return np.abs(zmax) <= rel * float(np.sqrt(np.mean(np.square(z))))


def unpool_neighbourhood_mask(diff, halo=1):
    """Voxel mask [N,D,H,W] (input resolution of the pool) of every voxel
    whose conv backward-data value can depend on a window in ``diff``
    ([N,Dp,Hp,Wp,C] bool): the window's 2^3 voxels grown by ``halo`` voxels
    on each side."""
    N, Dp, Hp, Wp = diff.shape[:4]
    anyc = diff.any(axis=4)
    mask = np.zeros((N, 2 * Dp, 2 * Hp, 2 * Wp), bool)
    for n, i, j, k in zip(*np.nonzero(anyc)):
        mask[n, max(0, 2 * i - halo):2 * i + 2 + halo, max(0, 2 * j - halo):2 * j + 2 + halo,
             max(0, 2 * k - halo):2 * k + 2 + halo] = True
    return mask
