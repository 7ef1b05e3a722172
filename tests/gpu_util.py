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
