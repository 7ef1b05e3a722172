"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle legs.

This module draws random inputs only; it holds none of the method's
arithmetic.  The real workloads are N-body dark-matter volumes: 4 channels
(redshifts) of particle-count histograms, 128^3 sub-volumes cut from 512^3
boxes (CosmoFlow, Sec. IV-C; Oyama et al., Sec. II-B), with the cosmological
parameters normalised to [-1, 1] as regression targets (Oyama et al.,
Sec. II-B).  Those data are not available here, so these generators stand in
for them with the same shapes and a similar value structure: a unit-mean
lognormal density per sample and channel, Poisson-sampled counts (many empty
voxels), and log(1 + counts) as the network input.

Streams: ``numpy.random.default_rng(SeedSequence([2026, seed_id]))`` spawned
into the fixed order [field, poisson, conv-weights, dense-weights, targets,
upstream-grad].
"""
import numpy as np

STREAMS = ("field", "poisson", "convw", "densew", "targets", "upstream")


def streams(seed_id: int, seed: int = 2026):
    """Dict of independent numpy Generators for one configuration."""
    ss = np.random.SeedSequence([seed, seed_id])
    return {name: np.random.default_rng(child) for name, child in zip(STREAMS, ss.spawn(len(STREAMS)))}


def bf16_round_f32(x):
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32.  Used only to quantise generated inputs to the bf16 grid."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    # keep NaN/Inf as they are (not produced by these generators)
    bad = ~np.isfinite(a)
    if bad.any():
        out = out.copy()
        out[bad] = a[bad]
    return out.reshape(np.shape(x))


def lognormal_density(rng, shape_ndhw, channels, dtype=np.float32):
    """delta = exp(g) / mean(exp(g)) per sample and channel, g ~ N(0,1) white.

    Returns [N,D,H,W,C] float.  Generated channel by channel to bound RAM."""
    N = shape_ndhw[0]
    out = np.empty(tuple(shape_ndhw) + (channels,), dtype)
    for n in range(N):
        for c in range(channels):
            e = np.exp(rng.standard_normal(shape_ndhw[1:], dtype=np.float32))
            e /= e.mean(dtype=np.float64)
            out[n, ..., c] = e
    return out


def lognormal_field_input(rng, shape_ndhw, channels):
    """log(1 + delta) of a unit-mean lognormal field (no Poisson sampling)."""
    d = lognormal_density(rng, shape_ndhw, channels)
    np.log1p(d, out=d)
    return d


def lognormal_poisson_input(rng_field, rng_pois, shape_ndhw, channels, bf16=True):
    """log(1 + Poisson(delta)) with delta a unit-mean lognormal density, per
    sample and channel; optionally quantised to the bf16 grid."""
    N = shape_ndhw[0]
    out = np.empty(tuple(shape_ndhw) + (channels,), np.float32)
    for n in range(N):
        for c in range(channels):
            e = np.exp(rng_field.standard_normal(shape_ndhw[1:], dtype=np.float32))
            e /= e.mean(dtype=np.float64)
            counts = rng_pois.poisson(e).astype(np.float32)
            np.log1p(counts, out=counts)
            out[n, ..., c] = counts
    return bf16_round_f32(out) if bf16 else out


def he_normal_conv(rng, cin, cout, dtype=np.float32):
    """He-normal conv weights, DHWIO [3,3,3,cin,cout], N(0, 2/(27*cin))."""
    std = np.sqrt(2.0 / (27.0 * cin))
    return (rng.standard_normal((3, 3, 3, cin, cout)) * std).astype(dtype)


def he_normal_dense(rng, fan_in, fan_out, dtype=np.float32):
    """He-normal dense weights [in,out], N(0, 2/in); zero bias."""
    std = np.sqrt(2.0 / fan_in)
    w = (rng.standard_normal((fan_in, fan_out)) * std).astype(dtype)
    return w, np.zeros((fan_out,), dtype)


def targets(rng, batch, k=3, dtype=np.float32):
    """Normalised regression targets U(-1, 1)."""
    return rng.uniform(-1.0, 1.0, size=(batch, k)).astype(dtype)


def normal(rng, shape, bf16=True, scale=1.0):
    """N(0, scale^2) values (upstream gradients, synthetic activations)."""
    x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))
    return bf16_round_f32(x) if bf16 else x


def pool_indices(rng, shape):
    """Uniform window positions 0..7 (synthetic max-pool argmax)."""
    return rng.integers(0, 8, size=shape, dtype=np.uint8)


# ------------------------------------------------------------------------
# Device-side generators for the 512^3 volumes (seeded torch Philox streams;
# same recipes as above, drawn on the GPU because host generation of 10^9
# values is slow).  They draw random numbers only.
def torch_generator(seed, device):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def lognormal_poisson_input_torch(g, shape_ndhw, channels, device):
    """log(1 + Poisson(delta)), delta = exp(N(0,1)) / mean, per sample and
    channel; returned as a bf16 NDHWC device tensor."""
    import torch
    out = torch.empty(tuple(shape_ndhw) + (channels,), dtype=torch.bfloat16, device=device)
    for n in range(shape_ndhw[0]):
        for c in range(channels):
            e = torch.randn(tuple(shape_ndhw[1:]), generator=g, device=device).exp_()
            e /= e.mean(dtype=torch.float64).float()
            counts = torch.poisson(e, generator=g)
            out[n, ..., c] = counts.log1p_().to(torch.bfloat16)
            del e, counts
    return out


def normal_torch(g, shape, device, scale=1.0):
    """N(0, scale^2) bf16 device tensor, drawn in 2^28-element chunks."""
    import torch
    out = torch.empty(tuple(shape), dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    step = 1 << 28
    for s in range(0, flat.numel(), step):
        e = min(flat.numel(), s + step)
        flat[s:e] = (torch.randn(e - s, generator=g, device=device) * scale).to(torch.bfloat16)
    return out
