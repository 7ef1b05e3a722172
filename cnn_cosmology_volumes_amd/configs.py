"""Network descriptions, shape inference and work counters.

A network is a stack of conv blocks followed by a dense head.  Each block is
a 3^3 convolution with "same" zero padding (stride 1 unless stated), then
leaky ReLU, then 2^3 pooling with stride 2 (Oyama et al., Table I: stride-1
convolutions and stride-2 pooling unless noted, "same" padding everywhere;
CosmoFlow, Sec. III-A: conv and fully connected layers with leaky ReLU).

Work is counted as 2 flops per multiply-add over all 27 taps at every output
voxel, padded taps included; with that convention the counter reproduces the
per-sample GFlop figures and parameter counts printed in Oyama et al.,
Table I (checked in the tests).
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple


@dataclass(frozen=True)
class ConvLayer:
    cin: int
    cout: int
    stride: int = 1          # conv stride (Table I's c4 has stride 2)
    pool: bool = True        # followed by a 2^3 stride-2 pool


@dataclass
class Network:
    in_channels: int
    in_size: int                         # cubic input width W_i
    convs: List[ConvLayer]
    dense: List[int]                     # output widths of the dense layers
    dense_bias: bool = True
    slope: float = 0.3

    def conv_shapes(self) -> List[Tuple[int, int, int]]:
        """(input width, conv output width, pooled output width) per block."""
        out = []
        w = self.in_size
        for L in self.convs:
            wc = -(-w // L.stride)       # "same" padding: ceil(w / stride)
            wp = wc // 2 if L.pool else wc
            out.append((w, wc, wp))
            w = wp
        return out

    def flatten_size(self) -> int:
        w = self.conv_shapes()[-1][2] if self.convs else self.in_size
        c = self.convs[-1].cout if self.convs else self.in_channels
        return w ** 3 * c

    def conv_fwd_flops(self) -> List[int]:
        """Per-sample forward flops of each conv layer."""
        fl = []
        for (w, wc, wp), L in zip(self.conv_shapes(), self.convs):
            fl.append(2 * 27 * L.cin * L.cout * wc ** 3)
        return fl

    def conv_params(self) -> int:
        return sum(27 * L.cin * L.cout for L in self.convs)

    def dense_params(self) -> int:
        n, fan = 0, self.flatten_size()
        for o in self.dense:
            n += fan * o + (o if self.dense_bias else 0)
            fan = o
        return n

    def dense_fwd_flops(self) -> int:
        n, fan = 0, self.flatten_size()
        for o in self.dense:
            n += 2 * fan * o
            fan = o
        return n


def cosmoflow_block_net(in_size: int, filters: List[int], dense=(128, 64, 3),
                        in_channels: int = 4, slope: float = 0.3) -> Network:
    """Blocks of [conv 3^3 pad 1 -> leaky ReLU -> max-pool 2^3] with the given
    filter counts, then the dense head."""
    convs, cin = [], in_channels
    for f in filters:
        convs.append(ConvLayer(cin, f))
        cin = f
    return Network(in_channels, in_size, convs, list(dense), True, slope)


def oyama_table1_net(in_size: int) -> Network:
    """The extended CosmoFlow network of Oyama et al., Table I, used here only
    to pin the work counters: filters 16..256, c4 with stride 2, pooling after
    c1..c5 (plus p6 at 256^3 and p6, p7 at 512^3), fc 2048-256-4, no biases."""
    filters = [16, 32, 64, 128, 256, 256, 256]
    extra_pools = {128: 0, 256: 1, 512: 2}[in_size]
    convs, cin = [], 4
    for i, f in enumerate(filters):
        pool = i < 5 + extra_pools
        convs.append(ConvLayer(cin, f, stride=2 if i == 3 else 1, pool=pool))
        cin = f
    return Network(4, in_size, convs, [2048, 256, 4], dense_bias=False)


@dataclass
class Config:
    seed_id: int                    # stream id of the seeded input generators
    name: str
    batch: int
    in_size: int
    filters: List[int]
    dtype: str                      # 'f32' or 'bf16'
    kind: str                       # 'conv_fwd' | 'block' | 'train' | 'partial'
    dense: Optional[List[int]] = None
    # Plain SGD with He-initialised weights and no normalisation starts from
    # predictions of order 10; steps of 1e-4 and above diverge on the 128^3
    # network, 1e-6 lowers the loss steadily.
    lr: float = 1e-6
    slope: float = 0.3
    in_channels: int = 4
    note: str = ""

    def network(self) -> Network:
        return cosmoflow_block_net(self.in_size, self.filters, self.dense or [],
                                   self.in_channels, self.slope)


_ALL = (
    Config(1, "conv3d_fwd_f32_32c4", 1, 32, [16], "f32", "conv_fwd",
           note="single conv forward, fp32, 1x32^3x4 -> 16, lognormal field input"),
    Config(2, "block_bf16_128c4_b4", 4, 128, [32], "bf16", "block",
           note="one block fwd+dgrad+wgrad, 4x128^3x4 -> 32, upstream grad N(0,1)"),
    Config(3, "train_bf16_128c4_b8", 8, 128, [32, 64, 128, 256, 256], "bf16", "train",
           dense=[128, 64, 3], note="full 5-block network training step"),
    Config(4, "partial_bf16_512c4_b1", 1, 512, [32, 64], "bf16", "partial",
           note="first two blocks fwd+bwd at 512^3"),
    Config(5, "train_bf16_512c4_b1", 1, 512, [32, 64, 128, 256, 256, 256, 256], "bf16", "train",
           dense=[128, 64, 3], note="full 7-block network training step at 512^3"),
)
# the workloads by name
CONFIGS = {c.name: c for c in _ALL}


def train_step_conv_flops(net: Network, batch: int, first_dgrad: bool = False) -> int:
    """Conv flops of one training step: forward + backward-weight for every
    layer, backward-data for every layer but the first (the input needs no
    gradient) unless ``first_dgrad``."""
    f = net.conv_fwd_flops()
    total = 2 * sum(f) + sum(f[1:]) + (f[0] if first_dgrad else 0)
    return total * batch
