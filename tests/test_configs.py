"""Pins of the shape-inference and work counters to the numbers printed in
Oyama et al., Table I (tests/golden/oyama_table1.json)."""
import json
import os

import pytest

from cnn_cosmology_volumes_amd.configs import (CONFIGS, oyama_table1_net,
                                               train_step_conv_flops)

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "oyama_table1.json")))


@pytest.mark.parametrize("w", [128, 256, 512])
def test_table1_forward_and_total_gflops(w):
    net = oyama_table1_net(w)
    fwd = sum(net.conv_fwd_flops()) / 1e9
    assert round(fwd, 4 - len(str(int(fwd)))) == pytest.approx(GOLD["forward_gflops_per_sample"][str(w)])
    tot = 3 * fwd  # forward + backward-data + backward-weight, every layer
    printed = GOLD["conv_ops_gflops_per_sample"][str(w)]
    assert abs(tot - printed) / printed < 5e-4


@pytest.mark.parametrize("w", [128, 256, 512])
def test_table1_parameter_count(w):
    net = oyama_table1_net(w)
    assert net.flatten_size() == GOLD["fc_widths"][0]
    p = (net.conv_params() + net.dense_params()) / 1e6
    assert round(p, 2) == GOLD["parameters_millions"][str(w)]


@pytest.mark.parametrize("w", [128, 256, 512])
def test_table1_output_widths(w):
    net = oyama_table1_net(w)
    got = [[wc, wp if L.pool else None] for (wi, wc, wp), L in zip(net.conv_shapes(), net.convs)]
    assert got == GOLD["output_widths"][str(w)]


def test_config_networks():
    # the headline configuration: 5 blocks at 128^3 end in 4^3 x 256 = 16384
    n3 = CONFIGS["train_bf16_128c4_b8"].network()
    assert n3.flatten_size() == 4 ** 3 * 256
    n5 = CONFIGS["train_bf16_512c4_b1"].network()
    assert n5.flatten_size() == 4 ** 3 * 256
    # conv work of one training step of the headline config (layer-1
    # backward-data not computed): 186.6 GF/sample
    f = train_step_conv_flops(n3, 1)
    assert abs(f / 1e9 - 186.63) < 0.01
    assert n3.conv_params() + n3.dense_params() == 2934144 + 2105731
