"""cf_conv3d_bwd_weight_noalloc (backward-weight with the split partial sums
in the library's static per-device scratch) against cf_conv3d_bwd_weight
with a caller workspace: identical bits, on two calls in a row where the
second is smaller (the scratch keeps the first call's contents, which the
second must not see), for each backward-weight path (bf16 MFMA for Cin % 32
== 0, the 4-channel first layer, fp32 on the matrix cores, the direct fp32
kernel)."""
import numpy as np
import pytest
import torch

import synthdata as sd
from cnn_cosmology_volumes_amd import cf

pytestmark = pytest.mark.gpu
BF, F32 = torch.bfloat16, torch.float32

CASES = [
    # (dtype, first shape, second smaller shape, cout)
    (BF, (8, 64, 64, 64, 32), (2, 16, 16, 16, 32), 64),      # the 128^3 step's second block, then a small one
    (BF, (8, 8, 8, 8, 256), (2, 6, 5, 7, 64), 256),          # volumes at most 8 wide: the 4 x 8 x 8 box
    (BF, (2, 34, 20, 18, 4), (1, 6, 10, 14, 4), 32),         # first-layer kernel, ragged boxes
    (F32, (2, 12, 10, 9, 8), (1, 5, 6, 7, 8), 16),           # fp32 matrix-core kernel
    (F32, (2, 6, 5, 7, 3), (1, 4, 3, 5, 3), 5),              # direct fp32 kernel (channels not multiples of 4)
]


def tensors(rng, shape, cout, dtype):
    N, D, H, W, C = shape
    x = torch.from_numpy(sd.normal(rng, shape, bf16=(dtype == BF))).cuda().to(dtype)
    dy = torch.from_numpy(sd.normal(rng, (N, D, H, W, cout), bf16=(dtype == BF))).cuda().to(dtype)
    return x, dy


@pytest.mark.parametrize("case", CASES)
def test_noalloc_equals_workspace_entry_point(case):
    dtype, big, small, cout = case
    rng = np.random.default_rng(sum(big) + cout)
    for shape in (big, small):
        x, dy = tensors(rng, shape, cout, dtype)
        dw_ref = cf.cf_conv3d_bwd_weight(x, dy)
        dw = torch.full((3, 3, 3, shape[4], cout), float("nan"), dtype=F32, device="cuda")
        cf.cf_conv3d_bwd_weight_noalloc(x, dy, dw)
        torch.cuda.synchronize()
        assert torch.equal(dw.view(torch.int32), dw_ref.view(torch.int32)), shape


def test_noalloc_rejects_shapes_beyond_the_scratch():
    # a 1024 -> 1024 layer's dW alone (27 x 1024 x 1024 fp32 = 113 MB) is
    # beyond the 64 MiB scratch, whatever the split
    x = torch.zeros((1, 2, 2, 2, 1024), dtype=F32, device="cuda")
    dy = torch.zeros((1, 2, 2, 2, 1024), dtype=F32, device="cuda")
    dw = torch.zeros((3, 3, 3, 1024, 1024), dtype=F32, device="cuda")
    with pytest.raises(cf.CfError) as e:
        cf.cf_conv3d_bwd_weight_noalloc(x, dy, dw)
    assert e.value.status == cf.CF_ERR_WORKSPACE
