"""The training step captured into a HIP graph (torch.cuda.CUDAGraph) and
replayed.  Every replay, with an eager step of its own on another copy of the
parameters and a device synchronization between replays, must equal that
eager step bit for bit (loss, prediction and every parameter), on one stream
and with the weight gradients on a second stream (cf_step_aux), whose fork
and join events put it into the capture."""
import pytest
import torch

from cnn_cosmology_volumes_amd import cf
from gpu_util import to_dev
from test_gpu_train import BF, F32, SLOPE, device_params, make_problem

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("two_streams", [False, True])
def test_train_step_graph_replays_equal_eager_steps(two_streams):
    B, size, filters, dense_w = 2, 32, [32, 64, 128], [64, 32, 3]
    x, conv, dense, t = make_problem(5, B, size, filters, dense_w, BF)
    m = cf.model_desc(4, size, filters, dense_w, SLOPE)
    xd, td = to_dev(x, BF), to_dev(t, F32)
    pe, pg = device_params(conv, dense), device_params(conv, dense)
    nbytes = cf.cf_train_step_workspace_size(m, cf.CF_BF16, B)
    ws_e = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ws_g = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    loss_e, loss_g = (torch.empty(1, dtype=F32, device="cuda") for _ in range(2))
    pred_e, pred_g = (torch.empty((B, dense_w[-1]), dtype=F32, device="cuda") for _ in range(2))
    aux_e = cf.StepAux() if two_streams else None
    aux_g = cf.StepAux() if two_streams else None
    lr = 1e-5          # (1e-4 and above diverge on this problem within a few steps)

    def eager():
        cf.cf_train_step(m, xd, td, pe, lr, ws=ws_e, loss=loss_e, pred=pred_e, aux=aux_e)

    def graphed():
        cf.cf_train_step(m, xd, td, pg, lr, ws=ws_g, loss=loss_g, pred=pred_g, aux=aux_g)

    def check(what):
        torch.cuda.synchronize()
        assert torch.isfinite(loss_e).all(), what
        assert torch.equal(loss_g, loss_e) and torch.equal(pred_g, pred_e), what
        for i, (p, q) in enumerate(zip(pe, pg)):
            assert torch.equal(p, q), (what, i)

    # one eager step each, the graph's on the stream it is captured on
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graphed()
    torch.cuda.current_stream().wait_stream(side)
    eager()
    check("eager steps")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed()
    check("capture executes nothing")
    for r in range(6):
        g.replay()
        eager()
        check("replay %d" % r)
    del g
    for a in (aux_e, aux_g):
        if a is not None:
            a.close()
