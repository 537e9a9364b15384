"""moe_layer captured in a HIP graph (the header allows capture: the library
records kernels only, no allocation, memset or synchronisation).  Each
replay is checked against an eager call of the same layer, bit for bit (the
path is deterministic), with eager work and synchronisations between the
replays, and after the inputs are changed in place."""

import numpy as np
import pytest
import torch

import workloads as W
from _helpers import device_routing, device_weights, inputs, to_device_x

pytestmark = pytest.mark.gpu

CFG = W.QWEN3_DECODE_MXFP8.replace(num_experts=16, tag=41)


def _workspace(lib, Wd, t, k, path, block):
    need = lib.layer_workspace_bytes(Wd, t, k, path=path, block=block)
    return torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("path,t", [("decode", 8), ("decode", 1), ("grouped", 96)])
def test_layer_replays_from_a_graph(lib, path, t):
    block = 64
    k = CFG.top_k
    Wd = device_weights(CFG)
    x, ids, w = inputs(CFG, t)
    xd = to_device_x(CFG, x)
    idd, wd = device_routing(ids, w)
    ws = _workspace(lib, Wd, t, k, path, block)
    y = torch.empty((t, CFG.hidden), dtype=torch.float32, device="cuda")

    # eager reference on separate buffers
    y_ref, chosen = lib.layer(Wd, xd, idd, wd, path=path, block=block)
    torch.cuda.synchronize()
    assert chosen == path

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside capture
        lib.layer(Wd, xd, idd, wd, path=path, block=block, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lib.layer(Wd, xd, idd, wd, path=path, block=block, y=y, workspace=ws)

    for rep in range(4):
        y.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), (path, t, rep)
        # an unrelated eager layer call on other buffers in between
        lib.layer(Wd, xd, idd, wd, path=path, block=block)
        torch.cuda.synchronize()

    # new inputs written in place: the replay reads the buffers at replay time
    x2, ids2, w2 = inputs(CFG, t, variant=1)
    xd.copy_(to_device_x(CFG, x2))
    i2, w2d = device_routing(ids2, w2)
    idd.copy_(i2)
    wd.copy_(w2d)
    y_ref2, _ = lib.layer(Wd, xd, idd, wd, path=path, block=block)
    torch.cuda.synchronize()
    assert not torch.equal(y_ref2, y_ref)
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref2), (path, t, "new inputs", rep)
    del g
    torch.cuda.synchronize()
    assert np.isfinite(y.cpu().numpy()).all()
