"""moe_layer_noalloc (the layer with the library's own device array as its
workspace) against moe_layer with a caller workspace: the same kernels on the
same inputs, so the outputs must be identical bit for bit.  Two calls in a
row per path, the second with fewer tokens, so the second reads an array
that still holds the first call's contents."""

import pytest
import torch

import workloads as W
from oracle import layer as L
from _helpers import (assert_layer_close, device_routing, device_weights, inputs, oracle_kw,
                      to_device_x, to_f64)

pytestmark = pytest.mark.gpu

CFG = W.QWEN3_DECODE_MXFP8.replace(num_experts=16, tag=41)
MODE = {"decode": "none", "grouped": "mxfp8"}


@pytest.mark.parametrize("path,block,sizes", [("decode", 0, (37, 6)), ("grouped", 32, (45, 11)),
                                              ("auto", 0, (200, 3))])
def test_noalloc_matches_layer_twice(lib, path, block, sizes):
    Wd = device_weights(CFG)
    for i, t in enumerate(sizes):
        x, ids, w = inputs(CFG, t, variant=i)
        xd = to_device_x(CFG, x)
        idd, wd = device_routing(ids, w)
        y_ref, chosen_ref = lib.layer(Wd, xd, idd, wd, path=path, block=block)
        y = torch.full((t, CFG.hidden), float("nan"), dtype=torch.float32, device="cuda")
        chosen = lib.layer_noalloc(Wd, xd, idd, wd, y, path=path, block=block)
        torch.cuda.synchronize()
        assert chosen == chosen_ref, (t, chosen, chosen_ref)
        assert torch.equal(y, y_ref), (path, t)
        rows = sorted({0, t // 2, t - 1})
        ref = L.moe_layer(L.activations_f64(x[rows], CFG.act), ids[rows], w[rows],
                          act_quant=MODE[chosen], **oracle_kw(CFG))
        assert_layer_close(to_f64(y)[rows], ref, (path, t))


def test_noalloc_refuses_a_call_beyond_its_array(lib):
    """A grouped call whose workspace exceeds the array is refused on the
    host with nothing enqueued; y keeps its contents."""
    Wd = device_weights(CFG)
    t = 4096
    need = lib.layer_workspace_bytes(Wd, t, CFG.top_k, "grouped", 128)
    assert need > lib.layer_noalloc_max_bytes()
    x, ids, w = inputs(CFG, t)
    y = torch.zeros((t, CFG.hidden), dtype=torch.float32, device="cuda")
    with pytest.raises(lib.MoeError) as err:
        lib.layer_noalloc(Wd, to_device_x(CFG, x), *device_routing(ids, w), y, path="grouped",
                          block=128)
    assert err.value.status == lib.ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert not y.any()
