"""Router front-end parity on the GPU: moe_topk_route against oracle.router.
The expert ids are compared bit-exactly (both sides decide on the same
float32 keys); the weights to 2e-6 relative (float32 exp and division
against float64)."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import router as R

pytestmark = pytest.mark.gpu


def _route(lib, scores, k, bias=None):
    s = torch.from_numpy(np.ascontiguousarray(scores, dtype=np.float32)).cuda()
    b = None if bias is None else torch.from_numpy(np.asarray(bias, dtype=np.float32)).cuda()
    ids, wts = lib.topk_route(s, k, bias=b)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), wts.cpu().numpy()


def _check(lib, scores, k, bias=None, rows=None):
    ids, wts = _route(lib, scores, k, bias)
    rows = np.arange(scores.shape[0]) if rows is None else rows
    ref_ids, ref_w = R.topk_route(scores[rows], k, bias)
    assert np.array_equal(ids[rows], ref_ids)
    assert np.allclose(wts[rows], ref_w, rtol=2e-6, atol=1e-8)
    return ids, wts


@pytest.mark.parametrize("name,t,kind", [("qwen3_decode_mxfp8", 32, None), ("qwen3_decode_mxfp8", 1, None),
                                         ("deepseek_v3_fp8_blk128", 64, None), ("mxfp4_sweep", 256, "zipf"),
                                         ("tiny_fp32", 4, None)])
def test_route_workload_scores(lib, name, t, kind):
    cfg = W.CONFIGS[name]
    scores, bias = W.gating_scores(cfg, t, kind)
    _check(lib, scores, cfg.top_k, bias)


def test_route_prefill_full_size_sampled(lib):
    cfg = W.PREFILL_ZIPF_MXFP8
    scores, bias = W.gating_scores(cfg, 16384)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(16384 - 64, 16384),
                                     np.random.default_rng(5).integers(0, 16384, 256)]))
    ids, _ = _check(lib, scores, cfg.top_k, bias, rows=rows)
    # every token's ids are distinct and in range
    srt = np.sort(ids, axis=1)
    assert np.all(srt[:, 1:] != srt[:, :-1]) and ids.min() >= 0 and ids.max() < cfg.num_experts


@pytest.mark.parametrize("e,k", [(70, 1), (70, 7), (8, 8), (1, 1), (1024, 64), (513, 5), (64, 64)])
def test_route_shapes(lib, e, k):
    rng = np.random.default_rng(e * 100 + k)
    scores = rng.standard_normal((37, e)).astype(np.float32)
    bias = rng.normal(0, 0.7, e).astype(np.float32)
    _check(lib, scores, k)
    _check(lib, scores, k, bias)


def test_route_ties_and_signed_zero(lib):
    rng = np.random.default_rng(9)
    scores = rng.integers(-2, 3, size=(200, 96)).astype(np.float32)     # heavy ties
    _check(lib, scores, 8)
    z = np.zeros((3, 16), dtype=np.float32)
    z[0, ::2] = -0.0                                                      # -0 ties +0
    z[1] = np.float32(1.5)
    z[2, 5] = np.float32(-1.0)
    _check(lib, z, 4)
    bias = np.where(np.arange(96) % 3 == 0, np.float32(1.0), np.float32(0.0)).astype(np.float32)
    _check(lib, scores, 8, bias)


def test_route_empty_batch(lib):
    ids, wts = _route(lib, np.zeros((0, 32), dtype=np.float32), 4)
    assert ids.shape == (0, 4) and wts.shape == (0, 4)


@pytest.mark.parametrize("path", ["decode", "grouped"])
def test_router_feeds_the_layer(lib, path):
    """Scores -> moe_topk_route -> moe_layer on the device, against the
    oracle router feeding the oracle layer (DeepSeek-style selection bias,
    shared expert).  The routed ids match bit for bit, so the layer is held
    to the usual parity bound of the path that ran."""
    from _helpers import assert_layer_close, device_weights, oracle_kw, to_device_x, to_f64
    from oracle import layer as L
    cfg = W.DEEPSEEK_V3_FP8_BLK128.replace(num_experts=16, hidden=1024, inter=512, tag=51)
    t = 24
    scores, bias = W.gating_scores(cfg, t)
    s = torch.from_numpy(scores).cuda()
    b = torch.from_numpy(bias).cuda()
    ids, wts = lib.topk_route(s, cfg.top_k, bias=b)
    x = W.activations(cfg, t)
    Wd = device_weights(cfg)
    y, chosen = lib.layer(Wd, to_device_x(cfg, x), ids, wts, path=path)
    torch.cuda.synchronize()
    assert chosen == path
    ref_ids, ref_w = R.topk_route(scores, cfg.top_k, bias)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    mode = "none" if path == "decode" else "mxfp8"
    ref = L.moe_layer(L.activations_f64(x, cfg.act), ref_ids.astype(np.int32),
                      ref_w.astype(np.float32), act_quant=mode, **oracle_kw(cfg))
    assert_layer_close(to_f64(y), ref, path)


@pytest.mark.parametrize("t,k,e,bad", [(0, 8, 128, []), (1, 8, 128, []), (32, 8, 128, [5, 77, 200]),
                                       (300, 9, 257, [0, 1, 2699]), (16384, 8, 256, [131071])])
def test_check_routing_counts_out_of_range_ids(t, k, e, bad):
    import mixture_experts_decode_amd as moe
    rng = np.random.default_rng(11)
    ids = rng.integers(0, e, size=(t, k)).astype(np.int32)
    flat = ids.reshape(-1)
    for i, p in enumerate(bad):
        flat[p] = (-1, e, 2**31 - 1, -2**31)[i % 4]
    res = moe.check_routing(torch.from_numpy(ids).cuda(), e)
    torch.cuda.synchronize()
    assert tuple(int(v) for v in res.cpu().numpy()) == R.check_routing(ids, e)


def test_check_routing_in_a_captured_graph():
    # the check records one kernel and writes its result without a clear, so a
    # graph replays it correctly after the ids change in place
    import mixture_experts_decode_amd as moe
    ids = torch.zeros((64, 8), dtype=torch.int32, device="cuda")
    res = torch.full((2,), 7, dtype=torch.int32, device="cuda")
    moe.check_routing(ids, 128, result=res)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.check_routing(ids, 128, result=res)
    for step, planted in enumerate(([], [40], [3, 511], [])):
        ids.zero_()
        for p in planted:
            ids.view(-1)[p] = 128
        g.replay()
        torch.cuda.synchronize()
        want = (len(planted), min(planted) if planted else -1)
        assert tuple(int(v) for v in res.cpu().numpy()) == want, step
