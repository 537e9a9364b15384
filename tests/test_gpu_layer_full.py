"""Full-size layers through moe_layer(AUTO), in the launch shape the
benchmark times, held per token to the oracle in the mode of the path the
call reports (decode: exact activations, mode "none"; grouped: MXFP8
activations with two-term h and BF16 slot outputs, mode "mxfp8"):
per-token cosine >= 0.99999 and relative L2 <= 5e-3.

Every token is compared where the float64 oracle finishes in seconds (the
Qwen3-style layer at B = 32, every decode-size batch); at the larger batches
a spread of tokens is compared (tokens are independent: each output row
depends only on its own token's activations and routing)."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import layer as L
from _helpers import (assert_layer_close, device_routing, device_weights, inputs, oracle_kw,
                      to_device_x, to_f64)

pytestmark = pytest.mark.gpu

MODE = {"decode": "none", "grouped": "mxfp8"}

# (workload, B, routing kind, tokens compared: None = every token, else how many)
CASES = [
    ("qwen3_decode_mxfp8", 32, None, None),
    # just past the decode down's expert-major switch (112 routed entries)
    ("qwen3_decode_mxfp8", 14, None, None),
    ("qwen3_decode_mxfp8", 64, None, 8),
    ("deepseek_v3_fp8_blk128", 1, None, None),
    # 18 routed entries: expert-major down on 32-lane FP8-128 rows
    ("deepseek_v3_fp8_blk128", 2, None, None),
    ("deepseek_v3_fp8_blk128", 64, None, 3),
    ("mxfp4_sweep", 8, "uniform", None),
    ("mxfp4_sweep", 8, "zipf", None),
    ("mxfp4_sweep", 128, "uniform", 6),
    ("mxfp4_sweep", 128, "zipf", 6),
]


def _sample(t, n):
    if n is None or n >= t:
        return list(range(t))
    return sorted({int(v) for v in np.linspace(0, t - 1, n)})


@pytest.mark.parametrize("name,t,kind,n", CASES)
def test_layer_auto_full_size(lib, name, t, kind, n):
    cfg = W.CONFIGS[name]
    x, ids, w = inputs(cfg, t, kind=kind)
    Wd = device_weights(cfg)
    want = lib.choose_path(Wd, t, cfg.top_k)
    y, chosen = lib.layer(Wd, to_device_x(cfg, x), *device_routing(ids, w), path="auto")
    torch.cuda.synchronize()
    assert chosen == want
    rows = _sample(t, n)
    x64 = L.activations_f64(x[rows], cfg.act)
    ref = L.moe_layer(x64, ids[rows], w[rows], act_quant=MODE[chosen], **oracle_kw(cfg))
    m = assert_layer_close(to_f64(y)[rows], ref, (name, t, kind, chosen))
    print(f"{name} B={t} {kind or cfg.routing} {chosen}: {len(rows)} tokens, {m}")
