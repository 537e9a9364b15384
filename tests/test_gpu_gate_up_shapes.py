"""Every shape of the decode gate_up kernel on the GPU: moe_gate_up on seeded
activations, FP32 and BF16 h (and, for FP32 weights, FP32 and BF16 x),
against the float64 oracle's h element by element.

The host picks the 16-byte chunks per lane of a weight row (1, 2, 4, 7 or 8;
rows that are not whole 64-lane passes take the guarded next size), the
neurons per wavefront (2 up to two chunks per lane, else 1), whether the
rows are converted to BF16 once per item, and for MXFP8 neuron pairs whether
the scales come in as one dword per lane.  Each combination with the x and h
types is its own compiled kernel.  The H values below are a smallest set
that launches every combination those rules can pick for H up to 8192 (2048
for FP32 rows); I is kept off the matrix-core kernel's grid for E2M1 rows, so
the vector kernel runs."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import layer as L
from _helpers import device_routing, device_weights, inputs, oracle_kw, to_device_x, to_f64

pytestmark = pytest.mark.gpu

BASE = {"f32": W.TINY_FP32, "mxfp8": W.QWEN3_DECODE_MXFP8, "mxfp4": W.MXFP4_SWEEP,
        "fp8_blk128": W.DEEPSEEK_V3_FP8_BLK128}
HIDDEN = {
    "f32": (32, 256, 288, 512, 544, 1024, 1056, 1792, 2048),
    "mxfp8": (32, 1024, 1056, 2048, 2080, 4096, 4128, 7168, 8192),
    "mxfp4": (32, 2048, 2080, 4096, 4128, 8192),
    "fp8_blk128": (128, 1024, 1152, 2048, 2176, 4096, 4224, 7168, 8192),
}
INTER = {"f32": 64, "mxfp8": 64, "mxfp4": 96, "fp8_blk128": 128}
CASES = [(f, h) for f in HIDDEN for h in HIDDEN[f]]


@pytest.mark.parametrize("fmt,hidden", CASES)
def test_gate_up_every_compiled_shape(lib, fmt, hidden):
    for act in (("f32", "bf16") if fmt == "f32" else ("bf16",)):
        cfg = BASE[fmt].replace(hidden=hidden, inter=INTER[fmt], num_experts=4, top_k=2,
                                num_shared=0, act=act, tag=300 + CASES.index((fmt, hidden)))
        t = 5
        x, ids, w = inputs(cfg, t)
        Wd = device_weights(cfg)
        xd = to_device_x(cfg, x)
        idd, _ = device_routing(ids, w)
        h_ref = L.gate_up(L.activations_f64(x, cfg.act), ids, **oracle_kw(cfg))
        scale = np.sqrt(np.mean(h_ref ** 2))
        for hdt in (("f32",) if fmt == "f32" else ("f32", "bf16")):
            h = lib.gate_up(Wd, xd, idd, h_dtype=hdt)
            torch.cuda.synchronize()
            err = np.abs(to_f64(h) - h_ref)
            # FP32 sums of exact products over H terms; BF16 h adds one rounding
            tol = 2e-4 * scale + 1e-6 + (2.0 ** -8 * np.abs(h_ref) if hdt == "bf16" else 0.0)
            assert np.all(err <= tol), (fmt, hidden, act, hdt, float(np.max(err / (scale + 1e-30))))
