"""Every shape of the decode down kernels on the GPU: moe_down alone on a
seeded h, token-major and expert-major, FP32 and BF16 h, against the float64
oracle's down product (per token: cosine >= 0.99999, relative L2 <= 5e-3),
and the two launch shapes bit for bit against each other.

The host picks the lanes per W_down row (4, 8, 16 or 32), the 16-byte chunks
per lane (2 to 16) and, expert-major, the rows per lane group (1, 2 or 4)
from the format, I and the type of h; each combination is its own compiled
kernel.  The I values below are a smallest set that, at H = 384, launches
every combination those rules can pick for I up to 8192 (for the E2M1 rows
H = 384 also keeps the matrix-core kernel out, so both launch shapes are the
vector kernels).  H = 384 is three 128-row FP8 tiles and not a whole number
of the wider row groups, so the last group of output rows is partial.
FP32 h on rows of 4096 and more quantised elements fits no compiled shape:
the library refuses it before any launch, and that is checked too."""

import numpy as np
import pytest
import torch

import mixture_experts_decode_amd as moe
import workloads as W
from oracle import layer as L
from _helpers import assert_layer_close, device_routing, device_weights, inputs, oracle_kw, to_f64

pytestmark = pytest.mark.gpu

BASE = {"f32": W.TINY_FP32, "mxfp8": W.QWEN3_DECODE_MXFP8, "mxfp4": W.MXFP4_SWEEP,
        "fp8_blk128": W.DEEPSEEK_V3_FP8_BLK128}
INTER = {
    "f32": (32, 64, 96, 128, 192, 256, 384, 512, 768, 1024, 1536, 2048),
    "mxfp8": (128, 192, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144),
    "mxfp4": (256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144),
    "fp8_blk128": (128, 256, 384, 512, 768, 1024, 1536, 2048, 3072, 4096, 6144),
}
CASES = [(f, i) for f in INTER for i in INTER[f]]


def _bf16_bits_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("fmt,inter", CASES)
def test_down_every_compiled_shape(lib, fmt, inter):
    cfg = BASE[fmt].replace(hidden=384, inter=inter, num_experts=4, top_k=2, num_shared=0,
                            tag=200 + CASES.index((fmt, inter)))
    t = 5
    _, ids, w = inputs(cfg, t)
    Wd = device_weights(cfg)
    idd, wd = device_routing(ids, w)
    for hdt in (("f32",) if fmt == "f32" else ("f32", "bf16")):
        h = W.hidden_states(cfg, t, dtype=hdt)
        if fmt != "f32" and hdt == "f32" and inter >= 4096:
            hd = torch.from_numpy(h).cuda()
            for variant in ("token", "expert"):
                with pytest.raises(moe.MoeError) as err:
                    lib.down(Wd, hd, idd, wd, variant=variant)
                assert err.value.status == moe.ERR_UNSUPPORTED
            continue
        if hdt == "f32":
            hd, h64 = torch.from_numpy(h).cuda(), h.astype(np.float64)
        else:
            hd = torch.from_numpy(h.view(np.int16)).cuda().view(torch.bfloat16)
            h64 = _bf16_bits_f64(h)
        ref = L.down(h64, ids, w, **oracle_kw(cfg))
        y_tok = lib.down(Wd, hd, idd, wd, variant="token")
        y_exp = torch.full_like(y_tok, float("nan"))
        lib.down(Wd, hd, idd, wd, y=y_exp, variant="expert")
        torch.cuda.synchronize()
        assert_layer_close(to_f64(y_tok), ref, (fmt, inter, hdt))
        assert torch.equal(y_tok, y_exp), (fmt, inter, hdt)
