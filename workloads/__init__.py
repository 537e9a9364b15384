"""Seeded synthetic inputs for the routed-expert MoE FFN.

This package is shared by both sides of every parity check: the HIP path (via
the tests and the benchmark) and the float64 oracle read the very same bytes.
It holds none of the layer's arithmetic: it only draws random numbers, encodes
the drawn weights into their storage formats with library casts, and shapes
routing decisions.  It imports neither the oracle nor the product path.

Workloads (shapes from the pages: top-8 of 128 experts with hidden 2048 in the
warp-decode post's traditional-path and buffer sections; DeepSeek-V3 with 256
experts and 16384 x top-8 tokens in the align-and-sort article's benchmark and
profiling sections):

  1 tiny_fp32      H 256,  I 128,  E 8,   k 2, fp32 weights and activations
  2 qwen3_decode   H 2048, I 768,  E 128, k 8, MXFP8 weights, BF16 x
  3 deepseek_v3    H 7168, I 2048, E 256 (+1 shared), k 8, FP8 + 128x128 scales
  4 prefill_zipf   H 4096, I 1536, E 256, k 8, MXFP8, T 16384, Zipf(1.1) routing
  5 mxfp4_sweep    H 4096, I 1536, E 128, k 8, MXFP4 weights, uniform or Zipf(1.2)

Seeding: numpy PCG64 with SeedSequence([config, stream, index...]).  Weights
are seeded per expert, so any one expert can be regenerated alone.

Weight encoding (not part of the method: it only fixes the stored bytes,
which both sides read): values ~ N(0, 1/fan_in) in float32, then
  * MXFP8: per 32 contiguous K values, shared exponent floor(log2 amax) - 8,
    scale, clip to +-448, torch cast to float8_e4m3fn (round to nearest even);
  * MXFP4: shared exponent floor(log2 amax) - 2, clip to +-6, nearest E2M1
    value (ties to the even code), two codes per byte, even element low;
  * FP8 + 128x128 tiles: s = amax/448 per tile (float32), torch cast of w/s.
"""

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np
import torch

STREAM_WEIGHTS = 1
STREAM_X = 2
STREAM_ROUTE = 3
STREAM_H = 4
STREAM_BIAS = 5
STREAM_RANK = 6


@dataclasses.dataclass(frozen=True)
class Config:
    seed: int           # seed stream of the recipe (part of every draw's seed)
    name: str
    hidden: int
    inter: int
    num_experts: int
    top_k: int
    num_shared: int
    fmt: str            # "f32" | "mxfp8" | "mxfp4" | "fp8_blk128"
    act: str            # "f32" | "bf16"
    routing: str        # "softmax_normal" | "uniform" | "biased" | "zipf"
    zipf_s: float = 0.0
    batches: tuple = ()
    blocks: tuple = ()
    tag: int = 0        # distinguishes reduced-size test variants of a recipe

    @property
    def experts_total(self):
        return self.num_experts + self.num_shared

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


TINY_FP32 = Config(1, "tiny_fp32", 256, 128, 8, 2, 0, "f32", "f32", "softmax_normal",
                   batches=(4,), blocks=(16,))
QWEN3_DECODE_MXFP8 = Config(2, "qwen3_decode_mxfp8", 2048, 768, 128, 8, 0, "mxfp8", "bf16",
                            "uniform", batches=(1, 4, 8, 16, 32))
DEEPSEEK_V3_FP8_BLK128 = Config(3, "deepseek_v3_fp8_blk128", 7168, 2048, 256, 8, 1, "fp8_blk128",
                                "bf16", "biased", batches=(1, 16, 64, 256))
PREFILL_ZIPF_MXFP8 = Config(4, "prefill_zipf_mxfp8", 4096, 1536, 256, 8, 0, "mxfp8", "bf16",
                            "zipf", zipf_s=1.1, batches=(16384,), blocks=(64, 128))
MXFP4_SWEEP = Config(5, "mxfp4_sweep", 4096, 1536, 128, 8, 0, "mxfp4", "bf16", "uniform",
                     zipf_s=1.2, batches=(1, 2, 8, 32, 64, 128, 256))

# by workload name
CONFIGS = {c.name: c for c in (TINY_FP32, QWEN3_DECODE_MXFP8, DEEPSEEK_V3_FP8_BLK128,
                               PREFILL_ZIPF_MXFP8, MXFP4_SWEEP)}


def rng(cfg, stream, *index):
    ss = np.random.SeedSequence([cfg.seed, cfg.tag, stream] + [int(i) for i in index])
    return np.random.Generator(np.random.PCG64(ss))


# --------------------------------------------------------------------------
# weight encodings (storage formats of the synthetic weights)
# --------------------------------------------------------------------------

def _block_exponent(amax, emax):
    _, ex = np.frexp(amax.astype(np.float32))
    e = ex.astype(np.int32) - 1 - emax
    e = np.where(amax == 0, -127, e)
    return np.clip(e, -127, 127).astype(np.int32)


def encode_mxfp8(w):
    """float32 [..., K] -> (E4M3 codes uint8 [..., K], E8M0 bytes [..., K/32])."""
    k = w.shape[-1]
    b = w.reshape(w.shape[:-1] + (k // 32, 32))
    e = _block_exponent(np.max(np.abs(b), axis=-1), 8)
    scaled = np.clip(b * np.ldexp(np.float32(1), -e)[..., None], -448.0, 448.0)
    q = torch.from_numpy(np.ascontiguousarray(scaled, dtype=np.float32)).to(torch.float8_e4m3fn)
    codes = q.view(torch.uint8).numpy().reshape(w.shape)
    return codes, (e + 127).astype(np.uint8)


_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float32)


def encode_mxfp4(w):
    """float32 [..., K] -> (packed E2M1 bytes [..., K/2], E8M0 bytes [..., K/32])."""
    k = w.shape[-1]
    b = w.reshape(w.shape[:-1] + (k // 32, 32))
    e = _block_exponent(np.max(np.abs(b), axis=-1), 2)
    scaled = b * np.ldexp(np.float32(1), -e)[..., None]
    a = np.minimum(np.abs(scaled), 6.0)
    hi = np.clip(np.searchsorted(_E2M1_MAG, a, side="left"), 0, 7)
    lo = np.clip(hi - 1, 0, 7)
    d_lo = a - _E2M1_MAG[lo]
    d_hi = _E2M1_MAG[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    codes = np.where(np.signbit(scaled), mag | 8, mag).astype(np.uint8).reshape(w.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def encode_fp8_blk128(w):
    """float32 [R][K] (R, K multiples of 128) -> (E4M3 codes [R][K],
    float32 scales [R/128][K/128])."""
    r, k = w.shape
    t = w.reshape(r // 128, 128, k // 128, 128)
    amax = np.max(np.abs(t), axis=(1, 3))
    s = np.where(amax == 0, np.float32(1), (amax / np.float32(448.0)).astype(np.float32))
    scaled = np.clip(t / s[:, None, :, None], -448.0, 448.0).astype(np.float32)
    q = torch.from_numpy(np.ascontiguousarray(scaled)).to(torch.float8_e4m3fn)
    codes = q.view(torch.uint8).numpy().reshape(r, k)
    return codes, s.astype(np.float32)


def _encode(fmt, w):
    if fmt == "f32":
        return w.astype(np.float32), None
    if fmt == "mxfp8":
        return encode_mxfp8(w)
    if fmt == "mxfp4":
        return encode_mxfp4(w)
    if fmt == "fp8_blk128":
        if w.ndim == 3:
            parts = [encode_fp8_blk128(w[p]) for p in range(w.shape[0])]
            return np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts])
        return encode_fp8_blk128(w)
    raise ValueError(fmt)


def expert(cfg, e):
    """Raw stored arrays of expert e (e == num_experts is the shared expert):
    w13 [2][I][H*] (gate = 0, up = 1), w2 [H][I*], and per-format scales."""
    g = rng(cfg, STREAM_WEIGHTS, e)
    h, i = cfg.hidden, cfg.inter
    w13 = g.standard_normal((2, i, h), dtype=np.float32) * np.float32(1.0 / np.sqrt(h))
    w2 = g.standard_normal((h, i), dtype=np.float32) * np.float32(1.0 / np.sqrt(i))
    q13, s13 = _encode(cfg.fmt, w13)
    q2, s2 = _encode(cfg.fmt, w2)
    return {"w13": q13, "w13_scale": s13, "w2": q2, "w2_scale": s2}


def weight_shapes(cfg):
    """Shapes/dtypes of the stacked arrays [E+S][...]."""
    n, h, i = cfg.experts_total, cfg.hidden, cfg.inter
    if cfg.fmt == "f32":
        return {"w13": ((n, 2, i, h), np.float32), "w2": ((n, h, i), np.float32)}
    if cfg.fmt == "mxfp8":
        return {"w13": ((n, 2, i, h), np.uint8), "w13_scale": ((n, 2, i, h // 32), np.uint8),
                "w2": ((n, h, i), np.uint8), "w2_scale": ((n, h, i // 32), np.uint8)}
    if cfg.fmt == "mxfp4":
        return {"w13": ((n, 2, i, h // 2), np.uint8), "w13_scale": ((n, 2, i, h // 32), np.uint8),
                "w2": ((n, h, i // 2), np.uint8), "w2_scale": ((n, h, i // 32), np.uint8)}
    if cfg.fmt == "fp8_blk128":
        return {"w13": ((n, 2, i, h), np.uint8),
                "w13_scale": ((n, 2, i // 128, h // 128), np.float32),
                "w2": ((n, h, i), np.uint8), "w2_scale": ((n, h // 128, i // 128), np.float32)}
    raise ValueError(cfg.fmt)


def all_experts(cfg, threads=None):
    """Stacked arrays of every expert, generated in parallel threads (numpy's
    generators release the GIL while filling)."""
    shapes = weight_shapes(cfg)
    out = {k: np.empty(s, dtype=d) for k, (s, d) in shapes.items()}
    threads = threads or min(16, os.cpu_count() or 1)

    def one(e):
        raw = expert(cfg, e)
        for k in out:
            out[k][e] = raw[k]

    with _cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(one, range(cfg.experts_total)))
    for k in ("w13_scale", "w2_scale"):
        out.setdefault(k, None)
    return out


# --------------------------------------------------------------------------
# activations, routing, standalone intermediates
# --------------------------------------------------------------------------

def to_bf16_bits(v):
    """float32 -> BF16 bit patterns (uint16), round to nearest even (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def activations(cfg, t, variant=0):
    """x [T][H] ~ N(0,1): float32 ("f32") or BF16 bit patterns ("bf16")."""
    x = rng(cfg, STREAM_X, t, variant).standard_normal((t, cfg.hidden), dtype=np.float32)
    return x if cfg.act == "f32" else to_bf16_bits(x)


def hidden_states(cfg, t, dtype="f32", variant=0):
    """A stand-alone h [T][k+S][I] ~ N(0,1) for testing the down product by
    itself: float32, or BF16 bit patterns."""
    h = rng(cfg, STREAM_H, t, variant).standard_normal(
        (t, cfg.top_k + cfg.num_shared, cfg.inter), dtype=np.float32)
    return h if dtype == "f32" else to_bf16_bits(h)


def mxfp8_rows(cfg, n, k, variant=0, scale=1.0):
    """Random MXFP8 activation rows [n][k] (E4M3 codes + E8M0 bytes per 32),
    encoded from N(0, scale^2) draws; for exercising the grouped GEMMs on
    their own."""
    v = rng(cfg, STREAM_H, n, k, variant).standard_normal((n, k), dtype=np.float32)
    return encode_mxfp8(v * np.float32(scale))


def _softmax(z):
    z = z - np.max(z, axis=-1, keepdims=True)
    p = np.exp(z)
    return p / np.sum(p, axis=-1, keepdims=True)


def _top_k(scores, k):
    idx = np.argsort(-scores, axis=-1, kind="stable")[:, :k]
    return idx


def gating_scores(cfg, t, kind=None, variant=0):
    """Gating scores of T tokens over the routed experts: (scores float32
    [T][E], bias float32 [E] or None).  Selection uses scores + bias.
      softmax_normal / biased: scores ~ N(0,1) (biased: bias ~ N(0, 0.5));
      uniform: scores ~ U(0,1);
      zipf: log p(e) + Gumbel noise with p(e) ~ rank(e)^-s over a seeded
            permutation of ranks (top-k of these is sampling k experts without
            replacement from the Zipf popularity)."""
    kind = kind or cfg.routing
    g = rng(cfg, STREAM_ROUTE, t, variant, {"softmax_normal": 0, "uniform": 1, "biased": 2,
                                            "zipf": 3}[kind])
    e = cfg.num_experts
    bias = None
    if kind in ("softmax_normal", "biased"):
        scores = g.standard_normal((t, e))
        if kind == "biased":
            bias = rng(cfg, STREAM_BIAS).normal(0.0, np.sqrt(0.5), size=e).astype(np.float32)
    elif kind == "uniform":
        scores = g.random((t, e))
    elif kind == "zipf":
        s = cfg.zipf_s or 1.1
        rank = rng(cfg, STREAM_RANK).permutation(e) + 1        # hot experts scattered
        logp = -s * np.log(rank.astype(np.float64))
        scores = logp[None, :] + g.gumbel(size=(t, e))
    else:
        raise ValueError(kind)
    return scores.astype(np.float32), bias


def routing(cfg, t, kind=None, variant=0):
    """(topk_ids int32 [T][k], topk_weights float32 [T][k]) for the routed
    slots, synthesised from gating_scores(): the k largest scores + bias
    (stable: ties to the lower index), weighted by a softmax over the
    selected raw scores.  The shared expert's slot is implied, not listed."""
    scores, bias = gating_scores(cfg, t, kind, variant)
    key = scores if bias is None else scores + bias[None, :]
    idx = _top_k(key, cfg.top_k)
    w = _softmax(np.take_along_axis(scores, idx, axis=1).astype(np.float64))
    return idx.astype(np.int32), w.astype(np.float32)


def touched_experts(cfg, ids):
    """Distinct experts a batch touches (the shared one included)."""
    u = set(np.unique(ids).tolist())
    if cfg.num_shared:
        u.add(cfg.num_experts)
    return sorted(u)


def expert_bytes(cfg):
    """Stored bytes of one expert (weights + scales)."""
    tot = 0
    for k, (shape, dt) in weight_shapes(cfg).items():
        tot += int(np.prod(shape[1:])) * np.dtype(dt).itemsize
    return tot
