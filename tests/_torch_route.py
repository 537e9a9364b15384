"""An independent route to the expert-centric numerics, for pinning the
oracle: MX quantisation through torch's own float8 casts and numpy's log2,
weights decoded through torch's float8 / e8m0 dtypes (and the OCP E2M1 value
table stored under tests/golden/), BF16 rounding through torch's bfloat16
cast, and the layer through torch float64 matmul and silu.

Nothing here imports the oracle; the tests compare the two.
"""

import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _e2m1_table():
    vals = np.zeros(16)
    with open(os.path.join(GOLDEN, "e2m1_ocp_values.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                vals[int(c, 16)] = float(v)
    return vals


E2M1 = _e2m1_table()


def e4m3_bytes_to_f64(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def e8m0_bytes_to_f64(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e8m0fnu).to(torch.float64).numpy()


def mx_exponent(amax):
    """floor(log2 amax) - 8 by numpy's log2, clamped to [-127, 127]; -127
    for an all-zero block."""
    safe = np.where(amax > 0, amax, 1.0)
    e = np.floor(np.log2(safe)).astype(np.int64) - 8
    return np.clip(np.where(amax > 0, e, -127), -127, 127)


def mx_quant(v):
    """Blocks of 32 along the last axis -> (codes, scale bytes) via torch's
    float8_e4m3fn cast of the saturated, scaled values."""
    v = np.asarray(v, dtype=np.float64)
    b = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    e = mx_exponent(np.abs(b).max(-1))
    s = np.clip(b / np.exp2(e.astype(np.float64))[..., None], -448.0, 448.0)
    codes = torch.from_numpy(s).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes.reshape(v.shape), (e + 127).astype(np.uint8)


def mx_dequant_e4m3(codes, scales):
    return e4m3_bytes_to_f64(codes) * np.repeat(e8m0_bytes_to_f64(scales), 32, axis=-1)


def mx_fake(v):
    return mx_dequant_e4m3(*mx_quant(v))


def mx_fake_two_term(v):
    hi = mx_fake(v)
    return hi + mx_fake(np.asarray(v, dtype=np.float64) - hi)


def to_bf16(v):
    """float64 -> BF16 value through torch's cast (float64 -> float32 ->
    bfloat16); the intermediate float32 rounding lands on a BF16 midpoint
    with probability about 2^-16 per value."""
    return torch.from_numpy(np.asarray(v, dtype=np.float64)).float().bfloat16().double().numpy()


def dequant_weights(fmt, raw):
    """One expert's raw arrays -> (Wg, Wu, Wd) float64 by the torch dtypes."""
    if fmt == "f32":
        w13 = np.asarray(raw["w13"], dtype=np.float32).astype(np.float64)
        w2 = np.asarray(raw["w2"], dtype=np.float32).astype(np.float64)
    elif fmt == "mxfp8":
        w13 = mx_dequant_e4m3(raw["w13"], raw["w13_scale"])
        w2 = mx_dequant_e4m3(raw["w2"], raw["w2_scale"])
    elif fmt == "mxfp4":
        def fp4(p, s):
            p = np.asarray(p, dtype=np.uint8)
            codes = np.stack([p & 0xF, p >> 4], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))
            return E2M1[codes] * np.repeat(e8m0_bytes_to_f64(s), 32, axis=-1)
        w13 = fp4(raw["w13"], raw["w13_scale"])
        w2 = fp4(raw["w2"], raw["w2_scale"])
    elif fmt == "fp8_blk128":
        def blk(c, s):
            s = np.asarray(s, dtype=np.float32).astype(np.float64)
            s = np.repeat(np.repeat(s, 128, axis=-2), 128, axis=-1)
            return e4m3_bytes_to_f64(c) * s[..., : c.shape[-2], : c.shape[-1]]
        w13 = blk(raw["w13"], raw["w13_scale"])
        w2 = blk(raw["w2"], raw["w2_scale"])
    else:
        raise ValueError(fmt)
    return w13[0], w13[1], w2


def expert_centric_layer(x, ids, w, *, fmt, num_experts, num_shared, get_expert, terms):
    """The expert-centric numerics, token by token and slot by slot: x -> its
    MX form, h = silu(Wg a) * (Wu a) by torch float64 ops, h -> its MX form
    with `terms` terms (1 or 2), each slot's w * (Wd h) rounded to BF16, then
    the slot-order sum in float64."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(w, dtype=np.float32).astype(np.float64)
    t_n, k = ids.shape
    a = torch.from_numpy(mx_fake(x))
    y = np.zeros(x.shape)
    cache = {}
    for t in range(t_n):
        slots = [(int(ids[t, j]), float(w[t, j])) for j in range(k)]
        slots += [(num_experts, 1.0)] * num_shared
        acc = np.zeros(x.shape[1])
        for e, wt in slots:
            if e not in cache:
                cache[e] = [torch.from_numpy(m) for m in dequant_weights(fmt, get_expert(e))]
            wg, wu, wd = cache[e]
            at = a[t:t + 1]
            h = (torch.nn.functional.silu(at @ wg.T) * (at @ wu.T)).numpy()
            hq = mx_fake_two_term(h) if terms == 2 else mx_fake(h)
            c = (torch.from_numpy(hq) @ wd.T).numpy()[0] * wt
            acc = acc + to_bf16(c)
        y[t] = acc
    return y
