"""Pins of oracle/layer.py: brute force with exactly rounded sums, the dense
SwiGLU FFN computed with torch library routines, a closed form, and
invariants (linearity in the routing weights, slot permutation, zero
weights, zero inputs)."""

import functools
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import layer as L
from oracle import formats as F

TINY = {
    "f32": W.TINY_FP32,
    "mxfp8": W.QWEN3_DECODE_MXFP8.replace(hidden=64, inter=64, num_experts=4, top_k=2, tag=11),
    "mxfp4": W.MXFP4_SWEEP.replace(hidden=64, inter=64, num_experts=4, top_k=2, tag=12),
    "fp8_blk128": W.DEEPSEEK_V3_FP8_BLK128.replace(hidden=256, inter=128, num_experts=4, top_k=2, num_shared=0,
                                        tag=13),
}


def _getter(cfg):
    return functools.lru_cache(maxsize=None)(lambda e: W.expert(cfg, e))


def _inputs(cfg, t):
    x = L.activations_f64(W.activations(cfg, t), cfg.act)
    ids, w = W.routing(cfg, t)
    return x, ids, w


def _kw(cfg, getter=None):
    return dict(fmt=cfg.fmt, num_experts=cfg.num_experts, num_shared=cfg.num_shared,
                get_expert=getter or _getter(cfg))


@pytest.mark.parametrize("fmt", list(TINY))
@pytest.mark.parametrize("mode", ["none", "mxfp8", "mxfp8_single"])
def test_vectorised_matches_scalar_brute_force(fmt, mode):
    cfg = TINY[fmt]
    t = 3 if fmt != "f32" else 4
    x, ids, w = _inputs(cfg, t)
    kw = _kw(cfg)
    y = L.moe_layer(x, ids, w, act_quant=mode, **kw)
    ys = L.moe_layer_scalar(x, ids, w, act_quant=mode, **kw)
    assert np.max(np.abs(y - ys)) <= 1e-12 * np.max(np.abs(ys))


def test_shared_expert_slot_scalar():
    cfg = TINY["fp8_blk128"].replace(num_shared=1)
    x, ids, w = _inputs(cfg, 2)
    kw = _kw(cfg)
    y = L.moe_layer(x, ids, w, **kw)
    ys = L.moe_layer_scalar(x, ids, w, **kw)
    assert np.max(np.abs(y - ys)) <= 1e-12 * np.max(np.abs(ys))


def _dense_ffn_torch(x, wg, wu, wd):
    xt = torch.from_numpy(x)
    g = torch.matmul(xt, torch.from_numpy(wg).T)
    u = torch.matmul(xt, torch.from_numpy(wu).T)
    return torch.matmul(torch.nn.functional.silu(g) * u, torch.from_numpy(wd).T).numpy()


@pytest.mark.parametrize("fmt", list(TINY))
def test_identical_experts_equal_dense_ffn(fmt):
    """All experts equal and weights summing to 1: the layer is one dense
    SwiGLU FFN (torch silu + matmul, float64)."""
    cfg = TINY[fmt]
    raw = W.expert(cfg, 0)
    x, ids, w = _inputs(cfg, 5)
    w = w / w.sum(axis=1, keepdims=True, dtype=np.float64)
    w = w.astype(np.float32)
    y = L.moe_layer(x, ids, w, **_kw(cfg, getter=lambda e: raw))
    wg, wu, wd = L.dequant_expert(cfg.fmt, raw)
    ref = _dense_ffn_torch(x, wg, wu, wd) * w.astype(np.float64).sum(axis=1, keepdims=True)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_shared_expert_adds_its_dense_ffn():
    cfg = TINY["fp8_blk128"]
    cfg_s = cfg.replace(num_shared=1)
    x, ids, w = _inputs(cfg, 3)
    get = _getter(cfg_s)
    y0 = L.moe_layer(x, ids, w, **_kw(cfg, getter=get))
    y1 = L.moe_layer(x, ids, w, **_kw(cfg_s, getter=get))
    wg, wu, wd = L.dequant_expert(cfg.fmt, get(cfg.num_experts))
    ref = _dense_ffn_torch(x, wg, wu, wd)
    assert np.max(np.abs((y1 - y0) - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_linear_in_weights_and_slot_permutation():
    cfg = TINY["mxfp8"]
    x, ids, w = _inputs(cfg, 4)
    kw = _kw(cfg)
    y = L.moe_layer(x, ids, w, **kw)
    y2 = L.moe_layer(x, ids, (2 * w).astype(np.float32), **kw)
    assert np.allclose(y2, 2 * y, rtol=0, atol=1e-13)
    perm = np.array([1, 0])
    yp = L.moe_layer(x, ids[:, perm], w[:, perm], **kw)
    assert np.allclose(yp, y, rtol=0, atol=1e-13)
    # additive in w over a split of the slots
    wa = w.copy()
    wa[:, 1] = 0
    wb = w.copy()
    wb[:, 0] = 0
    ya = L.moe_layer(x, ids, wa, **kw)
    yb = L.moe_layer(x, ids, wb, **kw)
    assert np.allclose(ya + yb, y, rtol=0, atol=1e-13)
    # a zero-weight slot contributes nothing: same as routing only slot 0
    y_one = L.moe_layer(x, ids[:, :1], w[:, :1], **kw)
    assert np.allclose(ya, y_one, rtol=0, atol=1e-15)


def test_zero_inputs():
    cfg = TINY["f32"]
    _, ids, w = _inputs(cfg, 4)
    kw = _kw(cfg)
    assert np.all(L.moe_layer(np.zeros((4, cfg.hidden)), ids, w, **kw) == 0)
    base = _getter(cfg)

    def no_gate(e):
        r = dict(base(e))
        w13 = r["w13"].copy()
        w13[0] = 0
        r["w13"] = w13
        return r

    x, _, _ = _inputs(cfg, 4)
    assert np.all(L.moe_layer(x, ids, w, **_kw(cfg, getter=no_gate)) == 0)


def test_closed_form_h1_i1():
    """H = I = 1: y = sum_j w_j d_j (g_j x) sigmoid(g_j x) (u_j x)."""
    gs, us, ds = [0.7, -1.3, 2.1], [0.4, 1.7, -0.6], [1.9, -0.8, 0.3]

    def get(e):
        return {"w13": np.array([[[gs[e]]], [[us[e]]]], dtype=np.float32),
                "w2": np.array([[ds[e]]], dtype=np.float32)}

    x = np.array([[1.25], [-0.5]])
    ids = np.array([[0, 2], [1, 0]], dtype=np.int32)
    w = np.array([[0.25, 0.75], [0.5, 0.5]], dtype=np.float32)
    y = L.moe_layer(x, ids, w, fmt="f32", num_experts=3, num_shared=0, get_expert=get)
    g32 = [float(np.float32(v)) for v in gs]
    u32 = [float(np.float32(v)) for v in us]
    d32 = [float(np.float32(v)) for v in ds]
    for t in range(2):
        ref = 0.0
        for j in range(2):
            e = ids[t, j]
            z = g32[e] * x[t, 0]
            ref += float(w[t, j]) * d32[e] * z / (1 + math.exp(-z)) * u32[e] * x[t, 0]
        assert abs(y[t, 0] - ref) <= 1e-15 * abs(ref)


def test_gate_up_then_down_is_the_layer():
    cfg = TINY["mxfp4"]
    x, ids, w = _inputs(cfg, 3)
    kw = _kw(cfg)
    h = L.gate_up(x, ids, **kw)
    assert np.allclose(L.down(h, ids, w, **kw), L.moe_layer(x, ids, w, **kw), rtol=0, atol=1e-13)
    hq = L.gate_up(x, ids, act_quant="mxfp8", **kw)
    assert np.allclose(L.down(hq, ids, w, act_quant="mxfp8", **kw),
                       L.moe_layer(x, ids, w, act_quant="mxfp8", **kw), rtol=0, atol=1e-13)


def test_mxfp8_mode_quantises_activations():
    """Mode mxfp8 equals mode none run on Q(x) with h replaced by its two-term
    MXFP8 form Q(h) + Q(h - Q(h)) and every slot's weighted output rounded to
    BF16 before the slot-order sum (each slot taken alone through mode none
    by zeroing the other slots' weights)."""
    cfg = TINY["mxfp8"]
    assert cfg.num_shared == 0
    x, ids, w = _inputs(cfg, 3)
    kw = _kw(cfg)
    xq = F.fake_quant_mx_e4m3(x)
    h = L.gate_up(xq, ids, **kw)
    hq = F.fake_quant_mx_e4m3(h)
    hh = hq + F.fake_quant_mx_e4m3(h - hq)
    y_ref = np.zeros((x.shape[0], cfg.hidden))
    for j in range(ids.shape[1]):
        wj = np.zeros_like(w)
        wj[:, j] = w[:, j]
        y_ref = y_ref + F.round_to_bf16(L.down(hh, ids, wj, **kw))
    assert np.allclose(L.moe_layer(x, ids, w, act_quant="mxfp8", **kw), y_ref, rtol=0, atol=1e-13)
    # and it differs from mode none (the quantisation is really applied)
    assert not np.allclose(L.moe_layer(x, ids, w, **kw), y_ref, rtol=0, atol=1e-6)


@pytest.mark.parametrize("fmt,shared", [("mxfp8", 0), ("mxfp4", 0), ("fp8_blk128", 0),
                                        ("fp8_blk128", 1), ("f32", 0)])
@pytest.mark.parametrize("mode,terms", [("mxfp8", 2), ("mxfp8_single", 1)])
def test_expert_centric_modes_match_an_independent_route(fmt, shared, mode, terms):
    """The MXFP8 modes' whole composition -- x quantised per 32 along H, h
    requantised per 32 along I with one or two terms, every slot's weighted
    output rounded to BF16, then the slot-order sum -- recomputed token by
    token through torch's float8_e4m3fn / float8_e8m0fnu / bfloat16 casts,
    numpy's log2, the OCP E2M1 table and torch float64 silu and matmul
    (tests/_torch_route.py, which does not import the oracle)."""
    import _torch_route as R
    cfg = TINY[fmt].replace(num_shared=shared)
    t = 4 if fmt != "f32" else 3
    x, ids, w = _inputs(cfg, t)
    get = _getter(cfg)
    y = L.moe_layer(x, ids, w, act_quant=mode, **_kw(cfg, getter=get))
    ref = R.expert_centric_layer(x, ids, w, fmt=cfg.fmt, num_experts=cfg.num_experts,
                                 num_shared=shared, get_expert=get, terms=terms)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref)), (fmt, mode)
    # the other term count is measurably different: the pin tells them apart
    other = R.expert_centric_layer(x, ids, w, fmt=cfg.fmt, num_experts=cfg.num_experts,
                                   num_shared=shared, get_expert=get, terms=3 - terms)
    assert np.max(np.abs(other - ref)) > 1e-6 * np.max(np.abs(ref))


def test_mxfp8_modes_are_the_documented_steps_of_each_other():
    """Mode mxfp8_single differs from mxfp8 only in the requantisation of h;
    the two-term form is within 2^-6 of each block maximum of h, the
    single-term one within 2^-4 relative of each normal element, so the
    two-term mode lies closer to the unquantised-h layer on Q(x)."""
    cfg = TINY["mxfp8"]
    x, ids, w = _inputs(cfg, 6)
    kw = _kw(cfg)
    xq = F.fake_quant_mx_e4m3(x)
    exact_h = L.moe_layer(xq, ids, w, **kw)          # Q(x), exact h, FP64 slots
    y1 = L.moe_layer(x, ids, w, act_quant="mxfp8_single", **kw)
    y2 = L.moe_layer(x, ids, w, act_quant="mxfp8", **kw)
    e1 = np.linalg.norm(y1 - exact_h) / np.linalg.norm(exact_h)
    e2 = np.linalg.norm(y2 - exact_h) / np.linalg.norm(exact_h)
    assert e2 < e1 / 4, (e1, e2)


def test_f64_weights_are_taken_as_given():
    """fmt "f64" hands over dequantised weights: the layer equals the one run
    on the stored format."""
    cfg = TINY["fp8_blk128"]
    x, ids, w = _inputs(cfg, 3)
    get = _getter(cfg)

    def get64(e):
        wg, wu, wd = L.dequant_expert(cfg.fmt, get(e))
        return {"w13": np.stack([wg, wu]), "w2": wd}
    for mode in L.MODES:
        y = L.moe_layer(x, ids, w, act_quant=mode, **_kw(cfg, getter=get))
        y64 = L.moe_layer(x, ids, w, act_quant=mode, fmt="f64", num_experts=cfg.num_experts,
                          num_shared=cfg.num_shared, get_expert=get64)
        assert np.array_equal(y, y64)
