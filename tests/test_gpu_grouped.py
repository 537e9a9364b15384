"""Expert-centric path on the GPU: MXFP8 activation quantiser (bit-exact),
grouped gate_up and down GEMMs on block-scaled MFMA, the ordered combine,
and moe_layer(GROUPED) against the float64 oracle in mode "mxfp8"."""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import align_sort as A
from oracle import formats as F
from oracle import layer as L
from _helpers import (assert_layer_close, device_routing, device_weights, expert_getter, inputs,
                      metrics, oracle_kw, to_device_x, to_f64)

pytestmark = pytest.mark.gpu

SMALL = {
    "mxfp8": W.PREFILL_ZIPF_MXFP8.replace(num_experts=8, tag=31),
    "mxfp4": W.MXFP4_SWEEP.replace(num_experts=8, tag=32),
    "fp8_blk128": W.DEEPSEEK_V3_FP8_BLK128.replace(num_experts=6, tag=33),
    # E2M1 rows with H not a multiple of 256: the 32-row gate_up tile keeps
    # 128-K stages (half-line weight slices) instead of 256-K ones, and the
    # last 512-row down tile is partial
    "mxfp4_h3968": W.MXFP4_SWEEP.replace(hidden=3968, num_experts=8, tag=34),
}


def _bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def test_quant_rows_all_bf16_values_bit_exact(lib):
    """Every finite BF16 value, in blocks whose maxima vary, quantises exactly
    as the oracle's MX quantiser does (codes and scale bytes); each token row
    is quantised once, in place of a gathered copy per slot."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = F.decode_bf16(bits)
    bits = bits[np.isfinite(vals)]
    rng = np.random.default_rng(7)
    perm = bits[rng.permutation(len(bits))]
    h = 4096
    rows = -(-len(perm) // h)
    x = np.zeros(rows * h, dtype=np.uint16)
    x[: len(perm)] = perm
    x = x.reshape(rows, h)
    x[-1, -64:] = 0                          # an all-zero block
    x[-1, -96] = 0x0001                      # a block holding only a subnormal
    xq, xs = lib.quant_rows(_bf16_tensor(x))
    torch.cuda.synchronize()
    codes, scales = F.quantize_mx_e4m3(F.decode_bf16(x))
    assert np.array_equal(xq.cpu().numpy(), codes)
    assert np.array_equal(xs.cpu().numpy(), scales)


def test_quant_rows_f32_input(lib):
    """FP32 rows: the same rule on float32 values (a float32 value divided by
    a power of two stays exact, so the oracle's float64 rule applies)."""
    rng = np.random.default_rng(8)
    x = (rng.standard_normal((37, 512)) * np.exp(rng.uniform(-20, 20, (37, 1)))).astype(np.float32)
    x[5, :32] = 0.0
    xq, xs = lib.quant_rows(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    codes, scales = F.quantize_mx_e4m3(x.astype(np.float64))
    assert np.array_equal(xq.cpu().numpy(), codes)
    assert np.array_equal(xs.cpu().numpy(), scales)


def _blocks_for(lib, ids, n_exp, bs):
    sort = lib.align_sort(torch.from_numpy(ids).cuda(), n_exp, 0, bs)
    torch.cuda.synchronize()
    return sort


@pytest.mark.parametrize("fmt,bs", [("mxfp8", 64), ("mxfp8", 128), ("mxfp8", 32), ("mxfp4", 128),
                                    ("mxfp4", 32), ("fp8_blk128", 128),
                                    ("mxfp4", 64), ("fp8_blk128", 32), ("fp8_blk128", 64)])
def test_grouped_gate_up_alone(lib, fmt, bs):
    """a7 on generator-made MXFP8 token rows, two slots per token: every sorted
    row reads its token's row (entry / slots), and h = SiLU(Wg a) * (Wu a) per
    block's expert is requantised as hi = Q(h), lo = Q(h - hi).  The matrix
    core accumulates with ~5e-5 relative error, so single codes may differ
    from the float64 oracle's; hi + lo tracks h to ~2^-9 whatever hi chose."""
    cfg = SMALL[fmt].replace(num_shared=0)
    rng = np.random.default_rng(3)
    t, slots = 75, 2
    ids = np.stack([rng.permutation(cfg.num_experts)[:slots] for _ in range(t)]).astype(np.int32)
    sort = _blocks_for(lib, ids, cfg.num_experts, bs)
    cap = sort["capacity"]
    xq_np, xs_np = W.mxfp8_rows(cfg, t, cfg.hidden)
    Wd = device_weights(cfg)
    hq, hs = lib.grouped_gate_up(Wd, torch.from_numpy(xq_np).cuda(), torch.from_numpy(xs_np).cuda(),
                                 t, slots, sort["sorted_token_ids"], sort["expert_ids"],
                                 sort["num_tokens_post_padded"], cap, bs)
    torch.cuda.synchronize()
    ref = A.align_sort(ids.reshape(-1), cfg.num_experts, bs)
    npp = ref["num_tokens_post_padded"]
    srt = np.asarray(ref["sorted_token_ids"][:npp])
    real = srt < t * slots                   # padding rows carry no token
    get = expert_getter(cfg)
    a_tok = F.dequant_mx(xq_np, xs_np, "e4m3")
    hq_np, hs_np = hq.cpu().numpy(), hs.cpu().numpy()
    hi = F.dequant_mx(hq_np[0, :npp], hs_np[0, :npp], "e4m3")[real]
    got = hi + F.dequant_mx(hq_np[1, :npp], hs_np[1, :npp], "e4m3")[real]
    want = np.zeros((npp, cfg.inter))
    for b, e in enumerate(ref["expert_ids"]):
        wg, wu, _ = L.dequant_expert(cfg.fmt, get(int(e)))
        rows = np.arange(b * bs, (b + 1) * bs)
        rows = rows[real[rows]]
        a = a_tok[srt[rows] // slots]
        want[rows] = L.silu(a @ wg.T) * (a @ wu.T)
    want = want[real]
    hq_hi = hq_np[0, :npp][real]
    # against the oracle's own two-term form of its float64 h: each side is
    # within half a lo step of its own h (<= 2^-9 of the element, 2^-6 of the
    # block maximum), and where accumulation noise flips a hi code the two lo
    # terms differ too, so a row may reach about 2 * 2^-9
    m = metrics(got, F.fake_quant_mx_e4m3_two_term(want))
    assert m["min_cos"] > 0.99999 and m["max_rel_l2"] < 4e-3, m
    # against the unquantised h: the lo term's own MX step (~2e-3 relative)
    m = metrics(got, want)
    assert m["min_cos"] > 0.99998 and m["max_rel_l2"] < 6e-3, m
    # the hi term alone is the single requantisation (about 2^-5 relative)
    assert 5e-3 < metrics(hi, want)["rel_l2"] < 0.05
    # hi codes agree with the oracle's Q(h) except where h sits within the
    # accumulation error of a rounding boundary
    ch, _ = F.quantize_mx_e4m3(want)
    assert np.mean(hq_hi == ch) > 0.99


@pytest.mark.parametrize("fmt,bs", [("mxfp8", 64), ("mxfp4", 128), ("fp8_blk128", 64), ("mxfp8", 128),
                                    ("mxfp8", 32), ("mxfp4", 64),
                                    ("fp8_blk128", 128)])
def test_grouped_down_alone(lib, fmt, bs):
    """a8 on generator-made two-term MXFP8 h: slot_out[i] = BF16(w_i * Wd (hi + lo))
    for every real (non-padding) sorted row; padding rows write nothing."""
    cfg = SMALL[fmt].replace(num_shared=0, top_k=2)
    t = 70
    _, ids, w = inputs(cfg, t)
    sort = _blocks_for(lib, ids, cfg.num_experts, bs)
    cap = sort["capacity"]
    hi_q, hi_s = W.mxfp8_rows(cfg, cap, cfg.inter, scale=0.3)
    lo_q, lo_s = W.mxfp8_rows(cfg, cap, cfg.inter, variant=1, scale=0.01)
    hq_np, hs_np = np.stack([hi_q, lo_q]), np.stack([hi_s, lo_s])
    Wd = device_weights(cfg)
    idd, wd = device_routing(ids, w)
    so = torch.full((t * cfg.top_k, cfg.hidden), float("nan"), device="cuda", dtype=torch.bfloat16)
    lib.grouped_down(Wd, torch.from_numpy(hq_np).cuda(), torch.from_numpy(hs_np).cuda(),
                     sort["sorted_token_ids"], sort["expert_ids"], sort["num_tokens_post_padded"],
                     cap, bs, wd, t, cfg.top_k, slot_out=so)
    torch.cuda.synchronize()
    ref = A.align_sort(ids.reshape(-1), cfg.num_experts, bs)
    get = expert_getter(cfg)
    h = F.dequant_mx(hi_q, hi_s, "e4m3") + F.dequant_mx(lo_q, lo_s, "e4m3")
    want = np.zeros((t * cfg.top_k, cfg.hidden))
    for b, e in enumerate(ref["expert_ids"]):
        _, _, wdn = L.dequant_expert(cfg.fmt, get(int(e)))
        for r in range(b * bs, (b + 1) * bs):
            ent = ref["sorted_token_ids"][r]
            if ent < t * cfg.top_k:
                want[ent] = (wdn @ h[r]) * float(w.reshape(-1)[ent])
    got = to_f64(so)
    assert np.isfinite(got).all()           # every slot row written exactly by its sorted row
    # exact products (E4M3 x E4M3/E2M1 with power-of-two scales), FP32
    # accumulation over I terms inside the matrix core (~1e-5 relative), then
    # one BF16 rounding on each side: almost every value is the oracle's BF16
    # value itself, the rest are one BF16 step away
    want = F.round_to_bf16(want)
    same = np.mean(got == want)
    assert same > 0.98, same
    m = metrics(got, want)
    assert m["min_cos"] > 0.999999 and m["max_rel_l2"] < 1e-3, m


def test_combine_slot_order(lib):
    t, slots, h = 37, 9, 2048
    rng = np.random.default_rng(11)
    sob = torch.from_numpy(rng.standard_normal((t * slots, h)).astype(np.float32)).to(torch.bfloat16)
    so = sob.to(torch.float32).numpy()      # the BF16 slot values, exactly
    y = lib.combine(sob.cuda(), t, slots)
    yb = lib.combine(sob.cuda(), t, slots, y_dtype="bf16")
    torch.cuda.synchronize()
    want = np.zeros((t, h), dtype=np.float32)
    for j in range(slots):                   # float32 sums in slot order
        want = want + so.reshape(t, slots, h)[:, j]
    assert np.array_equal(y.cpu().numpy(), want)
    assert torch.equal(yb.cpu().view(torch.int16),
                       torch.from_numpy(want).to(torch.bfloat16).view(torch.int16))


def _grouped_layer(lib, cfg, t, bs, kind=None):
    x, ids, w = inputs(cfg, t, kind=kind)
    Wd = device_weights(cfg)
    y, chosen = lib.layer(Wd, to_device_x(cfg, x), *device_routing(ids, w), path="grouped",
                          block=bs)
    torch.cuda.synchronize()
    assert chosen == "grouped"
    return x, ids, w, to_f64(y)


@pytest.mark.parametrize("fmt,t,bs", [("mxfp8", 40, 64), ("mxfp4", 33, 32), ("fp8_blk128", 21, 32),
                                      ("fp8_blk128", 150, 128), ("mxfp4", 170, 128), ("mxfp8", 1, 32),
                                      ("mxfp8", 300, 128), ("mxfp4_h3968", 33, 32)])
def test_grouped_layer_small(lib, fmt, t, bs):
    cfg = SMALL[fmt]
    x, ids, w, y = _grouped_layer(lib, cfg, t, bs)
    kw = oracle_kw(cfg)
    x64 = L.activations_f64(x, cfg.act)
    y_ref = L.moe_layer(x64, ids, w, act_quant="mxfp8", **kw)
    assert_layer_close(y, y_ref, (fmt, t, bs))
    # the same layer without activation quantisation is further away (the
    # grouped path really quantises, as the expert-centric design does)
    y_none = L.moe_layer(x64, ids, w, **kw)
    assert metrics(y, y_none)["rel_l2"] > metrics(y, y_ref)["rel_l2"]


def test_grouped_block_size_does_not_change_the_bits(lib):
    """Every output element is accumulated over K in the same order whatever
    the tile, so the layer is bit for bit the same with 32, 64 and 128-row
    blocks."""
    cfg = SMALL["mxfp8"]
    x, ids, w = inputs(cfg, 600)
    Wd = device_weights(cfg)
    xd = to_device_x(cfg, x)
    idd, wd = device_routing(ids, w)
    ys = [lib.layer(Wd, xd, idd, wd, path="grouped", block=bs)[0] for bs in (32, 64, 128)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(ys[0], y)


def test_grouped_layer_deterministic(lib):
    cfg = SMALL["mxfp8"]
    _, _, _, y1 = _grouped_layer(lib, cfg, 100, 64)
    _, _, _, y2 = _grouped_layer(lib, cfg, 100, 64)
    assert np.array_equal(y1, y2)


GROUPED_FULL = [("prefill_zipf_mxfp8", 16384, 128, "zipf"), ("prefill_zipf_mxfp8", 16384, 64, "zipf"),
                ("mxfp4_sweep", 256, 64, None), ("deepseek_v3_fp8_blk128", 256, 32, None)]


@pytest.mark.parametrize("name,t,bs,kind", GROUPED_FULL)
def test_grouped_layer_full_size_sampled(lib, name, t, bs, kind):
    cfg = W.CONFIGS[name]
    x, ids, w, y = _grouped_layer(lib, cfg, t, bs, kind=kind)
    sample = sorted({0, 1, t // 3, t // 2, t - 1})
    x64 = L.activations_f64(x[sample], cfg.act)
    ref = L.moe_layer(x64, ids[sample], w[sample], act_quant="mxfp8", **oracle_kw(cfg))
    assert_layer_close(y[sample], ref, (name, t, bs))


@pytest.mark.parametrize("t,want", [(8, "decode"), (200, "grouped")])
def test_layer_auto_matches_the_oracle_mode_of_its_path(lib, t, want):
    """moe_layer(AUTO) on the Qwen3-style layer picks output-centric decode at
    a small batch and expert-centric packing at a large one; each result is
    held to the oracle in the mode of the path it reports (decode: float64
    activations; grouped: MXFP8 activations and two-term h)."""
    cfg = W.QWEN3_DECODE_MXFP8
    x, ids, w = inputs(cfg, t)
    Wd = device_weights(cfg)
    assert lib.choose_path(Wd, t, cfg.top_k) == want
    y, chosen = lib.layer(Wd, to_device_x(cfg, x), *device_routing(ids, w), path="auto")
    torch.cuda.synchronize()
    assert chosen == want
    sample = sorted({0, t // 2, t - 1})
    x64 = L.activations_f64(x[sample], cfg.act)
    mode = "none" if chosen == "decode" else "mxfp8"
    ref = L.moe_layer(x64, ids[sample], w[sample], act_quant=mode, **oracle_kw(cfg))
    assert_layer_close(to_f64(y)[sample], ref, (t, chosen))


@pytest.mark.parametrize("t,bs", [(1, 32), (40, 64), (1100, 128)])
def test_layer_front_end_matches_the_separate_calls(lib, t, bs):
    """moe_layer's grouped front end (the sort and the token quantisation in
    one launch up to 8192 entries, separate launches beyond: 1100 tokens x 8
    slots here) gives the bits of the separate entry points."""
    cfg = SMALL["mxfp8"]
    x, ids, w = inputs(cfg, t)
    Wd = device_weights(cfg)
    xd = to_device_x(cfg, x)
    idd, wd = device_routing(ids, w)
    y, chosen = lib.layer(Wd, xd, idd, wd, path="grouped", block=bs)
    k, S = cfg.top_k, cfg.num_shared
    srt = lib.align_sort(idd, cfg.num_experts, S, bs)
    xq, xs = lib.quant_rows(xd)
    cap = lib.align_sort_capacity(t, k, cfg.num_experts, S, bs)
    hq, hs = lib.grouped_gate_up(Wd, xq, xs, t, k, srt["sorted_token_ids"], srt["expert_ids"],
                                 srt["num_tokens_post_padded"], cap, bs)
    so = lib.grouped_down(Wd, hq, hs, srt["sorted_token_ids"], srt["expert_ids"],
                          srt["num_tokens_post_padded"], cap, bs, wd, t, k)
    y_sep = lib.combine(so, t, k + S)
    torch.cuda.synchronize()
    assert chosen == "grouped" and torch.equal(y, y_sep)
