"""Decode-path parity on the GPU: moe_gate_up / moe_down / moe_layer(DECODE)
against the float64 oracle (mode "none"), element by element for h and per
token for y (cosine >= 0.99999, relative L2 <= 5e-3), plus batch invariance,
run-to-run determinism and full-write checks."""

import functools

import numpy as np
import pytest
import torch

import workloads as W
from oracle import layer as L
from _helpers import (assert_layer_close, device_routing, device_weights, inputs, oracle_kw,
                      to_device_x, to_f64)

pytestmark = pytest.mark.gpu

# reduced-expert variants: full H and I (so rows span every lane and several
# chunks), fewer experts so the oracle stays fast; odd token counts give a
# ragged tail of (token, slot) entries
SMALL = {
    "f32": W.TINY_FP32,
    "mxfp8": W.QWEN3_DECODE_MXFP8.replace(num_experts=16, tag=21),
    "mxfp4": W.MXFP4_SWEEP.replace(num_experts=16, tag=22),
    "fp8_blk128": W.DEEPSEEK_V3_FP8_BLK128.replace(num_experts=12, tag=23),
    # MXFP8 rows spanning 32 lanes (I = 1536): the other conversion-once shape
    "mxfp8_i1536": W.PREFILL_ZIPF_MXFP8.replace(num_experts=16, tag=25),
    # H = 1024: gate_up rows of one chunk per lane (its scale dwords from 16 lanes)
    "mxfp8_h1024": W.QWEN3_DECODE_MXFP8.replace(hidden=1024, num_experts=16, tag=26),
    # E2M1 rows off the matrix-core kernel's grid (I not a multiple of 256):
    # both products run on the vector kernels, rows converted per token
    "mxfp4_i384": W.MXFP4_SWEEP.replace(inter=384, num_experts=16, tag=27),
    # rows that are not whole 64-lane passes of 16-byte chunks: the guarded
    # gate_up shape in every format (and down rows past the last full group)
    "mxfp8_h1056": W.QWEN3_DECODE_MXFP8.replace(hidden=1056, num_experts=16, tag=28),
    "f32_h200": W.TINY_FP32.replace(hidden=200, inter=96, tag=29),
    "fp8_blk128_h1152": W.DEEPSEEK_V3_FP8_BLK128.replace(hidden=1152, inter=256, num_experts=12,
                                                        tag=30),
    "mxfp4_h1088": W.MXFP4_SWEEP.replace(hidden=1088, inter=384, num_experts=16, tag=31),
    # long rows: 3, 5 and 8 chunks per lane (the guarded 4- and 8-chunk shapes
    # and the unguarded 8-chunk one, rows streamed without the BF16 copy)
    "mxfp8_h3072": W.QWEN3_DECODE_MXFP8.replace(hidden=3072, inter=256, num_experts=16, tag=32),
    "mxfp8_h5120": W.QWEN3_DECODE_MXFP8.replace(hidden=5120, inter=256, num_experts=16, tag=33),
    "mxfp8_h8192": W.QWEN3_DECODE_MXFP8.replace(hidden=8192, inter=256, num_experts=16, tag=34),
    "f32_h2048": W.TINY_FP32.replace(hidden=2048, inter=64, tag=35),
    "f32_h1536": W.TINY_FP32.replace(hidden=1536, inter=64, tag=36),
}


def _run_decode(moe, cfg, t, h_dtype="f32", y_dtype="f32", kind=None, variant=0):
    x, ids, w = inputs(cfg, t, kind=kind, variant=variant)
    Wd = device_weights(cfg)
    xd = to_device_x(cfg, x)
    idd, wd = device_routing(ids, w)
    h = moe.gate_up(Wd, xd, idd, h_dtype=h_dtype)
    y = moe.down(Wd, h, idd, wd, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return x, ids, w, h, y


def _oracle(cfg, x, ids, w):
    x64 = L.activations_f64(x, cfg.act)
    kw = oracle_kw(cfg)
    return L.gate_up(x64, ids, **kw), L.moe_layer(x64, ids, w, **kw)


@pytest.mark.parametrize("fmt", list(SMALL))
@pytest.mark.parametrize("t", [1, 5, 32])
def test_decode_parity_small(lib, fmt, t):
    cfg = SMALL[fmt]
    if fmt == "f32" and t == 32:
        t = 4
    x, ids, w, h, y = _run_decode(lib, cfg, t)
    h_ref, y_ref = _oracle(cfg, x, ids, w)
    hh = to_f64(h)
    # each h scalar: FP32 accumulation of exact products over H terms
    scale = np.sqrt(np.mean(h_ref ** 2))
    assert np.max(np.abs(hh - h_ref)) <= 2e-4 * scale + 1e-6, np.max(np.abs(hh - h_ref)) / scale
    assert_layer_close(to_f64(y), y_ref, (fmt, t))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "fp8_blk128", "mxfp4_i384"])
def test_decode_bf16_intermediate_and_output(lib, fmt):
    cfg = SMALL[fmt]
    x, ids, w, h, y = _run_decode(lib, cfg, 7, h_dtype="bf16", y_dtype="bf16")
    assert h.dtype == torch.bfloat16 and y.dtype == torch.bfloat16
    _, y_ref = _oracle(cfg, x, ids, w)
    assert_layer_close(to_f64(y), y_ref, fmt)


def test_down_alone_on_given_h(lib):
    """moe_down on a generated h (not one from moe_gate_up) against the
    oracle's down product of the same h."""
    cfg = SMALL["mxfp8"]
    t = 9
    _, ids, w = inputs(cfg, t)
    h = W.hidden_states(cfg, t)
    Wd = device_weights(cfg)
    idd, wd = device_routing(ids, w)
    y = lib.down(Wd, torch.from_numpy(h).cuda(), idd, wd)
    ref = L.down(h.astype(np.float64), ids, w, **oracle_kw(cfg))
    assert_layer_close(to_f64(y), ref)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "fp8_blk128", "mxfp4_i384"])
def test_batch_invariance_and_determinism(lib, fmt):
    """Each output is produced by one wavefront in a fixed order, so a token's
    h and y do not depend on the rest of the batch and repeat bit for bit
    (MXFP4 gate_up runs on the matrix cores: a token's MFMA column does not
    change its bits either).  AUTO runs the down product token-major for the
    single tokens and expert-major for the batch of 32 (for the
    DeepSeek-V3-shaped rows from two tokens on), so this also holds across
    the launch shapes."""
    cfg = SMALL[fmt]
    x, ids, w = inputs(cfg, 32)
    Wd = device_weights(cfg)
    xd = to_device_x(cfg, x)
    idd, wd = device_routing(ids, w)
    h_all = lib.gate_up(Wd, xd, idd)
    y_all = lib.down(Wd, h_all, idd, wd)
    h_again = lib.gate_up(Wd, xd, idd)
    y_again = lib.down(Wd, h_again, idd, wd)
    torch.cuda.synchronize()
    assert torch.equal(h_all, h_again) and torch.equal(y_all, y_again)
    for t in (0, 13, 31):
        h1 = lib.gate_up(Wd, xd[t:t + 1].contiguous(), idd[t:t + 1].contiguous())
        y1 = lib.down(Wd, h1, idd[t:t + 1].contiguous(), wd[t:t + 1].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(h1[0], h_all[t]) and torch.equal(y1[0], y_all[t]), t


# FP32 weights take an FP32 h only (the library refuses a BF16 one)
@pytest.mark.parametrize("fmt,h_dtype", [(f, hd) for f in SMALL for hd in ("f32", "bf16")
                                         if not (SMALL[f].fmt == "f32" and hd == "bf16")])
def test_down_variants_bitwise_identical(lib, fmt, h_dtype):
    """Token-major and expert-major down give the same bits (same per-slot
    lane groups and reduction tree, slots added in slot order) -- except
    MXFP4 rows with BF16 h, whose expert-major down runs on the matrix cores:
    the same exact products summed in another FP32 order."""
    cfg = SMALL[fmt]
    t = 3 if fmt == "f32" else 13
    x, ids, w = inputs(cfg, t)
    Wd = device_weights(cfg)
    idd, wd = device_routing(ids, w)
    h = lib.gate_up(Wd, to_device_x(cfg, x), idd, h_dtype=h_dtype)
    for y_dtype in ("f32", "bf16"):
        y_tok = lib.down(Wd, h, idd, wd, y_dtype=y_dtype, variant="token")
        y_exp = torch.full_like(y_tok, float("nan"))
        lib.down(Wd, h, idd, wd, y=y_exp, variant="expert")
        torch.cuda.synchronize()
        if fmt == "mxfp4" and h_dtype == "bf16":
            a_, b_ = to_f64(y_tok), to_f64(y_exp)
            tol = 1e-5 if y_dtype == "f32" else 8e-3   # BF16 y: one rounding of either sum
            assert np.linalg.norm(a_ - b_) <= tol * np.linalg.norm(a_), (fmt, y_dtype)
        else:
            assert torch.equal(y_tok, y_exp), (fmt, y_dtype, "expert")


def test_expert_major_down_at_the_entry_limit(lib):
    """The expert-major down on the most entries it stages (256 tokens x top-8
    of the Qwen3-style layer) equals the token-major down bit for bit."""
    cfg = W.QWEN3_DECODE_MXFP8
    t = lib.load().moe_decode_max_entries() // cfg.top_k
    x, ids, w = inputs(cfg, t)
    Wd = device_weights(cfg)
    idd, wd = device_routing(ids, w)
    h = lib.gate_up(Wd, to_device_x(cfg, x), idd, h_dtype="bf16")
    y_tok = lib.down(Wd, h, idd, wd, variant="token")
    y_exp = lib.down(Wd, h, idd, wd, variant="expert")
    torch.cuda.synchronize()
    assert torch.equal(y_tok, y_exp)


def test_every_output_written(lib):
    cfg = SMALL["mxfp4"]
    x, ids, w = inputs(cfg, 11)
    Wd = device_weights(cfg)
    xd = to_device_x(cfg, x)
    idd, wd = device_routing(ids, w)
    h = torch.full((11, cfg.top_k, cfg.inter), float("nan"), device="cuda")
    y = torch.full((11, cfg.hidden), float("nan"), device="cuda")
    lib.gate_up(Wd, xd, idd, h=h)
    lib.down(Wd, h, idd, wd, y=y)
    torch.cuda.synchronize()
    assert torch.isfinite(h).all() and torch.isfinite(y).all()


def test_layer_decode_path_matches_oracle(lib):
    cfg = SMALL["fp8_blk128"].replace(num_shared=1)
    x, ids, w = inputs(cfg, 6)
    Wd = device_weights(cfg)
    y, chosen = lib.layer(Wd, to_device_x(cfg, x), *device_routing(ids, w), path="decode")
    torch.cuda.synchronize()
    assert chosen == "decode"
    _, y_ref = _oracle(cfg, x, ids, w)
    assert_layer_close(to_f64(y), y_ref)


def test_duplicate_ids_within_a_token(lib):
    """Two slots of one token on the same expert are legal and both count."""
    cfg = SMALL["mxfp8"]
    x, ids, w = inputs(cfg, 4)
    ids = ids.copy()
    ids[:, 1] = ids[:, 0]
    Wd = device_weights(cfg)
    idd, wd = device_routing(ids, w)
    h = lib.gate_up(Wd, to_device_x(cfg, x), idd)
    y = lib.down(Wd, h, idd, wd)
    torch.cuda.synchronize()
    _, y_ref = _oracle(cfg, x, ids, w)
    assert_layer_close(to_f64(y), y_ref)


# ---- full-size workloads, sampled tokens ---------------------------------

FULL = [("qwen3_decode_mxfp8", 32, None), ("qwen3_decode_mxfp8", 1, None),
        ("deepseek_v3_fp8_blk128", 16, None), ("mxfp4_sweep", 64, None),
        ("mxfp4_sweep", 32, "zipf"),
        # the MXFP4 matrix-core kernels' other launch shapes at full size: two
        # columns per pass (B = 1) and twelve with two passes per expert
        # (B = 256, Zipf: hot experts split over many wavefronts)
        ("mxfp4_sweep", 1, None), ("mxfp4_sweep", 256, "zipf")]


@pytest.mark.parametrize("name,t,kind", FULL)
def test_decode_full_size_sampled(lib, name, t, kind):
    """Full configuration and batch, in the launch shape the benchmark times;
    the oracle checks a sample of tokens (tokens are independent)."""
    cfg = W.CONFIGS[name]
    x, ids, w, h, y = _run_decode(lib, cfg, t, kind=kind)
    sample = sorted({0, t // 2, t - 1})
    x64 = L.activations_f64(x[sample], cfg.act)
    ref = L.moe_layer(x64, ids[sample], w[sample], **oracle_kw(cfg))
    assert_layer_close(to_f64(y)[sample], ref, (name, t))


def test_out_of_range_ids_read_as_expert_zero(lib):
    """An id outside [0, E) is read as expert 0 by every kernel (documented
    in the header); both paths then match the oracle run on the ids with
    those entries replaced by 0."""
    cfg = SMALL["mxfp8"]
    t = 6
    x, ids, w = inputs(cfg, t)
    bad = ids.copy()
    bad[0, 0], bad[2, 3], bad[5, 1] = cfg.num_experts, -1, cfg.num_experts + 1000
    fixed = np.where((bad < 0) | (bad >= cfg.num_experts), 0, bad).astype(np.int32)
    Wd = device_weights(cfg)
    xd = to_device_x(cfg, x)
    x64 = L.activations_f64(x, cfg.act)
    for path, mode in (("decode", "none"), ("grouped", "mxfp8")):
        y, chosen = lib.layer(Wd, xd, *device_routing(bad, w), path=path, block=32)
        torch.cuda.synchronize()
        assert chosen == path
        ref = L.moe_layer(x64, fixed, w, act_quant=mode, **oracle_kw(cfg))
        assert_layer_close(to_f64(y), ref, path)


def test_decode_at_the_entry_limit(lib):
    """T * slots equal to moe_decode_max_entries(): the largest batch the
    decode kernels stage on chip (Qwen3-style layer, 256 tokens x top-8);
    sampled tokens against the oracle, and one past it is refused."""
    cfg = W.QWEN3_DECODE_MXFP8
    limit = lib.load().moe_decode_max_entries()
    t = limit // cfg.top_k
    assert t * cfg.top_k == limit
    x, ids, w = inputs(cfg, t)
    Wd = device_weights(cfg)
    y, chosen = lib.layer(Wd, to_device_x(cfg, x), *device_routing(ids, w), path="decode")
    torch.cuda.synchronize()
    assert chosen == "decode"
    sample = sorted({0, 97, t - 1})
    x64 = L.activations_f64(x[sample], cfg.act)
    ref = L.moe_layer(x64, ids[sample], w[sample], **oracle_kw(cfg))
    assert_layer_close(to_f64(y)[sample], ref)
    x2, ids2, w2 = inputs(cfg, t + 1)
    with pytest.raises(lib.MoeError) as err:
        lib.layer(Wd, to_device_x(cfg, x2), *device_routing(ids2, w2), path="decode")
    assert err.value.status == lib.ERR_UNSUPPORTED


def test_mx4_matrix_core_passes_and_shared_expert(lib):
    """MXFP4 gate_up on the matrix cores takes 8 entries of an expert per
    pass: here every token's first slot goes to expert 3 (20 entries, three
    passes), nine tokens also send slot 1 to expert 5, and a shared expert
    adds one more slot per token."""
    cfg = SMALL["mxfp4"].replace(num_shared=1, tag=24)
    t = 20
    x, ids, w = inputs(cfg, t)
    ids = ids.copy()
    ids[:, 0] = 3
    ids[:9, 1] = 5
    Wd = device_weights(cfg)
    xd = to_device_x(cfg, x)
    idd, wd = device_routing(ids, w)
    h = lib.gate_up(Wd, xd, idd)
    y = lib.down(Wd, h, idd, wd)
    torch.cuda.synchronize()
    h_ref, y_ref = _oracle(cfg, x, ids, w)
    scale = np.sqrt(np.mean(h_ref ** 2))
    hh = to_f64(h)
    assert np.max(np.abs(hh - h_ref)) <= 2e-4 * scale + 1e-6, np.max(np.abs(hh - h_ref)) / scale
    assert_layer_close(to_f64(y), y_ref)


def test_mx4_matrix_core_results_do_not_depend_on_the_launch_shape(lib):
    """The MXFP4 matrix-core kernels pick 2, 8 or 12 columns per pass (and the
    ring depth) from the batch size; a token's h and y are the same bits
    alone (2 columns) and inside batches of 4 (8 columns), 32 and 256 (12)."""
    cfg = SMALL["mxfp4"]
    Wd = device_weights(cfg)
    t_max = lib.load().moe_decode_max_entries() // cfg.top_k
    x, ids, w = inputs(cfg, t_max)
    xd = to_device_x(cfg, x)
    idd, wd = device_routing(ids, w)
    ref = {}
    for t in (4, 32, t_max):
        h = lib.gate_up(Wd, xd[:t].contiguous(), idd[:t].contiguous(), h_dtype="bf16")
        y = lib.down(Wd, h, idd[:t].contiguous(), wd[:t].contiguous())
        torch.cuda.synchronize()
        ref[t] = (h[:3].clone(), y[:3].clone())
    for j in range(3):
        h1 = lib.gate_up(Wd, xd[j:j + 1].contiguous(), idd[j:j + 1].contiguous(), h_dtype="bf16")
        y1 = lib.down(Wd, h1, idd[j:j + 1].contiguous(), wd[j:j + 1].contiguous())
        torch.cuda.synchronize()
        for t, (h, y) in ref.items():
            assert torch.equal(h1[0], h[j]) and torch.equal(y1[0], y[j]), (j, t)


def test_mx4_matrix_core_expert_count_not_a_multiple_of_64(lib):
    """72 experts: the work map walks the expert ids 64 at a time."""
    cfg = W.MXFP4_SWEEP.replace(hidden=512, inter=256, num_experts=72, tag=25)
    x, ids, w = inputs(cfg, 9)
    Wd = device_weights(cfg)
    idd, wd = device_routing(ids, w)
    h = lib.gate_up(Wd, to_device_x(cfg, x), idd)
    y = lib.down(Wd, h, idd, wd)
    torch.cuda.synchronize()
    h_ref, y_ref = _oracle(cfg, x, ids, w)
    scale = np.sqrt(np.mean(h_ref ** 2))
    assert np.max(np.abs(to_f64(h) - h_ref)) <= 2e-4 * scale + 1e-6
    assert_layer_close(to_f64(y), y_ref)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp8_i1536"])
def test_down_scale_staging_fallback_bitwise(lib, fmt):
    """The conversion-once expert-major down stages each item's E8M0 scales in
    LDS when the scale array is 16-byte aligned; with the scales one byte off
    alignment it loads them byte by byte instead.  Both give the same bits,
    and the same bits as token-major."""
    cfg = SMALL[fmt]
    x, ids, w = inputs(cfg, 24)
    Wd = device_weights(cfg)
    w13, w13s, w2, w2s = Wd.tensors
    buf = torch.empty(w2s.numel() + 16, dtype=torch.uint8, device="cuda")
    mis = buf[1:1 + w2s.numel()].view(w2s.shape)
    mis.copy_(w2s)
    assert mis.data_ptr() % 16 == 1
    Wm = lib.Weights(cfg.fmt, cfg.hidden, cfg.inter, cfg.num_experts, cfg.num_shared,
                     w13, w13s, w2, mis)
    idd, wd = device_routing(ids, w)
    h = lib.gate_up(Wd, to_device_x(cfg, x), idd, h_dtype="bf16")
    y_staged = lib.down(Wd, h, idd, wd, variant="expert")
    y_bytes = lib.down(Wm, h, idd, wd, variant="expert")
    y_tok = lib.down(Wd, h, idd, wd, variant="token")
    torch.cuda.synchronize()
    assert torch.equal(y_staged, y_bytes) and torch.equal(y_staged, y_tok)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp8_h1024"])
@pytest.mark.parametrize("h_dtype", ["f32", "bf16"])
def test_gate_up_scale_dwords_fallback_bitwise(lib, fmt, h_dtype):
    """MXFP8 gate_up reads a neuron pair's scales as one dword per lane when
    the scale array is 4-byte aligned, byte by byte otherwise: same bits."""
    cfg = SMALL[fmt]
    x, ids, w = inputs(cfg, 13)
    Wd = device_weights(cfg)
    w13, w13s, w2, w2s = Wd.tensors
    buf = torch.empty(w13s.numel() + 16, dtype=torch.uint8, device="cuda")
    mis = buf[1:1 + w13s.numel()].view(w13s.shape)
    mis.copy_(w13s)
    assert mis.data_ptr() % 4 != 0
    Wm = lib.Weights(cfg.fmt, cfg.hidden, cfg.inter, cfg.num_experts, cfg.num_shared,
                     w13, mis, w2, w2s)
    xd = to_device_x(cfg, x)
    idd, _ = device_routing(ids, w)
    h_dw = lib.gate_up(Wd, xd, idd, h_dtype=h_dtype)
    h_bytes = lib.gate_up(Wm, xd, idd, h_dtype=h_dtype)
    torch.cuda.synchronize()
    assert torch.equal(h_dw, h_bytes)
