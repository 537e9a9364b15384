"""Float64 oracle of the routed-expert MoE FFN of one layer.

Test infrastructure (see the package docstring): nothing on the product path
imports this module.

Definition (warp-decode post, sections on the traditional MoE path and on how
the two kernels work; GC-MoE abstract for the shared expert being optional):
each token t is routed to k experts e_tj with weights w_tj, and

    h_tj = SiLU(Wg[e_tj] x_t) * (Wu[e_tj] x_t)          (SwiGLU, SiLU(z) = z*sigmoid(z))
    y_t  = sum_j  w_tj * Wd[e_tj] h_tj                   (weighted top-k combine)

Readings of the pages taken here:
* the combine uses the given weights as they are (no renormalisation);
* the gate is the first of the two stacked projections w13[e][0], up the
  second w13[e][1]; weights are stored [out][in] with the input axis
  contiguous;
* with one shared expert it is stored as expert index E and runs as an extra
  slot k with weight 1.0 for every token (the align-and-sort article notes
  DeepSeek's single shared expert; its weight is not stated, 1.0 is the plain
  reading);
* the expert-centric path runs its products on block-scaled matrix cores,
  which take 8-bit operands, so its activations are MX-quantised: x_t per 32
  along H before the gate/up products (the align-and-sort article's online
  FP8 quantisation step in the fused pipeline; the warp-decode post, accuracy
  section, on this extra rounding), and h_tj per 32 along I after SwiGLU
  (GC-MoE abstract: SwiGLU fused with requantisation).  It also keeps each
  slot's weighted output w_tj * Wd h_tj in a 2-byte buffer before the combine
  (the warp-decode post sizes that buffer as top-k x hidden x 2 bytes per
  token), read here as BF16 with round-to-nearest-even, so every slot
  contribution is rounded to BF16 before the slot-order sum.  No page says
  how many terms the requantisation of h keeps.  Two modes:
    - ``act_quant="mxfp8_single"``: h -> Q(h), one MXFP8 term: the plain
      reading of "requantization";
    - ``act_quant="mxfp8"``: h -> Q(h) + Q(h - Q(h)), two MXFP8 terms, both
      fed to the down product.  This is the library's own design choice: a
      matrix core's accumulation error moves h by about 5e-5 relative, which
      flips some single-term codes against any exact reference; the second
      term absorbs such flips.  The library's grouped path computes this mode.
  With ``act_quant="none"`` activations stay exact, as on the output-centric
  path.

All arithmetic is float64.  Experts are dequantised once per call, each only
if some slot routes to it.
"""

import math

import numpy as np

from . import formats as F


# --------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------

def activations_f64(x, dtype):
    """x as stored ("f32": float32 array, "bf16": uint16 bit patterns) ->
    float64."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return F.decode_bf16(x)
    raise ValueError(dtype)


def _lut_e4m3():
    return F.decode_e4m3fn(np.arange(256, dtype=np.uint8))


# Lookup tables of the exact decoders (formats.decode_*), indexed by the stored
# byte: one E4M3 value, one E8M0 scale, or the two E2M1 values of a packed byte
# (even element from the low nibble).
_E4M3 = _lut_e4m3()
_E8M0 = F.decode_e8m0(np.arange(256, dtype=np.uint8))
_E2M1_PAIR = F.decode_e2m1(F.unpack_fp4(np.arange(256, dtype=np.uint8)[:, None]))


def _mx(codes, scales, elem):
    codes = np.asarray(codes)
    if elem == "e4m3":
        v = _E4M3[codes]
    else:
        v = _E2M1_PAIR[codes].reshape(codes.shape[:-1] + (2 * codes.shape[-1],))
    s = np.repeat(_E8M0[np.asarray(scales)], F.MX_BLOCK, axis=-1)[..., : v.shape[-1]]
    return v * s


def _blk128(codes, scales):
    v = _E4M3[np.asarray(codes)]
    r, k = v.shape[-2], v.shape[-1]
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    s = np.repeat(np.repeat(s, 128, axis=-2), 128, axis=-1)[..., :r, :k]
    return v * s


def dequant_expert(fmt, raw):
    """One expert's raw arrays -> (Wg [I][H], Wu [I][H], Wd [H][I]) float64.

    raw: dict with "w13" [2][I][H*], "w2" [H][I*] and, per format,
    "w13_scale"/"w2_scale" (MX: E8M0 bytes per 32 along K; fp8_blk128: float32
    per 128x128 tile of each [out][in] matrix; "f64": float64 values, taken
    as they are).
    """
    if fmt == "f32":
        w13 = np.asarray(raw["w13"], dtype=np.float32).astype(np.float64)
        w2 = np.asarray(raw["w2"], dtype=np.float32).astype(np.float64)
    elif fmt == "f64":
        # values already dequantised (for callers that reuse one expert's
        # dequantised weights across several evaluations)
        w13 = np.asarray(raw["w13"], dtype=np.float64)
        w2 = np.asarray(raw["w2"], dtype=np.float64)
    elif fmt in ("mxfp8", "mxfp4"):
        elem = "e4m3" if fmt == "mxfp8" else "e2m1"
        w13 = _mx(raw["w13"], raw["w13_scale"], elem)
        w2 = _mx(raw["w2"], raw["w2_scale"], elem)
    elif fmt == "fp8_blk128":
        w13 = _blk128(raw["w13"], raw["w13_scale"])
        w2 = _blk128(raw["w2"], raw["w2_scale"])
    else:
        raise ValueError(fmt)
    return w13[0], w13[1], w2


def slots(topk_ids, topk_weights, num_experts, num_shared):
    """Routed slots plus the optional shared slot: ids/weights [T][k+S]."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    t = ids.shape[0]
    w = None if topk_weights is None else np.asarray(topk_weights, dtype=np.float32).astype(np.float64)
    if num_shared:
        ids = np.concatenate([ids, np.full((t, 1), num_experts, dtype=np.int64)], axis=1)
        if w is not None:
            w = np.concatenate([w, np.ones((t, 1))], axis=1)
    return ids, w


def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^-z), float64."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


MODES = ("none", "mxfp8", "mxfp8_single")


def _check_mode(act_quant):
    if act_quant not in MODES:
        raise ValueError(act_quant)


def quantise_x(x, act_quant):
    """The gate/up products' input: x itself, or its MX form Q(x)."""
    return x if act_quant == "none" else F.fake_quant_mx_e4m3(x)


def quantise_h(h, act_quant):
    """The down product's input: h itself, Q(h), or Q(h) + Q(h - Q(h))."""
    if act_quant == "mxfp8":
        return F.fake_quant_mx_e4m3_two_term(h)
    if act_quant == "mxfp8_single":
        return F.fake_quant_mx_e4m3(h)
    return np.asarray(h, dtype=np.float64)


def round_slot(c, act_quant):
    """A slot's weighted output as the path holds it before the combine."""
    return c if act_quant == "none" else F.round_to_bf16(c)


# --------------------------------------------------------------------------
# the layer, vectorised by grouping slots per expert
# --------------------------------------------------------------------------

def _group(ids):
    """expert -> (token rows, slot cols) of every slot routed to it."""
    flat = ids.reshape(-1)
    order = np.argsort(flat, kind="stable")
    experts, starts = np.unique(flat[order], return_index=True)
    bounds = list(starts) + [len(flat)]
    s = ids.shape[1]
    for i, e in enumerate(experts):
        sel = order[bounds[i]: bounds[i + 1]]
        yield int(e), sel // s, sel % s


def gate_up(x, topk_ids, *, fmt, num_experts, num_shared, get_expert, act_quant="none"):
    """h [T][k+S][I] float64: h_tj = SiLU(Wg x_t) * (Wu x_t) for e = e_tj.

    x: float64 [T][H].  In the MXFP8 modes the rows of x are MX-quantised
    first and h is returned unquantised (the quantisation of h belongs to the
    down product).
    """
    _check_mode(act_quant)
    ids, _ = slots(topk_ids, None, num_experts, num_shared)
    a = quantise_x(x, act_quant)
    h = None
    for e, rows, cols in _group(ids):
        wg, wu, _ = dequant_expert(fmt, get_expert(e))
        if h is None:
            h = np.zeros(ids.shape + (wg.shape[0],))
        xa = a[rows]
        h[rows, cols] = silu(xa @ wg.T) * (xa @ wu.T)
    return h


def down(h, topk_ids, topk_weights, *, fmt, num_experts, num_shared, get_expert, act_quant="none"):
    """y [T][H] float64 from a given h [T][k+S][I]: y_t = sum_j w_tj Wd h_tj,
    summed over j in slot order (MXFP8 modes: h in its MX form and every
    slot contribution rounded to BF16, as in moe_layer)."""
    _check_mode(act_quant)
    ids, w = slots(topk_ids, topk_weights, num_experts, num_shared)
    hh = quantise_h(h, act_quant)
    ys = None
    for e, rows, cols in _group(ids):
        _, _, wd = dequant_expert(fmt, get_expert(e))
        if ys is None:
            ys = np.zeros(ids.shape + (wd.shape[0],))
        contrib = (hh[rows, cols] @ wd.T) * w[rows, cols][:, None]
        ys[rows, cols] = round_slot(contrib, act_quant)
    y = np.zeros((ids.shape[0], ys.shape[2]))
    for j in range(ids.shape[1]):
        y += ys[:, j]
    return y


def moe_layer(x, topk_ids, topk_weights, *, fmt, num_experts, num_shared, get_expert,
              act_quant="none"):
    """y [T][H] float64 for the whole routed-expert FFN."""
    _check_mode(act_quant)
    ids, w = slots(topk_ids, topk_weights, num_experts, num_shared)
    a = quantise_x(x, act_quant)
    ys = None
    for e, rows, cols in _group(ids):
        wg, wu, wd = dequant_expert(fmt, get_expert(e))
        xa = a[rows]
        hh = quantise_h(silu(xa @ wg.T) * (xa @ wu.T), act_quant)
        if ys is None:
            ys = np.zeros(ids.shape + (wd.shape[0],))
        contrib = (hh @ wd.T) * w[rows, cols][:, None]
        ys[rows, cols] = round_slot(contrib, act_quant)
    y = np.zeros((ids.shape[0], ys.shape[2]))
    for j in range(ids.shape[1]):
        y += ys[:, j]
    return y


# --------------------------------------------------------------------------
# brute force: scalar loops with exactly rounded sums (tiny inputs only)
# --------------------------------------------------------------------------

def moe_layer_scalar(x, topk_ids, topk_weights, *, fmt, num_experts, num_shared, get_expert,
                     act_quant="none"):
    """Same definition as ``moe_layer`` written as plain Python loops over
    tokens, slots, neurons and outputs with math.fsum; for tiny shapes."""
    _check_mode(act_quant)
    ids, w = slots(topk_ids, topk_weights, num_experts, num_shared)
    t_n, s_n = ids.shape
    cache = {}
    rows = []
    for t in range(t_n):
        xt = [float(v) for v in x[t]]
        xt = [float(v) for v in quantise_x(np.array(xt), act_quant)]
        contrib = []
        for j in range(s_n):
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = dequant_expert(fmt, get_expert(e))
            wg, wu, wd = cache[e]
            n_i, n_h = wg.shape
            h = []
            for n in range(n_i):
                g = math.fsum(wg[n, c] * xt[c] for c in range(n_h))
                u = math.fsum(wu[n, c] * xt[c] for c in range(n_h))
                h.append(g / (1.0 + math.exp(-g)) * u)
            h = [float(v) for v in quantise_h(np.array(h), act_quant)]
            c = [w[t, j] * math.fsum(wd[d, n] * h[n] for n in range(n_i))
                 for d in range(wd.shape[0])]
            c = [float(v) for v in round_slot(np.array(c), act_quant)]
            contrib.append(c)
        rows.append([math.fsum(c[d] for c in contrib) for d in range(len(contrib[0]))])
    return np.array(rows, dtype=np.float64)
