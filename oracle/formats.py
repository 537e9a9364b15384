"""Exact float64 decoders for the stored number formats, and the MX quantiser.

Test infrastructure (see the package docstring): nothing on the product path
imports this module.

Sources.  The pages name the formats but do not define their bit layouts:
the warp-decode post (section on how the two kernels work) streams MXFP8
expert weights and converts them to FP32 in registers; the GC-MoE abstract
names FP8/FP4 operators with in-register FP4 decoding.  The layouts below are
the OCP ones (OCP 8-bit floating point spec, E4M3 "FN" variant without
infinities; OCP Microscaling (MX) spec v1.0: E2M1 elements, E8M0 shared scale,
32-element blocks).  Every decoder is pinned exhaustively in
``tests/test_oracle_formats.py``: E4M3FN / E8M0 / BF16 against torch's own
dtype conversions, E2M1 against the OCP value table stored under
``tests/golden/``.

Readings of the pages taken here:
* MX blocks run along the contiguous input (K) axis of each weight row.
* FP4 packs two elements per byte, the even element in the low nibble.
* The MX quantiser picks the shared exponent as floor(log2(amax)) minus the
  element format's largest exponent (8 for E4M3), clamps it to [-127, 127]
  (-127 when the block is all zero), divides, saturates to +-448 and rounds to
  nearest, ties to even.  The sign of the input is kept, so a negative value
  that rounds to zero encodes as 0x80.
"""

import numpy as np

MX_BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8        # largest power-of-two exponent below E4M3_MAX
E2M1_EMAX = 2        # largest power-of-two exponent below 6.0


def decode_e4m3fn(codes):
    """E4M3FN code -> float64.  Layout s.eeee.mmm, exponent bias 7.

    e == 0 is subnormal: (-1)^s * 2^-6 * m/8.  e == 15 with m == 7 is NaN
    (there are no infinities); every other code is (-1)^s * 2^(e-7) * (1+m/8).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sign = np.where(s == 1, -1.0, 1.0)
    sub = sign * np.ldexp(m.astype(np.float64) / 8.0, -6)
    nrm = sign * np.ldexp(1.0 + m.astype(np.float64) / 8.0, (e - 7).astype(np.int32))
    out = np.where(e == 0, sub, nrm)
    return np.where((e == 15) & (m == 7), np.nan, out)


def decode_e2m1(codes):
    """E2M1 code (low 4 bits) -> float64.  Layout s.ee.m, exponent bias 1.

    e == 0 is subnormal: (-1)^s * m/2; otherwise (-1)^s * 2^(e-1) * (1+m/2).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 0x3
    m = c & 0x1
    sign = np.where(s == 1, -1.0, 1.0)
    sub = sign * (m.astype(np.float64) / 2.0)
    nrm = sign * np.ldexp(1.0 + m.astype(np.float64) / 2.0, (e - 1).astype(np.int32))
    return np.where(e == 0, sub, nrm)


def decode_e8m0(codes):
    """E8M0 shared scale byte -> float64: 2^(b-127); b == 255 is NaN."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    out = np.ldexp(1.0, (b - 127).astype(np.int32))
    return np.where(b == 255, np.nan, out)


def decode_bf16(bits):
    """BF16 bit pattern (uint16) -> float64: the pattern is the top half of an
    IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(v):
    """float64 -> the nearest BF16 value (round to nearest, ties to even on the
    8-bit significand), as float64.  Finite inputs within the float32 range;
    BF16 keeps float32's exponent range, so only the significand is rounded
    (below 2^-126 the spacing stays 2^-133, the subnormal step)."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                        # v = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)               # spacing of 8 significant bits
    return np.ldexp(np.round(np.ldexp(v, -q)), q)


def unpack_fp4(packed):
    """[..., n/2] bytes -> [..., n] E2M1 codes; element 2p is the low nibble of
    byte p and element 2p+1 its high nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def _expand_blocks(scale, block, n):
    """Repeat each per-block scale `block` times along the last axis."""
    return np.repeat(scale, block, axis=-1)[..., :n]


def dequant_mx(codes, scales, elem):
    """MX dequantisation along the last (K) axis.

    elem = "e4m3": codes [..., K] bytes; elem = "e2m1": codes [..., K/2]
    packed bytes.  scales [..., K/32] E8M0 bytes.  Returns float64 [..., K]:
    W[r, c] = dec(q[r, c]) * 2^(s[r, c // 32] - 127).
    """
    if elem == "e4m3":
        v = decode_e4m3fn(codes)
    elif elem == "e2m1":
        v = decode_e2m1(unpack_fp4(codes))
    else:
        raise ValueError(elem)
    k = v.shape[-1]
    return v * _expand_blocks(decode_e8m0(scales), MX_BLOCK, k)


def dequant_blk128(codes, scales):
    """FP8 E4M3 with one float32 scale per 128x128 tile of a [rows][K] matrix.

    codes [..., R, K] bytes, scales [..., ceil(R/128), ceil(K/128)] float32.
    W[r, c] = dec(q[r, c]) * S[r // 128, c // 128].
    """
    v = decode_e4m3fn(codes)
    r, k = v.shape[-2], v.shape[-1]
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    s = np.repeat(np.repeat(s, 128, axis=-2), 128, axis=-1)[..., :r, :k]
    return v * s


# ---------------------------------------------------------------------------
# MX quantiser (E4M3 elements), as used for activations on the expert-centric
# path.  Written as "nearest point of the E4M3 grid, ties to the even code".
# ---------------------------------------------------------------------------

def _e4m3_grid():
    codes = np.arange(0, 0x7F, dtype=np.uint8)          # 0 .. 0x7E (448)
    return codes, decode_e4m3fn(codes)                  # ascending values


_GRID_CODES, _GRID_VALS = _e4m3_grid()


def round_to_e4m3(v):
    """float64 -> E4M3FN code: saturate to +-448, round to the nearest grid
    value, ties to the even code; the sign bit follows the input's sign."""
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_GRID_VALS, a, side="left")    # first grid >= a
    hi = np.clip(hi, 0, len(_GRID_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_GRID_VALS) - 1)
    d_lo = a - _GRID_VALS[lo]
    d_hi = _GRID_VALS[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_GRID_CODES[hi] % 2 == 0))
    mag = np.where(pick_hi, _GRID_CODES[hi], _GRID_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(v), mag | 0x80, mag).astype(np.uint8)


def mx_shared_exponent(amax, emax):
    """Shared block exponent: floor(log2(amax)) - emax, clamped to
    [-127, 127]; -127 for an all-zero block."""
    amax = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(amax)                 # amax = f * 2^ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1 - emax
    e = np.where(amax == 0.0, -127, e)
    return np.clip(e, -127, 127)


def quantize_mx_e4m3(v):
    """Quantise float64 [..., K] (K % 32 == 0) to MXFP8.

    Returns (codes uint8 [..., K], scale bytes uint8 [..., K/32]).
    """
    v = np.asarray(v, dtype=np.float64)
    k = v.shape[-1]
    if k % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    blocks = v.reshape(v.shape[:-1] + (k // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    e = mx_shared_exponent(amax, E4M3_EMAX)
    scaled = blocks / np.ldexp(1.0, e.astype(np.int32))[..., None]
    codes = round_to_e4m3(scaled).reshape(v.shape)
    return codes, (e + 127).astype(np.uint8)


def fake_quant_mx_e4m3(v):
    """Q(v): quantise to MXFP8 and decode back to float64."""
    codes, scales = quantize_mx_e4m3(v)
    return dequant_mx(codes, scales, "e4m3")


def quantize_mx_e4m3_two_term(v):
    """v ~ hi + lo with hi = Q(v) and lo = Q(v - hi): two MXFP8 terms.
    Returns (codes_hi, scales_hi, codes_lo, scales_lo)."""
    ch, sh = quantize_mx_e4m3(v)
    cl, sl = quantize_mx_e4m3(np.asarray(v, dtype=np.float64) - dequant_mx(ch, sh, "e4m3"))
    return ch, sh, cl, sl


def fake_quant_mx_e4m3_two_term(v):
    """hi + lo decoded back to float64."""
    ch, sh, cl, sl = quantize_mx_e4m3_two_term(v)
    return dequant_mx(ch, sh, "e4m3") + dequant_mx(cl, sl, "e4m3")
