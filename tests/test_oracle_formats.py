"""Pins of oracle/formats.py against routines other than itself: torch's own
dtype conversions (exhaustive over every code / bit pattern), numpy's log2,
and the OCP E2M1 value table stored under tests/golden/."""

import os

import numpy as np
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq)


def test_e4m3fn_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert _same(F.decode_e4m3fn(codes), ref)
    # named special values of the format
    assert F.decode_e4m3fn(np.uint8(0x7E)) == 448.0
    assert np.isnan(F.decode_e4m3fn(np.uint8(0x7F)))
    assert F.decode_e4m3fn(np.uint8(0x01)) == 2.0 ** -9


def test_e8m0_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert _same(F.decode_e8m0(codes), ref)


def test_bf16_all_patterns_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert _same(F.decode_bf16(bits), ref)


def test_e2m1_all_codes_vs_ocp_table():
    table = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_values.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            table[int(c, 16)] = float(v)
    codes = np.arange(16, dtype=np.uint8)
    assert _same(F.decode_e2m1(codes), [table[c] for c in range(16)])


def test_fp4_nibble_order():
    packed = np.array([[0x21, 0xF7]], dtype=np.uint8)
    assert F.unpack_fp4(packed).tolist() == [[0x1, 0x2, 0x7, 0xF]]
    # dequant with a unit scale (127) gives 0.5, 1.0, 6.0, -6.0 ... padded block
    row = np.zeros((1, 16), dtype=np.uint8)
    row[0, :2] = packed
    w = F.dequant_mx(row, np.array([[127]], dtype=np.uint8), "e2m1")
    assert w[0, :4].tolist() == [0.5, 1.0, 6.0, -6.0]


def test_mx_dequant_scale_applies_per_32_columns():
    codes = np.full((2, 64), 0x38, dtype=np.uint8)        # 0x38 = 1.0 in E4M3
    scales = np.array([[127, 130], [120, 127]], dtype=np.uint8)
    w = F.dequant_mx(codes, scales, "e4m3")
    assert np.all(w[0, :32] == 1.0) and np.all(w[0, 32:] == 8.0)
    assert np.all(w[1, :32] == 2.0 ** -7) and np.all(w[1, 32:] == 1.0)


def test_blk128_dequant_tiles():
    codes = np.full((256, 256), 0x38, dtype=np.uint8)
    s = np.array([[1.0, 2.0], [3.0, 0.5]], dtype=np.float32)
    w = F.dequant_blk128(codes, s)
    assert w[0, 0] == 1.0 and w[127, 128] == 2.0 and w[128, 127] == 3.0 and w[255, 255] == 0.5


def _finite_bf16_values():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = F.decode_bf16(bits)
    return v[np.isfinite(v)]


def test_round_to_e4m3_exhaustive_vs_torch_cast():
    """Every finite BF16 value, divided by every power of two 2^e the quantiser
    can use, rounds exactly like torch's float8_e4m3fn cast of the saturated
    value."""
    v = _finite_bf16_values()
    for e in range(-127, 128):
        s = np.clip(v / np.ldexp(1.0, e), -F.E4M3_MAX, F.E4M3_MAX)
        ours = F.round_to_e4m3(s)
        ref = torch.from_numpy(s.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        # float64 -> float32 is exact here except far below E4M3's range, where
        # both sides give a (signed) zero
        assert np.array_equal(ours, ref), e


def test_shared_exponent_vs_log2():
    v = np.abs(_finite_bf16_values())
    v = v[v > 0]
    ref = np.clip(np.floor(np.log2(v)).astype(np.int64) - 8, -127, 127)
    assert np.array_equal(F.mx_shared_exponent(v, 8), ref)
    assert F.mx_shared_exponent(np.array([0.0]), 8)[0] == -127


def test_quantize_mx_block_properties():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-20, 20, (64, 1)))
    x[3] = 0.0
    codes, sc = F.quantize_mx_e4m3(x)
    deq = F.dequant_mx(codes, sc, "e4m3")
    blocks = x.reshape(64, 8, 32)
    amax = np.abs(blocks).max(-1)
    # scale is 2^(floor(log2 amax) - 8): the block maximum lands in [256, 512)
    # before saturation, so it encodes at the top binade of E4M3
    nz = amax > 0
    e = sc.astype(np.int64) - 127
    top = amax[nz] / np.ldexp(1.0, e[nz].astype(np.int32))
    assert np.all((top >= 256) & (top < 512))
    # elements in E4M3's normal range keep 3 mantissa bits: relative error at
    # most 2^-4 (half a step); elements beyond 448 after scaling saturate
    unit = np.repeat(np.ldexp(1.0, e.astype(np.int32)), 32, axis=1)
    scaled = np.abs(x) / unit
    normal = (scaled >= 2.0 ** -6) & (scaled <= 448)
    rel = np.abs(deq - x)[normal] / np.abs(x[normal])
    assert np.all(rel <= 2.0 ** -4 + 1e-12)
    sat = scaled > 448
    assert np.all(np.abs(deq[sat]) == 448 * unit[sat])
    assert np.all(codes[3] == 0) and np.all(sc[3] == 0)
    # the same pipeline through torch's cast and numpy's log2
    e2 = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1))) - 8, -127)
    s2 = np.clip(blocks / np.ldexp(1.0, e2.astype(np.int32))[..., None], -448, 448)
    ref = torch.from_numpy(s2.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, ref.reshape(64, 256))


def test_two_term_mx_quantisation():
    """hi = Q(v), lo = Q(v - hi): the second term's block scale follows the
    residual.  The residual is at most a quarter of the block maximum (when the
    maximum saturates at 448 scale units; a sixteenth otherwise) and lo keeps
    it to half an E4M3 step (2^-4), so hi + lo is within 2^-6 of the block
    maximum; a one-step change of a hi code is absorbed by lo."""
    rng = np.random.default_rng(9)
    v = rng.standard_normal((32, 256)) * np.exp(rng.uniform(-5, 5, (32, 1)))
    ch, sh, cl, sl = F.quantize_mx_e4m3_two_term(v)
    hi = F.dequant_mx(ch, sh, "e4m3")
    assert np.array_equal(ch, F.quantize_mx_e4m3(v)[0])
    approx = F.fake_quant_mx_e4m3_two_term(v)
    bmax = np.repeat(np.abs(v).reshape(32, 8, 32).max(-1), 32, axis=1)
    assert np.all(np.abs(approx - v) <= bmax * 2.0 ** -6)
    assert np.median(np.abs(approx - v) / bmax) < 2.0 ** -10
    # move one hi code by one step: the residual's quantisation compensates
    ch2 = ch.copy()
    ch2[0, 5] = ch2[0, 5] + 1 if ch2[0, 5] not in (0x7E, 0xFE) else ch2[0, 5] - 1
    hi2 = F.dequant_mx(ch2, sh, "e4m3")
    lo2 = F.fake_quant_mx_e4m3(v - hi2)
    assert np.abs((hi2 + lo2) - v)[0, :32].max() <= np.abs(v[0, :32]).max() * 2.0 ** -6
    assert np.abs(hi - v).max() > np.abs(approx - v).max()


def test_two_term_lo_term_scale_rule():
    """The second term is an MX quantisation of the residual r = v - hi with
    its own shared exponent, floor(log2 max|r|) - 8 (numpy log2, clamped,
    -127 for an all-zero residual block), and codes equal to torch's
    float8_e4m3fn cast of clip(r / 2^e, +-448): checked against the
    independent route, with blocks spanning many magnitudes, exactly
    representable blocks (zero residual) and an all-zero block."""
    import _torch_route as R
    rng = np.random.default_rng(21)
    v = rng.standard_normal((48, 256)) * np.exp(rng.uniform(-30, 30, (48, 1)))
    v[5] = 0.0                                            # all-zero blocks
    v[6] = np.ldexp(np.round(rng.uniform(-8, 8, 256)), 3)  # exact in E4M3: zero residual
    v[7, :32] = 448.0 * 2.0 ** 3                          # saturating block maximum
    ch, sh, cl, sl = F.quantize_mx_e4m3_two_term(v)
    rc, rs = R.mx_quant(v)
    assert np.array_equal(ch, rc) and np.array_equal(sh, rs)
    r = v - R.mx_dequant_e4m3(rc, rs)
    lc, ls = R.mx_quant(r)
    assert np.array_equal(sl, ls) and np.array_equal(cl, lc)
    ramax = np.abs(r).reshape(48, 8, 32).max(-1)
    want = np.where(ramax > 0, np.clip(np.floor(np.log2(np.where(ramax > 0, ramax, 1))) - 8,
                                       -127, 127), -127) + 127
    assert np.array_equal(sl.astype(np.int64), want.astype(np.int64))
    assert np.all(sl[6] == 0) and np.all(cl[6] & 0x7F == 0)
    # lo has its own exponent: at least three binades below hi's wherever the
    # block is non-zero, so a quantiser that encoded lo on hi's shared
    # exponent would fail the equalities above
    nz = (np.abs(v).reshape(48, 8, 32).max(-1) > 0) & (ramax > 0)
    assert np.all(sl.astype(np.int64)[nz] <= sh.astype(np.int64)[nz] - 3)
    e_hi = sh.astype(np.int64) - 127
    on_hi = np.clip(r.reshape(48, 8, 32) / np.exp2(e_hi.astype(np.float64))[..., None], -448, 448)
    codes_on_hi = torch.from_numpy(on_hi).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert not np.array_equal(codes_on_hi.reshape(48, 256), cl)


def test_round_to_bf16_vs_torch_and_ties():
    """float32 inputs: equal to torch's float32 -> bfloat16 cast (RNE);
    exact halfway cases go to the even significand; idempotent."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        rng.standard_normal(2000) * 1e-39]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = F.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: even significand is 1.0;
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6
    assert F.round_to_bf16(1.0 + 2.0 ** -8) == 1.0
    assert F.round_to_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert F.round_to_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == -(1.0 + 2.0 ** -7)
    assert np.array_equal(F.round_to_bf16(got), got)
