"""Pins for the number formats: the oracle's decoders against the public
format definitions (IEEE binary32 upper half for bf16; OCP Microscaling v1.0
E2M1 and OCP FP8 E4M3FN), and the FP4 encoder used to prepare inputs."""
import numpy as np

from oracle.formats import bf16_to_f64, e2m1_to_f64, e4m3fn_to_f64, fp4_dequant, fp8_dequant
from sparse_moe_layer_logits_amd import synth


def _bf16_from_fields(b):
    """bf16 value from its sign / exponent / mantissa fields (IEEE binary32 layout,
    8-bit exponent with bias 127, 7 stored mantissa bits, subnormals at exponent 0)."""
    b = b.astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    m = (b & 0x7F).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        normal = sign * np.ldexp(1.0 + m / 128.0, (e - 127).astype(np.int32))
        out = np.where(e == 0, sign * np.ldexp(m / 128.0, -126), normal)
        return np.where(e == 0xFF, np.where(m == 0, sign * np.inf, np.nan), out)


def test_bf16_decoder_against_field_definition():
    # every one of the 65536 patterns, decoded from its bit fields
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = _bf16_from_fields(b)
    with np.errstate(invalid="ignore"):
        got = bf16_to_f64(b)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_known_values():
    v = bf16_to_f64(np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x3F81], np.uint16))
    assert v[0] == 1.0 and v[1] == -2.0 and v[2] == 0.0
    assert np.signbit(v[3]) and v[3] == 0.0
    assert v[4] == (2 - 2 ** -7) * 2.0 ** 127
    assert v[5] == 2.0 ** -133
    assert v[6] == 1.0 + 2 ** -7


def test_bf16_encoder_rne():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -3.5, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    got = bf16_to_f64(synth.f32_to_bf16_bits(f))
    # tie at 1+2^-8 rounds to even (1.0); tie at 1+3*2^-8 rounds up to 1+2^-6
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, -3.5, 1.0 + 2 ** -7]


def test_e2m1_table_ocp():
    # OCP MX v1.0 FP4 E2M1 value table for codes 0..7; 8..15 are their negatives
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = e2m1_to_f64(np.arange(16, dtype=np.uint8))
    assert got[:8].tolist() == table
    assert got[8:].tolist() == [-v for v in table]
    assert np.signbit(got[8])


def test_e4m3fn_table_ocp():
    got = e4m3fn_to_f64(np.arange(256, dtype=np.uint16).astype(np.uint8))
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5,
             0x38: 1.0, 0x39: 1.125, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in known.items():
        assert got[c] == v, hex(c)
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.isnan(got).sum() == 2
    pos = got[:127]
    assert np.all(np.diff(pos) > 0)          # monotone over the positive finite codes
    assert np.array_equal(got[128:255], -pos)


def test_e2m1_encoder_ties_to_even():
    v = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 100.0, -0.1, -0.3, -5.0, 0.0])
    got = e2m1_to_f64(synth.encode_e2m1(v))
    assert got.tolist() == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 0.0, -0.5, -4.0, 0.0]
    assert synth.encode_e2m1(np.array([-0.1]))[0] == 0  # negative zero encodes as 0x0


def test_e4m3_encoder_rne_and_saturation():
    pos = e4m3fn_to_f64(np.arange(127, dtype=np.uint8))
    codes = synth.encode_e4m3(pos)
    assert np.array_equal(codes, np.arange(127))
    mid = (pos[:-1] + pos[1:]) / 2           # exact midpoints -> even code
    c = synth.encode_e4m3(mid)
    lo = np.arange(126)
    assert np.array_equal(c, np.where(lo % 2 == 0, lo, lo + 1))
    assert synth.encode_e4m3(np.array([1e6]))[0] == 126


def test_fp4_nibble_order_and_block_scales():
    packed = np.array([[0x21] + [0x00] * 15], np.uint8)        # 32 elements
    scales = np.array([[0x38, 0x40]], np.uint8)                # 1.0, then 2.0
    w = fp4_dequant(packed, scales, np.float32(2.0))
    assert w[0, 0] == 1.0 and w[0, 1] == 2.0                   # low nibble first
    packed2 = np.zeros((1, 16), np.uint8)
    packed2[0, 8] = 0x7F                                       # elements 16 (code F), 17 (code 7)
    w2 = fp4_dequant(packed2, scales, np.float32(1.0))
    assert w2[0, 16] == -12.0 and w2[0, 17] == 12.0            # second block uses scale 2


def test_e2m1_times_e4m3_is_exact_in_bf16():
    """Every E2M1 value times every finite E4M3 scale is a bf16 number, so an
    in-register dequantisation to bf16 loses nothing."""
    q = e2m1_to_f64(np.arange(16, dtype=np.uint8))
    s = e4m3fn_to_f64(np.arange(127, dtype=np.uint8))
    p = (q[:, None] * s[None, :]).astype(np.float32)
    assert np.array_equal(bf16_to_f64(synth.f32_to_bf16_bits(p)), p.astype(np.float64))


def test_fp4_roundtrip_on_grid_and_error_bound():
    rng = np.random.default_rng(5)
    rows, cols = 24, 64
    # weights already on the grid q * s_b * s_t (s_t a power of two, one block at
    # the largest scale 448 so that amax / (6*448) gives s_t back) quantise back
    # to themselves
    q = e2m1_to_f64(rng.integers(0, 16, size=(rows, cols)).astype(np.uint8))
    q[:, ::16] = 6.0                                            # each block reaches amax 6*s_b
    sbc_in = rng.integers(0x30, 0x48, size=(rows, cols // 16)).astype(np.uint8)
    sbc_in[0, 0] = 0x7E
    ts = 2.0 ** -10
    w = q * np.repeat(e4m3fn_to_f64(sbc_in), 16, axis=1) * ts
    wb = synth.f32_to_bf16_bits(w.astype(np.float32))
    assert np.array_equal(bf16_to_f64(wb), w)
    packed, sbc, tsc = synth.encode_fp4(wb)
    assert tsc == np.float32(ts) and np.array_equal(sbc, sbc_in)
    assert np.array_equal(fp4_dequant(packed, sbc, tsc), w)
    # random weights: per-element error within half an E2M1 step (<= 1 unit) plus block clipping
    wr = synth.f32_to_bf16_bits(rng.standard_normal((rows, cols)).astype(np.float32))
    packed, sbc, tsc = synth.encode_fp4(wr)
    back = fp4_dequant(packed, sbc, tsc)
    wf = bf16_to_f64(wr)
    unit = np.repeat(e4m3fn_to_f64(sbc), 16, axis=1) * float(tsc)
    bmax = np.repeat(np.abs(wf).reshape(rows, -1, 16).max(2), 16, axis=1)
    clip = np.maximum(bmax - 6 * unit, 0)
    assert np.all(np.abs(back - wf) <= unit + clip + 1e-12)
    # the block maximum maps to about 6 units (within E4M3 rounding of the scale)
    assert np.all(np.abs(bmax / (6 * unit) - 1) <= 2 ** -4 + 1e-9)


def test_fp8_dequant_known_values_and_scale():
    codes = np.array([[0x38, 0xB8, 0x7E, 0x01, 0x00, 0x80, 0x3C, 0xC4]], np.uint8)
    got = fp8_dequant(codes, np.float32(0.25))
    assert got.tolist() == [[0.25, -0.25, 112.0, 2.0 ** -11, 0.0, -0.0, 0.375, -0.75]]
    # the tensor scale is applied as its float32 value
    assert fp8_dequant(np.array([[0x38]], np.uint8), 0.1)[0, 0] == float(np.float32(0.1))


def test_fp8_encoder_on_grid_and_error_bound():
    rng = np.random.default_rng(11)
    # values already on the grid e4m3 * 2^-8 (amax at code 0x7E so amax / 448 gives the
    # scale back) quantise back to themselves, signs included
    c = rng.integers(0, 127, size=(12, 40)).astype(np.uint8)
    c[0, 0] = 0x7E
    sgn = rng.integers(0, 2, size=c.shape).astype(np.uint8) << 7
    c = np.where(c == 0, c, c | sgn).astype(np.uint8)
    w = fp8_dequant(c, np.float32(2.0 ** -8))
    wb = synth.f32_to_bf16_bits(w.astype(np.float32))
    assert np.array_equal(bf16_to_f64(wb), w)
    codes, ts = synth.encode_fp8(wb)
    assert ts == np.float32(2.0 ** -8)
    assert np.array_equal(fp8_dequant(codes, ts), w)
    # random weights: relative error at most 2^-4 (half an E4M3 step) in the normal
    # range, absolute at most 2^-10 * scale among the subnormals; amax maps to 448
    wr = synth.f32_to_bf16_bits((rng.standard_normal((64, 96)) * 0.03).astype(np.float32))
    codes, ts = synth.encode_fp8(wr)
    wf = bf16_to_f64(wr)
    back = fp8_dequant(codes, ts)
    err = np.abs(back - wf)
    normal = np.abs(wf) >= 2.0 ** -6 * float(ts)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(wf[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= 2.0 ** -10 * float(ts) * (1 + 1e-6))
    assert np.all(np.sign(back[back != 0]) == np.sign(wf[back != 0]))
    assert abs(np.max(np.abs(back)) - np.max(np.abs(wf))) <= 2.0 ** -4 * np.max(np.abs(wf))
