"""Number formats, decoded to float64 from their bit fields.

bf16: sign, 8-bit exponent (bias 127), 7-bit mantissa -- the upper half of an
IEEE binary32.

E2M1 (4-bit float, OCP Microscaling Formats v1.0): sign, 2-bit exponent
(bias 1), 1-bit mantissa; exponent 0 is subnormal (0 or 0.5).  The Nemotron 3
Ultra page names E2M1 as the element type of NVFP4.

E4M3FN (OCP 8-bit float): sign, 4-bit exponent (bias 7), 3-bit mantissa;
exponent 0 is subnormal; S.1111.111 is NaN, there is no infinity.  The Nemotron
3 Ultra page (limitations) names E4M3 as the NVFP4 block-scale type.

Block-scaled FP4 weight ("dual scale", Nemotron 3 Super section 3.6):
w = e2m1(code) * e4m3(block scale) * tensor scale, one block scale per 16
consecutive input-dim elements, one float32 tensor scale per expert matrix.
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    m = (b & 0x7F).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 128.0, (e - 127).astype(np.int32))
    sub = sign * np.ldexp(m / 128.0, -126)
    out = np.where(e == 0, sub, normal)
    out = np.where(e == 0xFF, np.where(m == 0, sign * np.inf, np.nan), out)
    return out


def e4m3fn_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & (m == 7), np.nan, out)


def e2m1_to_f64(code: np.ndarray) -> np.ndarray:
    c = np.asarray(code, dtype=np.uint8).astype(np.int64) & 0xF
    sign = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = (c & 0x1).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int32))
    sub = sign * (m / 2.0)
    return np.where(e == 0, sub, normal)


def fp4_dequant(packed: np.ndarray, block_scale: np.ndarray, tensor_scale) -> np.ndarray:
    """Decode one block-scaled FP4 matrix.

    packed: [rows, cols/2] uint8, element 2j in the low nibble of byte j.
    block_scale: [rows, cols/16] uint8 E4M3FN.  tensor_scale: float32 scalar.
    Returns float64 [rows, cols].
    """
    packed = np.asarray(packed, dtype=np.uint8)
    rows, half = packed.shape
    codes = np.empty((rows, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    q = e2m1_to_f64(codes)
    s = np.repeat(e4m3fn_to_f64(block_scale), 16, axis=1)
    return q * s * float(np.float32(tensor_scale))
