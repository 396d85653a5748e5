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
The same format serves the shared expert's two matrices: the released recipe
puts the GEMMs of the MoE experts and of the shared expert in NVFP4 and other
projection layers in FP8 ("Nemotron 3.5 Super and Lightning", section on
keeping accuracy under 4-bit quantisation).

Per-tensor FP8 weight (that recipe's FP8 layers; here optionally W_down and
W_up, a reading: the pages do not name the latent projections' precision):
w = e4m3(code) * tensor scale, one float32 scale per matrix.
"""
import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64: the pattern is the upper half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


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
    # decode through 16- and 256-entry tables built with the field decoders above
    q_table = e2m1_to_f64(np.arange(16, dtype=np.uint8))
    s_table = e4m3fn_to_f64(np.arange(256, dtype=np.uint16).astype(np.uint8))
    q = np.empty((rows, half, 2), dtype=np.float64)
    q[:, :, 0] = np.take(q_table, packed & 0xF)
    q[:, :, 1] = np.take(q_table, packed >> 4)
    s = np.take(s_table, np.asarray(block_scale, dtype=np.uint8)) * float(np.float32(tensor_scale))
    return (q.reshape(rows, -1, 16) * s[:, :, None]).reshape(rows, 2 * half)


def fp8_dequant(codes: np.ndarray, tensor_scale) -> np.ndarray:
    """Decode one per-tensor-scaled E4M3FN matrix.

    codes: [rows, cols] uint8 E4M3FN.  tensor_scale: float32 scalar.
    Returns float64 [rows, cols].
    """
    return e4m3fn_to_f64(codes) * float(np.float32(tensor_scale))
