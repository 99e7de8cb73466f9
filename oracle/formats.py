"""MXFP4 number formats, written out from their definitions (oracle; test use only).

The RFQ pages ("Activation Outliers Matter: Robust Recovery for Quantized
Multimodal LLMs", Abstract and §1) name MXFP4 as the 4-bit format but their
definition section (§3.1) is cut off. These definitions are the OCP
Microscaling Formats (MX) v1.0 ones:

* E2M1 element: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
  Exponent field 0 is subnormal: value = m * 2^(1 - bias) * 1/2.
  Otherwise value = 2^(e - bias) * (1 + m/2). No infinities, no NaN.
* E8M0 shared scale: unsigned 8-bit exponent with bias 127, value
  2^(c - 127) for c in 0..254; c = 255 encodes NaN. No sign, no zero.
* Block: 32 consecutive elements along the reduction dimension K share one
  scale.
"""

import numpy as np

BLOCK = 32          # elements per shared scale
E2M1_BIAS = 1
E2M1_EMAX = 2       # exponent of the largest E2M1 normal (6 = 1.5 * 2^2)
E8M0_BIAS = 127
E8M0_NAN = 255


def e2m1_value(code: int) -> float:
    """Value of a 4-bit E2M1 code, from its sign/exponent/mantissa fields."""
    code = int(code) & 0xF
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = m * 0.5 * 2.0 ** (1 - E2M1_BIAS)
    else:
        mag = 2.0 ** (e - E2M1_BIAS) * (1.0 + m / 2.0)
    return -mag if s else mag


# Magnitudes of the 8 non-negative codes 0..7, derived from the field definition.
E2M1_MAGNITUDES = np.array([e2m1_value(i) for i in range(8)], dtype=np.float64)


def e8m0_value(code):
    """Value 2^(code - 127) of E8M0 scale codes; NaN for code 255."""
    c = np.asarray(code, dtype=np.int64)
    v = np.ldexp(np.ones(c.shape, dtype=np.float64), (c - E8M0_BIAS).astype(np.int64))
    return np.where(c == E8M0_NAN, np.nan, v)


def bf16_bits_to_f64(bits):
    """Exact value of bfloat16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits):
    """Exact value of float32 bit patterns (uint32) as float64."""
    with np.errstate(invalid="ignore"):
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)
