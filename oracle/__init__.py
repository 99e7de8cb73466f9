"""CPU oracle for Residual Fallback Quantization (RFQ) on MXFP4.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
links anything in this package. Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark use it. It shares no code, table or helper
with the HIP library: it is an independent, slow, float64 statement of what
the method computes, written so that a reader can check it against the
sources by eye.

Sources followed (cited by page title and section):

* "Activation Outliers Matter: Robust Recovery for Quantized Multimodal LLMs"
  (arXiv 2608.26581; Chinese translation page and English summary page),
  Abstract and §1 (the RFQ paragraph and the contributions list): the
  activation is split into a primary low-bit (MXFP4) part and the full
  quantization error, which is itself quantized by a second low-bit path; the
  residual is re-quantized during the GEMM and its contribution accumulated.
* The MXFP4 element and scale encodings are only named on those pages (their
  §3.1 text is cut off). The oracle uses the public OCP Microscaling Formats
  (MX) v1.0 definitions: 32-element blocks, an E8M0 power-of-two shared scale
  chosen as floor(log2(amax)) - emax(E2M1), and E2M1 elements (sign, 2-bit
  exponent with bias 1, 1-bit mantissa) rounded to nearest, ties to even,
  saturating at +-6.

* The block-Hadamard rotation (``rotate.py``) follows the QuaRot description
  on "大模型量化中的双线性尾部问题与QuaRot正交旋转解决方案" §3; see that module.
* MXFP8 (``mxfp8.py``): E4M3 elements per OCP MX v1.0, for the W4A8 layer and
  for RFQ with an MXFP8 residual path (the pages study MXFP8 beside MXFP4,
  Abstract and §1); see that module.
* The straight-through backward pass (``backward.py``): the pages present
  RFQ as training-aware but do not write the backward out; see that module
  for the reading taken.

Every function is pinned by tests in ``tests/test_oracle_*.py`` against facts
that do not come from this code (worked examples, closed forms, brute force,
library routines, invariants). The one result without such a pin is the
model-level accuracy benefit of RFQ, which is outside this package.
"""

from .formats import (
    BLOCK,
    E2M1_EMAX,
    E2M1_MAGNITUDES,
    E8M0_NAN,
    bf16_bits_to_f64,
    e2m1_value,
    e8m0_value,
    f32_bits_to_f64,
)
from .quantize import (
    dequantize,
    pack_codes,
    quantize_mxfp4,
    residual_quantize,
    scale_exponent,
    encode_block_elements,
    unpack_codes,
)
from .gemm import gemm_w4a4, linear
from .rotate import (ROTATION_SIZES, fraction_to_f32, hadamard32_rounded, hadamard_rounded, linear_rotated,
                     rotate_quantize_weight, rotate_residual_quantize)
from .backward import backward_dw, backward_dx, linear_backward
from .mxfp8 import (
    E4M3_MAGNITUDES,
    E4M3_MAX,
    dequantize_mxfp8,
    e4m3_value,
    encode_e4m3,
    gemm_w4a4_fp8_residual,
    gemm_w4a8,
    linear_fp8_residual,
    linear_w4a8,
    quantize_mxfp8,
    residual_quantize_fp8,
    scale_exponent_e4m3,
)

__all__ = [
    "BLOCK", "E2M1_EMAX", "E2M1_MAGNITUDES", "E8M0_NAN",
    "bf16_bits_to_f64", "f32_bits_to_f64",
    "e2m1_value", "e8m0_value",
    "scale_exponent", "encode_block_elements", "quantize_mxfp4", "residual_quantize",
    "dequantize", "pack_codes", "unpack_codes",
    "gemm_w4a4", "linear",
    "hadamard32_rounded", "hadamard_rounded", "ROTATION_SIZES", "fraction_to_f32", "rotate_residual_quantize", "rotate_quantize_weight", "linear_rotated",
    "E4M3_MAGNITUDES", "E4M3_MAX", "e4m3_value", "scale_exponent_e4m3", "encode_e4m3",
    "quantize_mxfp8", "dequantize_mxfp8", "residual_quantize_fp8",
    "gemm_w4a8", "gemm_w4a4_fp8_residual", "linear_w4a8", "linear_fp8_residual",
    "backward_dx", "backward_dw", "linear_backward",
]
