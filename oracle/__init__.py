"""CPU oracle for the NVFP4 post-training-quantization hot path.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, float64 numpy
restatement of what the pages define; it exists to check the HIP library.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The library (``nvfp4_post_quantization_amd``)
never imports it and shares no code, table or helper with it; the only thing
both sides share is the seeded input generator module ``datagen``.

Sources (page title, section):
* "Coder390 NVFP4 校正（校准）方式" (NVFP4 calibration method note), §2:
  the three per-Linear steps - max calibration, block-diagonal local Hessian
  H = sum X^T X per 16 input channels, and the E4M3 scale sweep minimising
  (W-Wq)^T H (W-Wq) over all block-scale codes; NVFP4 = E2M1 elements, one
  E4M3 scale per 16, one FP32 tensor scale.
* "NVFP4 量化流程说明" (pi05 Gemma-2B NVFP4 flow note), §2.2 (E2M1 / E4M3
  signature of the format), §3.4 (tensor scale = amax/6/448; dynamic
  activation quantizer), §5.4 (two-DequantizeLinear weight form, two FP4
  values per byte).
* "从MXFP4到NVFP4：Model Optimizer混合精度格式转换完全攻略" (ModelOpt
  MXFP4->NVFP4 guide), §1 (E8M0 = exponent only), §2 (closed-form cast and
  its window/fallback), §3 (gate/up share one tensor scale).
* "从校准到导出：DeepSeek-V4-Pro-0813-nvfp4-DSpark 三阶段 NVFP4 量化流程实战"
  (DeepSeek-V4 NVFP4 pipeline article), export stage: nibbles move unchanged,
  scale bytes double.
* "FP4量化技术概述" (FP4 survey), §1.1 (E2M1 value set), §1.2 (block sizes,
  bits per element).
* "Coder390 NVFP4 校正（校准）方式" §3 (layer table of the W4A4+W8A8 tier):
  FP8 E4M3 weights and activations with static per-tensor scales (fp8.py).
* "FP4量化技术概述" §3.1 (MR-GPTQ): block Hadamard rotation fused into the
  weights, W' = W H, activations rotated online (rotate.py).

Readings where the pages are silent are marked "reading:" in the docstrings.

Readings no worked example on the pages can confirm (every function is
still pinned by the tests to closed forms, brute force, library routines
and invariants; what stays open is only whether the pages meant these
readings): the argmin tie-break (lowest code), the sign of a zero nibble, the
exact-quotient rounding rule, nibble order within a byte, the clamp of a
nonzero block's code to 0x01, the synthetic input recipes, (for the W4A4
Hessian variant) that the layer input is taken after its activation
quantizer, (FP8 tier) the static scale amax/448 and the exact-quotient
encode, and (rotation) the per-group input-channel rotation, its butterfly
order and the single rounding to bf16.
"""
from .formats import (
    E2M1_MAGNITUDES, E4M3_VALUES, e2m1_decode, e2m1_encode, e4m3_value,
    e4m3_encode_ratio, e8m0_value, bf16_bits_to_f64, f64_to_bf16_bits, f32,
    pack_nibbles, unpack_nibbles, f64_to_bf16_rne,
)
from .nvfp4 import (
    tensor_scale, hessian, block_scale, quantize_at_code, block_cost,
    sweep_costs, scale_sweep, max_code, quantize_dynamic, dequant, hessian_fakequant,
    fakequant, quantlinear_forward,
)
from .mxcast import mxfp4_to_nvfp4, mxfp4_dequant
from .fp8 import fp8_tensor_scale, fp8_quantize, fp8_dequant
from .rotate import hadamard16, rotate_blocks, rotate_hessian

__all__ = [
    "E2M1_MAGNITUDES", "E4M3_VALUES", "e2m1_decode", "e2m1_encode", "e4m3_value",
    "e4m3_encode_ratio", "e8m0_value", "bf16_bits_to_f64", "f64_to_bf16_bits", "f32",
    "pack_nibbles", "unpack_nibbles", "f64_to_bf16_rne",
    "tensor_scale", "hessian", "block_scale", "quantize_at_code", "block_cost",
    "sweep_costs", "scale_sweep", "max_code", "quantize_dynamic", "dequant", "hessian_fakequant",
    "fakequant", "quantlinear_forward",
    "mxfp4_to_nvfp4", "mxfp4_dequant",
    "fp8_tensor_scale", "fp8_quantize", "fp8_dequant",
    "hadamard16", "rotate_blocks", "rotate_hessian",
]
