"""fp64 CPU oracle of joint text+image attention with 2D-axial RoPE.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call anything in this package.  The product
path (the HIP library and its Python binding) never does, and shares no code,
table or constant with it.

What is computed, and where it comes from ("Speed Up Image Generation with
FLUX 3 Image Klein on NVIDIA Blackwell GPUs"):

* joint attention over the concatenated text / noisy-target / reference
  streams (section "FLUX 3 inference with TensorRT LLM VisualGen"): dense,
  bidirectional softmax(Q K^T / sqrt(D)) V over the whole joint sequence;
* RoPE applied to Q and K where they are produced, i.e. before attention
  (section "GEMM kernel optimization": the QKV projection epilogue carries
  query/key normalization and rotary position embeddings); attention then
  consumes rotated Q and K stored in bf16;
* FP8 Q/K and V (section "Quantized and sparse attention", qk_dtype and
  v_dtype fp8), and the repair of the tokens with the largest quantization
  error (same section, VC-Attention FP8 with vc_repair_budget);
* block-sparse attention on a given block mask (same section: Sol-Attention
  runs on a general block-sparse attention kernel);
* RMS normalization of Q and K before RoPE (section "GEMM kernel
  optimization": query/key normalization in the QKV epilogue).

The pages state none of the arithmetic; the readings taken where they are
silent (2D-axial frequencies, pair convention, the bf16 rounding point of the
rotated Q/K, FP8 scale granularity, e4m3 format) are documented at each
function.  The arithmetic is the plain definition in fp64 throughout; where
the method stores a value in a narrower format (the rotated Q/K in bf16, the
e4m3 codes, the fp32 V scales) the fp64 value is rounded once to that format.
Every function here is pinned by tests in `tests/test_oracle_*.py` against
closed forms, brute force, exact rational arithmetic and library routines.
"""
from .rope import rope_angles, apply_rope
from .bf16 import bf16_round
from .norm import NORM_EPS, rms_norm, prologue
from .attention import (attention, rotated_qk, joint_attention, brute_force_attention,
                        block_sparse_attention, QUERY_BLOCK, KEY_BLOCK)
from .fp8 import (e4m3_round, e4m3_encode, e4m3_decode, pow2_scale, quant_rope_fp8,
                  dequantize, fp8_attention, repair_count, quant_error, repair_errors,
                  repair_select, repair_values, fp8_repaired_attention)

__all__ = [
    "rope_angles", "apply_rope", "bf16_round", "NORM_EPS", "rms_norm", "prologue",
    "attention", "rotated_qk", "joint_attention", "brute_force_attention",
    "block_sparse_attention", "QUERY_BLOCK", "KEY_BLOCK",
    "e4m3_round", "e4m3_encode", "e4m3_decode", "pow2_scale", "quant_rope_fp8",
    "dequantize", "fp8_attention", "repair_count", "quant_error", "repair_errors",
    "repair_select", "repair_values", "fp8_repaired_attention",
]
