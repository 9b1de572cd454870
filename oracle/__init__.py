"""CPU oracle for the ternary BitLinear mpGEMM (I2_S weights x per-token absmax int8).

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously-correct
definition of what the hot path computes. Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import it. The product path (the HIP
library and its Python binding) never imports, calls or links anything here,
and nothing here imports the product path.

Sources (web pages on the method; cited by title and section):
  * "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading notes
    (egguo-blog, arXiv 2502.11880): Part A §2.3 (I2_S keeps BitNet b1.58
    ternary weights with one scale and per-tensor int8 activations), §4.1
    (lossless conditions: no extra quantization of partial sums), Part B
    "方法公式化" (lossless = ternary weights + int8 activations + no extra
    quantization step).
  * FairyFuse article (ainews.cool): "三元量化方案" (per-layer scale alpha,
    threshold at +-0.5 alpha), "融合内核设计" (2-bit codes 00/01/10 for 0/+1/-1,
    add or subtract the activation per nonzero weight).
  * bitnet.cpp how-to blog (mhpq.cn) §1.2: with weights in {-1,0,+1} the
    matmul's multiply-adds become additions and subtractions.
  * BinaryAI Engine forum post, "关键技术机制解析" §2: the residual add and
    the RMS normalization fused into one pass.

Modules:
  quant    absmax int8 activation quantization, per token or per tensor;
           token sums of the codes (the library's side output)
  norm     residual add + RMSNorm fused with the per-token quantizer
  ternary  absmean weight scale (exact sum) and the +-0.5*gamma threshold
  i2s      2-bit I2_S pack / unpack (code table and bit layout)
  t3       base-3 pack / unpack, five weights per byte (1.6 bits per weight)
  dot      exact integer contraction (int64), plus an fp64-BLAS exact variant
  lut      element-wise lookup-table sums (TL1/TL2 style), a cross-check only
  dequant  y = acc * gamma * d in fp64; the fp32 epilogue; bf16 rounding

Every function is pinned by the CPU tests in tests/test_oracle_*.py against
hand-worked examples (tests/golden/), closed forms, brute force and
invariants. Parity unpinned: byte compatibility with bitnet.cpp's own i2_s
GGUF layout, and end-to-end "lossless vs Float16" (needs trained weights).
"""
from .quant import widen_bf16, quantize_act_absmax, quantize_act_absmax_tensor, token_sums
from .norm import rmsnorm_quant, round_fraction_to_f32
from .ternary import absmean_gamma, ternarize, ternarize_absmean
from .i2s import pack_i2s, unpack_i2s, CODE_ZERO, CODE_POS, CODE_NEG
from .t3 import pack_t3, unpack_t3
from .dot import mpgemm_acc, mpgemm_acc_entries, mpgemm_acc_f64blas
from .lut import lut_dot
from .dequant import dequant_f64, dequant_f32, round_f64_to_bf16_bits, bf16_bits_to_f64

__all__ = [
    "widen_bf16", "quantize_act_absmax", "quantize_act_absmax_tensor", "token_sums",
    "absmean_gamma", "ternarize", "ternarize_absmean",
    "pack_i2s", "unpack_i2s", "CODE_ZERO", "CODE_POS", "CODE_NEG",
    "pack_t3", "unpack_t3",
    "mpgemm_acc", "mpgemm_acc_entries", "mpgemm_acc_f64blas",
    "lut_dot",
    "dequant_f64", "dequant_f32", "round_f64_to_bf16_bits", "bf16_bits_to_f64",
]
