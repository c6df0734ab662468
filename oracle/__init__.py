"""CPU oracle for fine-grained FP8 (E4M3) block-scaled quantization and GEMM.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` use it.  It shares
no code, constant table or helper with the HIP library and imports nothing
from it.

The oracle is plain and slow on purpose.  Each function states, in its own
docstring, which passage of the source pages it follows:

* ``HolySheep (zh)``: the Chinese HolySheep AI article on FP8 mixed-precision
  training at DeepSeek-671B scale; its section "2.2 细粒度量化实现"
  (fine-grained quantization implementation) holds ``FP8BlockQuantizer``, and
  its troubleshooting section "错误 1: FP8 精度溢出" (overflow) states the
  E4M3 range.
* ``codingmall (sv)``: the codingmall.com knowledge-base article on the role
  of FP8 precision in DeepSeek-V3 training; its sections "Finkornig
  kvantisering" (1x128 activation tiles, 128x128 weight blocks), "Online
  -kvantisering" (per-tile scales from the current data), "Ökad
  ackumuleringsprecision" (FP32 promotion of GEMM partial sums) and "Unified
  E4M3 Format".

Precision: the quantizer works in float32, because the pages fix the scale as
an FP32 value and divide the tile by it in that precision; the GEMM reference
works in float64, where every 128-deep block partial of E4M3 products is exact.
"""
from .e4m3 import (E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_magnitudes,
                   e4m3_half_ulp)
from .quantize import (SCALE_GUARD, tile_scale, quant_1x128, quant_128x1_t,
                       quant_128x128, dequant_1x128, dequant_128x128)
from .gemm import (blockscaled_gemm_ref, grouped_gemm_ref,
                   blockscaled_gemm_fp32_model, gemm_tolerance_ok)
from .dequant import dequant_f32, dequant_bf16, f32_to_bf16_rne
from .e5m2 import E5M2_MAX, e5m2_decode, e5m2_encode, e5m2_magnitudes, e5m2_half_ulp
from .tensor_scaling import tensor_scale, quant_tensor_current, quant_tensor_delayed

__all__ = [
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "e4m3_magnitudes", "e4m3_half_ulp",
    "SCALE_GUARD", "tile_scale", "quant_1x128", "quant_128x1_t", "quant_128x128",
    "dequant_1x128", "dequant_128x128",
    "blockscaled_gemm_ref", "grouped_gemm_ref", "blockscaled_gemm_fp32_model",
    "gemm_tolerance_ok", "dequant_f32", "dequant_bf16", "f32_to_bf16_rne",
    "E5M2_MAX", "e5m2_decode", "e5m2_encode", "e5m2_magnitudes", "e5m2_half_ulp",
    "tensor_scale", "quant_tensor_current", "quant_tensor_delayed",
]
