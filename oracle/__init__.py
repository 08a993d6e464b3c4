"""CPU oracle for the quantized MoE grouped GEMM path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product (the HIP
library and its Python binding) never imports, links or calls it, and this
package shares no code with it.

Every function is the plain definition of what the path computes, written in
numpy with float64 (and exact integer) arithmetic, no blocking, fusion or
reordering.  Sources, by page:
  * CUTLASS discussion #2855, "How to implement dequantization of row and
    column broadcast in Epilogue of GroupGemm" (W4A4 INT4 grouped GEMM with
    per-token x per-channel scales; the [E+1] row-offset table).
  * CUTLASS issue #2087, "how to use groupwise scaling along M for FP8 gemm to
    implement per-token-per-128-channel and blockwise" (FP8 e4m3 with 1x128 A
    scales and 128x128 B scales; the M-contiguous A-scale layout).
  * nvfp4-megamoe-kernel, tilelang_kernels.py, grouped_gemm_fp4 (NVFP4 routed
    grouped GEMM and weighted scatter-add).
  * (CUTLASS discussion #2855 also fixes the per-token int4 quantization of
    fp16 activations; its rule is a reading, see quant.py.)
  * megamoe_rm.cu (route_prep, fc1_rm, fc2_rm, combine kernels: stable
    per-expert ordering, -1 ids, per-expert global scale, SiLU-gated FC1,
    k-ordered fp32 combine; the up-first w13 and 128x4-swizzled scale layout
    it reads, layouts.py).

Parity pins: every function here is checked, in tests/test_oracle_*.py,
against something other than itself (torch's codecs, brute force in pure
Python, a differently structured algorithm, invariants).  No function is
parity unpinned.
"""
from .formats import (unpack_nibbles, int4_value, e2m1_value, e4m3fn_value, ue4m3_value,
                      bf16_value, round_to_f16, round_to_bf16, round_to, f16_value, f16_bits,
                      bf16_to_f16_bits)
from .route import route_prep
from .gemm import (grouped_gemm_qint4, grouped_gemm_qfp8_block, grouped_gemm_qnvfp4, silu_mul,
                   gemm_rows, weight_rows)
from .combine import scatter_combine, pair_rows, sum_pairs
from .layer import int4_layer, int4_ffn_layer, nvfp4_layer, fp8_dense, token_rows, combine_tokens
from .quant import quantize_int4_rows
from .layouts import (scale_swizzle_offset, unswizzle_scales, swizzle_scales, repack_nvfp4,
                      quads_from_rows, rows_from_quads, tiles_from_rows, rows_from_tiles)

__all__ = [n for n in dir() if not n.startswith("_")]
