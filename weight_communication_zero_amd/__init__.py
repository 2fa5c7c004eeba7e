"""libzq: ZeRO++ / LoCo block-quantized gradient and weight communication
kernels and llm.c-style stochastic-rounding accumulation for MI355X (gfx950).

The compute lives in ``libzq.so`` (hand-written HIP kernels behind the C ABI
in ``include/zq.h``); this package is its thin ctypes binding.
"""
from .zq import (  # noqa: F401
    ZQ_BF16, ZQ_FP32, DrSegmentTable, EfqSegmentTable, SrSegmentTable, ZQError, int4_code_bytes,
    lib, num_blocks, zeropp_slots, zq_dequant_int8, zq_dequant_reduce, zq_dequant_reduce_batched,
    zq_quant_int8, zq_quantize_ef_int4, zq_quantize_ef_int4_batched, zq_quantize_ef_int4_permuted,
    zq_sr_accumulate, zq_sr_accumulate_batched,
)
