"""fp64 CPU oracle for exact attention. TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the HIP library and its Python binding never do.
"""

from .attention import (
    attention_backward,
    attention_backward_bias,
    attention_backward_head,
    attention_decode,
    attention_forward,
    attention_forward_bias,
    attention_forward_fp8,
    attention_forward_mxfp8,
    attention_forward_chunk,
    attention_forward_rows,
    dequantize_fp8,
    dequantize_mx_cols,
    dequantize_mx_rows,
    e4m3_decode,
    e8m0_decode,
    merge_chunks,
)

__all__ = [
    "attention_forward",
    "attention_forward_chunk",
    "attention_forward_rows",
    "merge_chunks",
    "attention_decode",
    "attention_backward",
    "attention_backward_head",
    "attention_forward_bias",
    "attention_backward_bias",
    "e4m3_decode",
    "dequantize_fp8",
    "attention_forward_fp8",
    "e8m0_decode",
    "dequantize_mx_rows",
    "dequantize_mx_cols",
    "attention_forward_mxfp8",
]
