"""CPU oracle for the attention forward pass -- test infrastructure only.

This package is the plain, slow, obviously correct definition that the GPU
kernels are checked against.  It materialises the full score matrix and the
softmax in float64, exactly the "standard attention" that the pages contrast
FlashAttention with, because FlashAttention reaches that same result up to
rounding order.

Only the test suite, the smoke check of the entry module and the benchmark's
CPU-baseline leg may import it.  The product path never does, and nothing here
imports the GPU package: the two share no code.  Inputs come from the seeded
generator as plain numpy arrays.

Every function is pinned by tests that do not reuse its own formula (closed
forms, invariants, an mpmath brute force, torch's float64 CPU attention and a
mutation check); see the module docstrings for the passages followed.
"""
from .formats import decode, decode_e4m3, decode_bf16_bits, dequantize
from .attention import attention_slice, attention, attention_varlen, slice_sample
from .backward import attention_backward_slice, attention_backward
from .dropout import philox4x32_10, keep_threshold, dropout_bytes, attention_dropout_slice, attention_dropout
from .projection import qkv_projection

__all__ = [
    "decode",
    "decode_e4m3",
    "decode_bf16_bits",
    "dequantize",
    "attention_slice",
    "attention",
    "attention_varlen",
    "slice_sample",
    "attention_backward_slice",
    "attention_backward",
    "philox4x32_10",
    "keep_threshold",
    "dropout_bytes",
    "attention_dropout_slice",
    "attention_dropout",
    "qkv_projection",
]
