"""Exact float64 values of the stored input formats (oracle side).

Storage formats and where the pages name them:

* FP16 inputs with FP32 accumulation: page "从RTX 3090到H100：FlashAttention在
  NVIDIA各代GPU架构上的性能全景分析", section 1 (Tensor Core mixed FP16/FP32
  precision) and the tuning dict of section 3.2 (``fp16: True``).
* FP8: page "Optimization Flash Attention 基准测试", H100 80GB forward-time
  table (the "Flash Attn 3 (FP8)" column) and page "FlashAttention与TensorRT
  10集成", section on future directions (commercial use of FP8 precision).
  The pages do not name an FP8 encoding; the reading taken is OCP FP8 E4M3
  ("e4m3fn"), the format the CDNA4 matrix cores consume.

Every decode here is written from the format's definition, not from a library
conversion, so that a test can compare it with torch's conversions:

* binary16 is decoded by numpy (its float16 type is IEEE binary16).
* bfloat16 is the upper 16 bits of an IEEE binary32.
* OCP E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 encodes subnormals m/8 * 2^-6; all other patterns are
  (1 + m/8) * 2^(e-7), except S.1111.111 which is NaN; there is no infinity.
"""
from __future__ import annotations

import numpy as np


def decode_bf16_bits(bits: np.ndarray) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> exact float64 values."""
    bits = np.asarray(bits, dtype=np.uint16)
    wide = bits.astype(np.uint32) << np.uint32(16)
    return wide.view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            value = np.nan
        elif exp_field == 0:
            value = (mant / 8.0) * 2.0 ** (1 - 7)
        else:
            value = (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
        table[code] = sign * value
    return table


_E4M3 = _e4m3_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """uint8 OCP E4M3 codes -> exact float64 values (NaN for 0x7F/0xFF)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def decode(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of each stored element of format ``dtype``."""
    if dtype == "f16":
        return np.asarray(stored, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16_bits(stored)
    if dtype == "fp8":
        return decode_e4m3(stored)
    raise ValueError(f"unknown storage format {dtype!r}")


def dequantize(stored: np.ndarray, dtype: str, descale: float = 1.0) -> np.ndarray:
    """The value an input element stands for: decoded code times its descale.

    For f16/bf16 the descale is 1.  For fp8 it is the float32 per-tensor scale
    the quantiser chose; the product is formed in float64 and is exact.
    """
    x = decode(stored, dtype)
    if descale != 1.0:
        x = x * np.float64(np.float32(descale))
    return x
