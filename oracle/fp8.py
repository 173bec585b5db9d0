"""Decode over an FP8 (OCP E4M3) KV cache with per-KV-head scales, in float64.

TEST INFRASTRUCTURE ONLY: the HIP library never imports or calls this module.

Sources (page title, then section):

* deepconcepts.dev, "Grouped-Query Attention", section "Checking it on a real
  system": quantising the KV cache is the serving-time lever that halves its
  bytes again (on top of the KV-head count).
* anrans.github.io, "Attention variants: MQA, GQA, MLA", section "Other ways
  to shrink the KV cache": K and V stored in FP8 (vLLM and SGLang support an
  FP8 KV cache).

The pages fix neither the FP8 format nor the scaling.  Readings used here:
the OCP 8-bit E4M3 format (sign, 4 exponent bits with bias 7, 3 mantissa
bits; exponent field 0 is subnormal; codes 0x7F and 0xFF are NaN; no
infinities), and one float32 scale per KV head for K and one for V, so the
cache value is code value * scale.  The oracle decodes every code exactly in
float64, multiplies by its head's scale, and applies the plain decode
definition unchanged.
"""
from __future__ import annotations

import numpy as np

from .attention import decode


def e4m3_value(codes) -> np.ndarray:
    """Exact float64 value of OCP E4M3 codes (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (8.0 + m) * 2.0 ** (e - 10.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def dequantize(codes, scales) -> np.ndarray:
    """[B, Hkv, T, d] codes times the scale of their KV head, in float64."""
    v = e4m3_value(codes)
    return v * np.asarray(scales, dtype=np.float64)[None, :, None, None]


def decode_fp8(q, k_codes, v_codes, k_scale, v_scale, seq_lens, scale: float, return_lse: bool = False):
    """Decode output [B, Hq, d] over an E4M3 cache: dequantise, then decode."""
    return decode(q, dequantize(k_codes, k_scale), dequantize(v_codes, v_scale), seq_lens, scale,
                  return_lse=return_lse)
