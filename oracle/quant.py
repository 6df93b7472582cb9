"""Symmetric abs-max int8 group quantisation of KV pages.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[SYS] §3.2 (quantised compression, group quantisation): within a group the
scale is the largest magnitude divided by 2^(bits-1) - 1; values are divided
by the scale, clamped to [-2^(bits-1), 2^(bits-1) - 1] and rounded.  Here
bits = 8 and a group is one (physical page, KV head): all P slots x D values
of that head in that page, so the scale does not depend on how many slots of
the page are in use.  K and V pools are quantised separately.

Precision: the scale and the division are taken in float32 with IEEE
round-to-nearest (the HIP path's precision, so the integer codes agree bit
for bit); "round" is round-half-to-even.  A group whose largest magnitude is
0 gets scale 1 and codes 0.
"""
from __future__ import annotations

import numpy as np


def quantize_int8_pages(pages):
    """pages [N, P, Hkv, D] (float32-representable values, e.g. bf16 upcast)
    -> (codes int8 [N, P, Hkv, D], scales float32 [N, Hkv])."""
    x = np.asarray(pages, dtype=np.float32)
    absmax = np.abs(x).max(axis=(1, 3))                       # [N, Hkv], exact
    scales = (absmax / np.float32(127.0)).astype(np.float32)  # fp32 division
    scales = np.where(absmax == 0, np.float32(1.0), scales).astype(np.float32)
    y = (x / scales[:, None, :, None]).astype(np.float32)     # fp32 division
    y = np.clip(y, np.float32(-128.0), np.float32(127.0))
    codes = np.rint(y).astype(np.int8)                        # half-to-even
    return codes, scales


def dequantize_int8_pages(codes, scales):
    """codes * scale in float64 (exact: a 7-bit integer times a float32)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[:, None, :, None]
