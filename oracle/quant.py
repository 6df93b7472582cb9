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


def append_int8_pages(codes, scales, rows_new, block_table, start_pos, cu_new, page_size: int):
    """Append new rows (float32-representable values, e.g. bf16 upcast) to an
    int8 pool: the cache-growth step of [KV3X] ("KV Cache" section) through
    the page table of [FAPKV] §3.2, with the group quantiser above.

    codes [N, P, Hkv, D] int8, scales [N, Hkv] float32, rows_new
    [cu_new[B], Hkv, D]; row r of sequence b lands at position
    start_pos[b] + r.  Returns new (codes, scales).

    Reading for a group that is only partly filled (the pages fix no rule):
    every (physical page, KV head) group that receives rows is requantised
    over its valid slots after the append.  Slots of positions already in the
    sequence (before start_pos[b]) hold the value code * old_scale (float32
    product); new slots hold the new rows; the new scale is the largest
    magnitude of those values / 127 (float32 division; 1 if it is 0); every
    valid slot gets round_half_even(clamp(value / scale, -128, 127)) (float32
    division).  Slots past the sequence's new end are left as they are.  A
    whole page appended at once into an empty page is therefore exactly
    ``quantize_int8_pages`` of that page."""
    codes = np.array(codes, dtype=np.int8, copy=True)
    scales = np.array(scales, dtype=np.float32, copy=True)
    x = np.asarray(rows_new, dtype=np.float32)
    block_table = np.asarray(block_table)
    for b in range(len(start_pos)):
        s0, r0 = int(start_pos[b]), int(cu_new[b])
        n = int(cu_new[b + 1]) - r0
        if n == 0:
            continue
        end = s0 + n
        for lp in range(s0 // page_size, (end - 1) // page_size + 1):
            phys = int(block_table[b, lp])
            p0 = lp * page_size
            n_old = max(0, min(s0, p0 + page_size) - p0)   # old valid slots [0, n_old)
            hi = min(end, p0 + page_size) - p0              # valid slots after: [0, hi)
            first_row = r0 + (p0 + n_old - s0)              # input row of slot n_old
            for hk in range(codes.shape[2]):
                old = codes[phys, :n_old, hk, :].astype(np.float32) * scales[phys, hk]
                new = x[first_row:first_row + (hi - n_old), hk, :]
                vals = np.concatenate([old, new], axis=0).astype(np.float32)
                amax = np.abs(vals).max()
                s = np.float32(1.0) if amax == 0 else np.float32(amax / np.float32(127.0))
                y = np.clip((vals / s).astype(np.float32), np.float32(-128.0), np.float32(127.0))
                codes[phys, :hi, hk, :] = np.rint(y).astype(np.int8)
                scales[phys, hk] = s
    return codes, scales
