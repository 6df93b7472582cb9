"""Paged FlashAttention for MI355X (gfx950): exact softmax(QK^T/sqrt(d))V
read from a paged KV cache, as hand-written HIP kernels behind a C ABI.

The compute entry points live in ``flashattention_paged_kv_amd.ops``; they
load the HIP library ``libpagedattn.so`` on first use and raise if it is
missing.  ``workloads`` holds the seeded input generators.
"""
__all__ = ["ops", "workloads"]
