"""Logical view of a paged KV cache (test infrastructure).

Source: "FlexAttention: from rules to fused kernels", section 5 -- a paged cache maps
logical KV block j of request b to a physical cache block through a page table
P_b(j); the attention rules keep logical positions, and the slow reference
materialises the logical K/V first and then runs dense attention.  Requests that
share a prefix may point at the same physical page.

Layout read here (the one the library documents for its paged caches):
cache[num_pages, Hkv, page_size, d], table[B, pt_stride]; logical key j of request b
is row j mod page_size of page table[b, j // page_size].

Parity: pinned by tests/test_oracle_pins.py (a hand-worked two-request example, the
identity table, and shared pages).
"""
from __future__ import annotations

import numpy as np


def gather_logical_kv(cache, table, kv_len):
    """cache [num_pages, Hkv, page_size, d], table [B, pt_stride] -> [B, Hkv, kv_len, d]."""
    cache = np.asarray(cache)
    table = np.asarray(table)
    num_pages, hkv, page_size, d = cache.shape
    B = table.shape[0]
    out = np.empty((B, hkv, kv_len, d), dtype=cache.dtype)
    for b in range(B):
        for lp in range(-(-kv_len // page_size)):
            page = int(table[b, lp])
            if not 0 <= page < num_pages:
                raise ValueError(f"page {page} of request {b} is outside the cache")
            j0 = lp * page_size
            n = min(page_size, kv_len - j0)
            out[b, :, j0:j0 + n, :] = cache[page, :, :n, :]
    return out
