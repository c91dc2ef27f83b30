"""Seeded synthetic workloads shared by the tests, the bench and the oracle checks.

This module only describes shapes and draws random inputs.  It performs none of
the attention arithmetic: no masking, no score modification, no softmax.  Both
the GPU path and the CPU oracle receive the exact bits drawn here.

The workloads follow the shapes the pages describe:

* a tiny causal sliding window (the worked N=8, W=4 example of "FlexAttention:
  from rules to fused kernels", section 2.2, Fig. 1, scaled up to N=512);
* causal attention with tanh soft-capping ("FlexAttention: compiler optimization
  of custom attention", section 2);
* GQA with a document mask intersected with a sliding window and an ALiBi bias
  ("FlexAttention: from rules to fused kernels", sections 1.1 and 1.2);
* a 64K prefix-LM with a per-head relative-position table (same page, section
  6.3 for prefix-LM, section 1.2 for the table; section 2.1 for the
  262,144-block grid of a 64K sequence);
* split-KV decode with a sliding window ending at the query position
  ("FlexAttention: compiler optimization of custom attention", section 6), also
  over a paged KV cache ("FlexAttention: from rules to fused kernels", section 5);
* per-head selector output (top-k KV blocks per query block) inside a causal rule,
  with even or long-tailed row lengths (same page, sections 5.2 and 6.3).

Mask specifications are plain nested tuples, independent of any binary layout:
``("causal",)``, ``("swa", W)``, ``("doc",)``, ``("prefix", P)``,
``("and", a, b)``, ``("or", a, b)``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Any, Optional, Tuple

import numpy as np

try:  # torch is only needed for the bf16 draws
    import torch
except Exception:  # pragma: no cover
    torch = None


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    q_len: int
    kv_len: int
    d: int
    block_q: int
    block_kv: int
    mask: Tuple[Any, ...]
    score: str                      # identity | alibi | softcap | relpos
    cap: float = 0.0                # soft-cap constant
    relpos_radius: int = 0          # clip radius of the relative-position table
    q_offset: int = 0               # global position of query row 0
    seed: int = 0                   # torch seed for Q, K, V (drawn in that order)
    aux_seed: int = 0               # numpy seed for the auxiliary tensors
    doc_seed: Optional[int] = None  # numpy seed for the document lengths
    doc_len_range: Tuple[int, int] = (256, 2048)
    table_B: int = 1                # batch extent of the block tables (1 = broadcast)
    page_size: int = 0              # > 0: K/V live in a paged cache with this page size
    selector: Optional[Tuple[str, float]] = None   # (row-length profile, mean kept fraction)

    @property
    def g(self) -> int:
        return self.Hq // self.Hkv


WORKLOADS = {
    "tiny_swa": Workload(
        name="tiny_swa", B=1, Hq=2, Hkv=2, q_len=512, kv_len=512, d=64,
        block_q=64, block_kv=64, mask=("swa", 128), score="identity",
        seed=1001, aux_seed=1001),
    "causal_softcap": Workload(
        name="causal_softcap", B=2, Hq=16, Hkv=16, q_len=4096, kv_len=4096, d=128,
        block_q=128, block_kv=128, mask=("causal",), score="softcap", cap=20.0,
        seed=1002, aux_seed=1002),
    "gqa_doc_swa_alibi": Workload(
        name="gqa_doc_swa_alibi", B=1, Hq=32, Hkv=8, q_len=8192, kv_len=8192, d=128,
        block_q=128, block_kv=128, mask=("and", ("doc",), ("swa", 1024)),
        score="alibi", seed=1003, aux_seed=1003, doc_seed=0),
    "prefix_relpos_64k": Workload(
        name="prefix_relpos_64k", B=1, Hq=16, Hkv=2, q_len=65536, kv_len=65536, d=128,
        block_q=128, block_kv=128, mask=("prefix", 4096), score="relpos",
        relpos_radius=1024, seed=1004, aux_seed=1004),
    "decode_swa_softcap": Workload(
        name="decode_swa_softcap", B=64, Hq=32, Hkv=8, q_len=1, kv_len=32768, d=128,
        block_q=128, block_kv=128, mask=("swa", 4096), score="softcap", cap=30.0,
        q_offset=32767, seed=1005, aux_seed=1005),
    # the same decode over a paged KV cache: 16-key pages placed by a random
    # permutation ("FlexAttention: from rules to fused kernels", section 5)
    "decode_paged_swa_softcap": Workload(
        name="decode_paged_swa_softcap", B=64, Hq=32, Hkv=8, q_len=1, kv_len=32768, d=128,
        block_q=128, block_kv=128, mask=("swa", 4096), score="softcap", cap=30.0,
        q_offset=32767, seed=1005, aux_seed=1006, page_size=16),
    # per-head block selection as a selector would emit it, over every pair
    # (bidirectional: PREFIX(N) allows all keys): the same mean of 10% of the KV blocks
    # per row, spread evenly over the rows or held by a few full rows ("FlexAttention:
    # from rules to fused kernels", sections 5.2 and 6.3; "Kernels: turning logical
    # sparsity into real speed", section 1.2)
    "select_uniform": Workload(
        name="select_uniform", B=1, Hq=32, Hkv=8, q_len=16384, kv_len=16384, d=128,
        block_q=128, block_kv=128, mask=("prefix", 16384), score="identity",
        seed=1007, aux_seed=1007, selector=("uniform", 0.1)),
    "select_longtail": Workload(
        name="select_longtail", B=1, Hq=32, Hkv=8, q_len=16384, kv_len=16384, d=128,
        block_q=128, block_kv=128, mask=("prefix", 16384), score="identity",
        seed=1007, aux_seed=1008, selector=("longtail", 0.1)),
    # decode with per-head selections (32 of the 256 KV blocks per query head, the newest
    # block always in), each query head reading its own blocks of its group's KV head
    "decode_select": Workload(
        name="decode_select", B=64, Hq=32, Hkv=8, q_len=1, kv_len=32768, d=128,
        block_q=128, block_kv=128, mask=("causal",), score="softcap", cap=30.0,
        q_offset=32767, seed=1005, aux_seed=1010, selector=("uniform", 0.125)),
    # the same selection inside a causal rule (candidates at or before the diagonal)
    "select_causal": Workload(
        name="select_causal", B=1, Hq=32, Hkv=8, q_len=16384, kv_len=16384, d=128,
        block_q=128, block_kv=128, mask=("causal",), score="identity",
        seed=1007, aux_seed=1009, selector=("longtail", 0.1)),
}

# The N=8, W=4, 2x2-block classification case that goes with the tiny workload.
WORKED_N8 = dict(q_len=8, kv_len=8, block_q=2, block_kv=2, mask=("swa", 4))


def mask_uses_doc(spec) -> bool:
    if spec[0] == "doc":
        return True
    if spec[0] in ("and", "or"):
        return mask_uses_doc(spec[1]) or mask_uses_doc(spec[2])
    return False


def doc_lengths(total: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Document lengths drawn uniformly from [lo, hi] one at a time until they
    cover ``total`` tokens; the last one is truncated to fit."""
    rng = np.random.default_rng(seed)
    out = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return np.asarray(out, dtype=np.int64)


def doc_ids_from_lengths(lengths: np.ndarray) -> np.ndarray:
    """Packed document IDs 0, 1, 2, ... (int32), one per token."""
    return np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)


def alibi_slopes(Hq: int) -> np.ndarray:
    """Per-query-head ALiBi slopes 2^(-8(h+1)/Hq) as float32 values."""
    h = np.arange(Hq, dtype=np.float64)
    return np.exp2(-8.0 * (h + 1.0) / Hq).astype(np.float32)


def relpos_table(Hq: int, radius: int, seed: int, std: float = 0.1) -> np.ndarray:
    """Per-query-head relative-position table, float32 [Hq, 2R+1], N(0, std^2)."""
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((Hq, 2 * radius + 1)) * std).astype(np.float32)


def aux_inputs(w: Workload) -> dict:
    """Document IDs, ALiBi slopes and relative-position table for a workload (numpy)."""
    aux = {"doc_ids": None, "slopes": None, "table": None}
    if mask_uses_doc(w.mask):
        total = w.q_offset + max(w.q_len, w.kv_len)
        seed = w.doc_seed if w.doc_seed is not None else w.aux_seed
        lens = doc_lengths(total, w.doc_len_range[0], w.doc_len_range[1], seed)
        aux["doc_lengths"] = lens
        aux["doc_ids"] = doc_ids_from_lengths(lens)[None, :]   # [1, doc_len]
    if w.score == "alibi":
        aux["slopes"] = alibi_slopes(w.Hq)
    if w.score == "relpos":
        aux["table"] = relpos_table(w.Hq, w.relpos_radius, w.aux_seed)
    return aux


def randn_bf16(shape, seed: int, device="cpu", chunk_elems: int = 1 << 28):
    """iid N(0,1) drawn in float32 from a seeded torch generator and rounded to
    bfloat16 (round to nearest even).  Large tensors are drawn in chunks along
    the leading dimension so that the float32 staging stays bounded."""
    assert torch is not None
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    n = flat.numel()
    pos = 0
    while pos < n:
        m = min(chunk_elems, n - pos)
        flat[pos:pos + m] = torch.randn(m, generator=gen, device=device,
                                        dtype=torch.float32).to(torch.bfloat16)
        pos += m
    return out


def qkv(w: Workload, device="cpu"):
    """Q [B,Hq,q_len,d], K and V [B,Hkv,kv_len,d], bf16, drawn in that order
    from one generator seeded with ``w.seed``."""
    assert torch is not None
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed)
    out = []
    for shape in ((w.B, w.Hq, w.q_len, w.d), (w.B, w.Hkv, w.kv_len, w.d),
                  (w.B, w.Hkv, w.kv_len, w.d)):
        t = torch.empty(shape, dtype=torch.bfloat16, device=device)
        flat = t.view(-1)
        n = flat.numel()
        pos = 0
        chunk = 1 << 27
        while pos < n:
            m = min(chunk, n - pos)
            flat[pos:pos + m] = torch.randn(m, generator=gen, device=device,
                                            dtype=torch.float32).to(torch.bfloat16)
            pos += m
        out.append(t)
    return tuple(out)


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (for small parity cases)."""
    return dataclasses.replace(w, **kw)


def page_table(w: Workload) -> np.ndarray:
    """Page table int32 [B, ceil(kv_len / page_size)] of a paged workload: the B * pages
    logical pages take the physical pages of one random permutation (numpy seed
    ``w.aux_seed``), so consecutive logical pages are scattered over the cache."""
    npg = -(-w.kv_len // w.page_size)
    rng = np.random.default_rng(w.aux_seed)
    return rng.permutation(w.B * npg).astype(np.int32).reshape(w.B, npg)


def paged_caches(w: Workload, k, v, table):
    """K/V caches [B * pages, Hkv, page_size, d] holding the logical K and V
    [B, Hkv, kv_len, d] at the pages ``table`` names (unused tail rows are zero)."""
    assert torch is not None
    ps = w.page_size
    npg = table.shape[1]
    pad = npg * ps - w.kv_len
    out = []
    for t in (k, v):
        cache = torch.zeros((w.B * npg, w.Hkv, ps, w.d), dtype=t.dtype, device=t.device)
        src = t if pad == 0 else torch.nn.functional.pad(t, (0, 0, 0, pad))
        src = src.view(w.B, w.Hkv, npg, ps, w.d).permute(0, 2, 1, 3, 4).reshape(w.B * npg, w.Hkv, ps, w.d)
        idx = torch.as_tensor(table.reshape(-1), dtype=torch.long, device=t.device)
        cache.index_copy_(0, idx, src)
        out.append(cache)
    return tuple(out)


def selector_indices(w: Workload) -> np.ndarray:
    """Synthetic selector output int32 [B, Hq, NQB, k_max] for a selector workload:
    for each (batch, head, query block r) the diagonal KV block (the one holding the
    block's last row) plus distinct other candidates drawn uniformly -- earlier blocks
    under a causal rule, any block otherwise -- padded with -1.  Row lengths: "uniform"
    gives every row round(frac * NKB) blocks (fewer where the causal rule leaves fewer);
    "longtail" gives a row all of its candidate blocks with probability p and 4 blocks
    otherwise, p set so that the mean matches the uniform profile's target.  numpy seed
    ``w.aux_seed``; this draws inputs only."""
    kind, frac = w.selector
    causal = w.mask == ("causal",)
    rng = np.random.default_rng(w.aux_seed)
    nqb = -(-w.q_len // w.block_q)
    nkb = -(-w.kv_len // w.block_kv)
    target = max(1, int(round(frac * nkb)))
    small = 4
    avg_avail = (nkb + 1) / 2.0 if causal else float(nkb)
    p_heavy = min(1.0, max(0.0, (target - small) / (avg_avail - small)))
    rows = []
    for _ in range(w.B * w.Hq):
        for r in range(nqb):
            diag = min(nkb - 1, (min((r + 1) * w.block_q, w.q_len) - 1 + w.q_offset) // w.block_kv)
            others = np.arange(diag) if causal else np.delete(np.arange(nkb), diag)
            avail = len(others) + 1
            if kind == "uniform":
                k = min(avail, target)
            else:
                k = avail if rng.random() < p_heavy else min(avail, small)
            pick = rng.choice(others, size=k - 1, replace=False) if k > 1 else np.zeros(0, np.int64)
            rows.append(np.concatenate([[diag], pick]))
    kmax = max(len(x) for x in rows)
    out = np.full((len(rows), kmax), -1, dtype=np.int32)
    for n, x in enumerate(rows):
        out[n, :len(x)] = x
    return out.reshape(w.B, w.Hq, nqb, kmax)
