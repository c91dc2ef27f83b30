"""Exact block classification and compacted block tables (test infrastructure).

Sources (page title, then section):

* "FlexAttention: from rules to fused kernels", section 6.3 ("how BlockMask
  correctness can be proved") -- for query block Q_r and KV block K_c the allowed
  edge set is E_rc; the block is skipped if E_rc is empty, is a full block if
  E_rc = Q_r x K_c, and is partial otherwise.  Completeness, exclusivity and
  exactness are required.
* Same page, section 2.1 -- the table is BCSR-like: per query block a count of
  KV blocks and their column indices; section 2.2 -- full and partial lists are
  kept separately; the backward needs the transposed (query-side) index.
* "Causal block geometric pruning", section 5 -- the last block of a ragged
  length is clipped to the real sequence end.

Readings taken (the pages leave them open): classification looks only at
in-range pairs (rows < q_len, columns < kv_len); column lists are ascending;
row pointers are the exclusive prefix sum of the counts over rows ordered by
(b', h', r); the query-side tables are the exact transposes; full and partial
lists are disjoint; no conservative "partial when unsure" is allowed.
"""
from __future__ import annotations

import numpy as np

from . import masks

EMPTY, PARTIAL, FULL = 0, 1, 2


def n_blocks(length, block):
    return (int(length) + int(block) - 1) // int(block)


def classify(spec, q_len, kv_len, block_q, block_kv, q_offset=0, doc_row=None,
             row_chunk_blocks=None):
    """Class grid [NQB, NKB] (uint8: 0 empty, 1 partial, 2 full) for one batch entry.

    Each query block's allowed-pair slab is materialised once and reduced per
    KV block with any/all over its in-range pairs.
    """
    nqb, nkb = n_blocks(q_len, block_q), n_blocks(kv_len, block_kv)
    grid = np.zeros((nqb, nkb), dtype=np.uint8)
    for r in range(nqb):
        r0, r1 = r * block_q, min((r + 1) * block_q, q_len)
        slab = masks.dense(spec, q_len, kv_len, q_offset, doc_row, rows=np.arange(r0, r1))
        # pad the column axis to whole blocks; padded pairs are neither allowed
        # nor required (in-range pairs only)
        pad = nkb * block_kv - kv_len
        allowed = np.pad(slab, ((0, 0), (0, pad)), constant_values=False)
        inrange = np.pad(np.ones_like(slab), ((0, 0), (0, pad)), constant_values=False)
        a = allowed.reshape(r1 - r0, nkb, block_kv)
        g = inrange.reshape(r1 - r0, nkb, block_kv)
        any_ = a.any(axis=(0, 2))
        all_ = (a | ~g).all(axis=(0, 2))
        grid[r] = np.where(all_, FULL, np.where(any_, PARTIAL, EMPTY))
    return grid


def _compact(grid_rows):
    """Compacted lists of a [R, C] class grid, row by row in ascending column order.

    Returns (partial_num, partial_ptr, partial_idx, full_num, full_ptr, full_idx).
    """
    R = grid_rows.shape[0]
    out = []
    for cls in (PARTIAL, FULL):
        num = np.zeros(R, dtype=np.int32)
        idx = []
        for r in range(R):
            cols = np.nonzero(grid_rows[r] == cls)[0].astype(np.int32)
            num[r] = len(cols)
            idx.append(cols)
        ptr = np.zeros(R + 1, dtype=np.int32)
        ptr[1:] = np.cumsum(num)
        idx = np.concatenate(idx) if idx else np.zeros(0, np.int32)
        out += [num, ptr, idx.astype(np.int32)]
    return tuple(out)


def tables(spec, B_tab, H_tab, q_len, kv_len, block_q, block_kv, q_offset=0, doc_ids=None):
    """Both sides of the block tables for table extents (B_tab, H_tab).

    Rows are ordered (b', h', r) and columns (b', h', c).  Every head h' of a
    batch entry b' repeats the same rows because no mask of the menu depends on
    the head.  Returns a dict of int32 arrays with keys

    kv_num, kv_ptr, kv_idx, full_kv_num, full_kv_ptr, full_kv_idx,
    q_num,  q_ptr,  q_idx,  full_q_num,  full_q_ptr,  full_q_idx,

    plus ``grid`` ([B_tab, NQB, NKB] uint8).
    """
    grids = []
    for b in range(B_tab):
        doc_row = masks.doc_row_for(doc_ids, b)
        grids.append(classify(spec, q_len, kv_len, block_q, block_kv, q_offset, doc_row))
    grid = np.stack(grids)                                   # [B', NQB, NKB]
    rows = np.concatenate([np.concatenate([grid[b]] * H_tab) for b in range(B_tab)])
    cols = np.concatenate([np.concatenate([grid[b].T] * H_tab) for b in range(B_tab)])
    kv = _compact(rows)
    q = _compact(cols)
    names = ("num", "ptr", "idx")
    out = {}
    for k, v in zip([f"kv_{n}" for n in names] + [f"full_kv_{n}" for n in names], kv):
        out[k] = v
    for k, v in zip([f"q_{n}" for n in names] + [f"full_q_{n}" for n in names], q):
        out[k] = v
    out["grid"] = grid
    return out


def expand(tab, B_tab, H_tab, q_len, kv_len, block_q, block_kv, spec, q_offset=0,
           doc_ids=None, b=0, h=0):
    """The element matrix implied by the kv-side tables for table entry (b, h).

    Full blocks expand to all-true, partial blocks to the element predicate,
    unlisted blocks to all-false.  Used to check M_hat == M.
    """
    nqb = n_blocks(q_len, block_q)
    doc_row = masks.doc_row_for(doc_ids, b)
    M = masks.dense(spec, q_len, kv_len, q_offset, doc_row)
    out = np.zeros((q_len, kv_len), dtype=bool)
    for r in range(nqb):
        row = (b * H_tab + h) * nqb + r
        r0, r1 = r * block_q, min((r + 1) * block_q, q_len)
        for c in tab["full_kv_idx"][tab["full_kv_ptr"][row]:tab["full_kv_ptr"][row + 1]]:
            c0, c1 = c * block_kv, min((c + 1) * block_kv, kv_len)
            out[r0:r1, c0:c1] = True
        for c in tab["kv_idx"][tab["kv_ptr"][row]:tab["kv_ptr"][row + 1]]:
            c0, c1 = c * block_kv, min((c + 1) * block_kv, kv_len)
            out[r0:r1, c0:c1] = M[r0:r1, c0:c1]
    return out


def slice_rows(src, B_tab, H_tab, src_q_len, src_kv_len, block_q, block_kv, src_q_offset,
               q_len, kv_len, q_offset):
    """Block tables for query rows [q_offset, q_offset + q_len) (global positions) and keys
    [0, kv_len), cut out of tables ``src`` built for a longer geometry.

    Source: "FlexAttention: from rules to fused kernels", section 5.2 -- a mask prebuilt
    for a maximum length is reused by taking the query block that holds the current
    position (the rule keeps seeing global positions), and partial blocks keep the
    exact rule; the query rows of one new block must lie inside one prebuilt block.
    Section 2.2 of the same page -- a shorter square mask is the top-left crop of the
    longer one, valid only for rules that do not read the total length.
    A prebuilt FULL block stays FULL for a subset of its rows and in-range columns, a
    listed PARTIAL block stays PARTIAL (it is masked exactly), an unlisted block stays
    unlisted; columns past the new kv_len are dropped.

    Raises ValueError when the new query blocks do not each sit inside one prebuilt
    query block, or the new rows or keys are not covered by the prebuilt ones.
    """
    if kv_len > src_kv_len or q_offset < src_q_offset or q_offset + q_len > src_q_offset + src_q_len:
        raise ValueError("the slice must lie inside the prebuilt rows and keys")
    delta = q_offset - src_q_offset
    nqb, nkb = n_blocks(q_len, block_q), n_blocks(kv_len, block_kv)
    nqb_src = n_blocks(src_q_len, block_q)
    aligned = delta % block_q == 0
    single = nqb == 1 and delta // block_q == (delta + q_len - 1) // block_q
    if nqb > 0 and not (aligned or single):
        raise ValueError("each new query block must sit inside one prebuilt query block")
    r_base = delta // block_q
    rows = np.zeros((B_tab * H_tab * nqb, nkb), dtype=np.uint8)
    for bh in range(B_tab * H_tab):
        for k in range(nqb):
            srow = bh * nqb_src + r_base + k
            for key, cls in (("kv", PARTIAL), ("full_kv", FULL)):
                lst = src[f"{key}_idx"][src[f"{key}_ptr"][srow]:src[f"{key}_ptr"][srow + 1]]
                for c in lst:
                    if c < nkb:
                        rows[bh * nqb + k, c] = cls
    cols = np.concatenate([rows[bh * nqb:(bh + 1) * nqb].T for bh in range(B_tab * H_tab)]) \
        if B_tab * H_tab * nqb else np.zeros((B_tab * H_tab * nkb, 0), np.uint8)
    kv = _compact(rows)
    q = _compact(cols)
    names = ("num", "ptr", "idx")
    out = {}
    for k, v in zip([f"kv_{n}" for n in names] + [f"full_kv_{n}" for n in names], kv):
        out[k] = v
    for k, v in zip([f"q_{n}" for n in names] + [f"full_q_{n}" for n in names], q):
        out[k] = v
    return out
