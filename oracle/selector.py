"""Block tables from selector output, and the longest-row-first work order (test
infrastructure).

Sources (page title, then section):

* "FlexAttention: from rules to fused kernels", section 5.2 -- a dynamic selector
  emits, per query block, candidate KV blocks; when its granularity is the kernel's
  block, sorting and de-duplicating the candidates yields each row's KV block list;
  rows of different candidate counts unbalance the work, and the row lengths of the
  tables are the signal for bucketing query tiles by their executed blocks.
  Section 6.3 -- a selector's output is a candidate list whose range, order and
  repeats must be checked.
* "Kernels: turning logical sparsity into real speed", section 3 -- a repeated block
  would be computed twice and change the probabilities, so repeats are removed before
  the kernel; section 3.1 -- with whole-block selection every legal token of a chosen
  block takes part in the softmax; sections 1.2 and 5 -- uneven candidate counts are
  met by bucketing rows by length or by a task queue.

Readings taken: a candidate outside [0, NKB) is dropped (padding such as -1 uses this);
repeats count once (set semantics); the allowed pairs are those of the structural rule
inside the chosen blocks, M(i, j) = R(i, j) and floor(j / B_kv) in S(b', h', r) with
r = floor(i_local / B_q); blocks are then classified exactly (section 6.3).  The work
order lists, per table entry (b', h'), the query blocks by descending executed-block
count, ties by descending block index.
"""
from __future__ import annotations

import numpy as np

from . import blockmask as OB
from . import masks


def canonical_sets(sel, nkb):
    """Per row of ``sel`` (int array [..., k]): the sorted, repeat-free candidates in
    [0, nkb).  Returns a list (row-major over the leading axes) of int32 arrays."""
    sel = np.asarray(sel)
    out = []
    for row in sel.reshape(-1, sel.shape[-1]) if sel.size else np.zeros((int(np.prod(sel.shape[:-1])), 0), int):
        kept = sorted({int(c) for c in row if 0 <= int(c) < nkb})
        out.append(np.asarray(kept, dtype=np.int32))
    return out


def selected_mask(spec, sets, H_tab, b, h, q_len, kv_len, block_q, block_kv, q_offset=0, doc_row=None,
                  rows=None):
    """Dense allowed-pair matrix of table entry (b', h') = (b, h): the rule inside the
    chosen blocks.  ``sets`` is canonical_sets over [B', H', NQB, k]."""
    nqb = OB.n_blocks(q_len, block_q)
    li = np.arange(q_len) if rows is None else np.asarray(rows, np.int64)
    M = masks.dense(spec, q_len, kv_len, q_offset, doc_row, rows=li)
    chosen = np.zeros((len(li), kv_len), dtype=bool)
    cols = np.arange(kv_len) // block_kv
    for n, i in enumerate(li):
        S = sets[(b * H_tab + h) * nqb + int(i) // block_q]
        chosen[n] = np.isin(cols, S)
    return M & chosen


def classify_dense(M, block_q, block_kv):
    """Class grid [NQB, NKB] of an arbitrary allowed-pair matrix: EMPTY when no in-range
    pair of the block is allowed, FULL when all are, PARTIAL otherwise."""
    q_len, kv_len = M.shape
    nqb, nkb = OB.n_blocks(q_len, block_q), OB.n_blocks(kv_len, block_kv)
    grid = np.zeros((nqb, nkb), dtype=np.uint8)
    for r in range(nqb):
        for c in range(nkb):
            blk = M[r * block_q:(r + 1) * block_q, c * block_kv:(c + 1) * block_kv]
            grid[r, c] = OB.FULL if blk.all() else (OB.PARTIAL if blk.any() else OB.EMPTY)
    return grid


def tables_from_selection(spec, sel, B_tab, H_tab, q_len, kv_len, block_q, block_kv, q_offset=0, doc_ids=None):
    """Both sides of the block tables for selector output ``sel`` [B', H', NQB, k] under
    rule ``spec``; rows ordered (b', h', r), columns (b', h', c)."""
    nkb = OB.n_blocks(kv_len, block_kv)
    sets = canonical_sets(sel, nkb)
    row_grids, col_grids = [], []
    for b in range(B_tab):
        doc_row = masks.doc_row_for(doc_ids, b)
        for h in range(H_tab):
            M = selected_mask(spec, sets, H_tab, b, h, q_len, kv_len, block_q, block_kv, q_offset, doc_row)
            g = classify_dense(M, block_q, block_kv)
            row_grids.append(g)
            col_grids.append(g.T)
    rows = np.concatenate(row_grids) if row_grids else np.zeros((0, nkb), np.uint8)
    cols = np.concatenate(col_grids) if col_grids else np.zeros((0, 0), np.uint8)
    out = {}
    names = ("num", "ptr", "idx")
    for pre, part in (("", rows), ("q_", cols)):
        vals = OB._compact(part)
        keys = [f"{pre or 'kv_'}{n}" for n in names] + [f"full_{pre or 'kv_'}{n}" for n in names]
        out.update(zip(keys, vals))
    return out


def work_order(tab, B_tab, H_tab, q_len, block_q):
    """Per table entry (b', h'): query blocks by descending executed-block count (full
    plus partial), ties by descending block index.  int32 [B' * H' * NQB]."""
    nqb = OB.n_blocks(q_len, block_q)
    order = np.zeros(B_tab * H_tab * nqb, dtype=np.int32)
    n = tab["kv_num"] + tab["full_kv_num"]
    for g in range(B_tab * H_tab):
        lens = n[g * nqb:(g + 1) * nqb]
        order[g * nqb:(g + 1) * nqb] = sorted(range(nqb), key=lambda r: (-int(lens[r]), -r))
    return order


def row_lists(spec, sets, H_tab, b, h, r, q_len, kv_len, block_q, block_kv, q_offset=0, doc_row=None):
    """(partial, full) KV block lists of one table row (b', h', r), from the rows of its
    query block only (for sampled checks at sizes where whole tables are too slow)."""
    rows = np.arange(r * block_q, min((r + 1) * block_q, q_len))
    M = selected_mask(spec, sets, H_tab, b, h, q_len, kv_len, block_q, block_kv, q_offset, doc_row, rows=rows)
    g = classify_dense(M, block_q, block_kv)[0]
    return np.nonzero(g == OB.PARTIAL)[0].astype(np.int32), np.nonzero(g == OB.FULL)[0].astype(np.int32)
