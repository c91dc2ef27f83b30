"""Element predicate of the mask menu, evaluated on index arrays (test infrastructure).

Sources (page title, then section):

* "FlexAttention: from rules to fused kernels", section 1.1 -- a mask function
  takes only indices and captured tensors and decides whether the connection
  (q, k) exists; causal is ``i >= j``, a left window W adds ``i - j < W``, a
  document mask requires ``d_b(i) == d_b(j)``; and/or compositions are set
  intersection and union.
* "FlexAttention: compiler optimization of custom attention", section 1 and 2 --
  the window W includes the current token (``q - kv < W`` and ``q >= kv``; with
  W = 4, query 6 sees keys 3..6).
* "FlexAttention: from rules to fused kernels", section 6.3 -- prefix-LM lets
  every query read the first P keys and is causal afterwards; the document
  version is the intersection with the document mask.
* "FlexAttention: compiler optimization of custom attention", section 6 -- in
  decode the local query index is shifted by the global offset t before the
  rule is evaluated.

Reading taken where the pages lost the formula: SWA(W) = (j <= i) and (i - j < W);
PREFIX(P) = (j < P) or (j <= i); positions are global (i = local row + q_offset).
"""
from __future__ import annotations

import numpy as np


def evaluate(spec, i, j, doc_row=None):
    """Boolean array M[i, j] for the mask tree ``spec``.

    ``i`` and ``j`` are integer arrays that broadcast against each other (global
    query positions and key positions).  ``doc_row`` is the int32 document-ID
    vector of the batch entry, indexed by global position; it is needed only
    when the tree contains a ``("doc",)`` leaf.
    """
    op = spec[0]
    if op == "causal":
        return j <= i
    if op == "swa":
        W = int(spec[1])
        return (j <= i) & ((i - j) < W)
    if op == "prefix":
        P = int(spec[1])
        return (j < P) | (j <= i)
    if op == "doc":
        if doc_row is None:
            raise ValueError("document mask needs document IDs")
        return doc_row[i] == doc_row[j]
    if op == "and":
        return evaluate(spec[1], i, j, doc_row) & evaluate(spec[2], i, j, doc_row)
    if op == "or":
        return evaluate(spec[1], i, j, doc_row) | evaluate(spec[2], i, j, doc_row)
    raise ValueError(f"unknown mask node {op!r}")


def doc_row_for(doc_ids, b):
    """Document-ID vector for batch entry ``b`` (a single row broadcasts)."""
    if doc_ids is None:
        return None
    doc_ids = np.asarray(doc_ids)
    if doc_ids.ndim == 1:
        return doc_ids
    return doc_ids[0] if doc_ids.shape[0] == 1 else doc_ids[b]


def dense(spec, q_len, kv_len, q_offset=0, doc_row=None, rows=None):
    """The [q_len, kv_len] boolean matrix of allowed pairs for one batch entry.

    ``rows`` optionally restricts to a subset of local query rows (the result
    then has ``len(rows)`` rows).
    """
    li = np.arange(q_len, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    i = (li + int(q_offset))[:, None]
    j = np.arange(kv_len, dtype=np.int64)[None, :]
    return np.broadcast_to(evaluate(spec, i, j, doc_row), (len(li), kv_len)).copy()
