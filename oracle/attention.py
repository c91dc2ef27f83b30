"""Dense attention with score modification and masking, float64 (test infrastructure).

Definition followed (page title, then section):

* "FlexAttention: compiler optimization of custom attention", section 1 --
  O = softmax(Q K^T / sqrt(d)) V per batch entry and head; section 2 -- the
  score handed to score_mod is already scaled; the order is: modify the valid
  scores first, then set disallowed positions to -inf.  Soft-capping is
  CAP * tanh(score / CAP).  Section 5 -- the default scale is 1/sqrt(D).
* "FlexAttention: from rules to fused kernels", section 1.2 -- ALiBi adds a
  head-specific bias proportional to distance, indexed by the query head; a
  relative-position table adds r_h(i - j); GQA maps h_kv = floor(h_q / g).
  Section 3.1 -- a row with no valid key has no ordinary softmax; the output
  convention here is O = 0 and LSE = -inf.  Section 3.2 -- the log-sum-exp is
  an output next to O.
* "Flash Attention self-test answers", Q1 and Q24-29 -- S = Q K^T scale,
  P = softmax(S + mask), O = P V; the log-sum-exp summarises each row.

Readings taken: ALiBi bias = slope[h_q] * (j - i) with i, j global positions;
relative-position bias = table[h_q][clip(i - j, -R, R) + R]; LSE is the natural
log-sum-exp of the modified, masked row.  The score matrix is materialised
row-chunk by row-chunk; no online softmax is used.
"""
from __future__ import annotations

import math

import numpy as np

from . import masks


def score_mod(S, kind, h, i, j, cap=None, slopes=None, table=None, radius=None):
    """Apply the score modification to the (already scaled) float64 scores S.

    ``i`` (global query positions, column vector) and ``j`` (key positions, row
    vector) broadcast against S.
    """
    if kind == "identity":
        return S
    if kind == "softcap":
        return cap * np.tanh(S / cap)
    if kind == "alibi":
        return S + float(slopes[h]) * (j - i).astype(np.float64)
    if kind == "relpos":
        R = int(radius)
        rel = np.clip(i - j, -R, R) + R
        return S + np.asarray(table[h], dtype=np.float64)[rel]
    raise ValueError(f"unknown score_mod {kind!r}")


def _as_f64(x):
    if hasattr(x, "detach"):   # torch tensor (any dtype, including bfloat16)
        x = x.detach().to("cpu")
        import torch
        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def attention(q, k, v, mask, score="identity", cap=None, slopes=None, table=None,
              radius=None, q_offset=0, doc_ids=None, scale=None, rows=None,
              heads=None, batches=None, chunk=256):
    """O [B, Hq, n_rows, d] and LSE [B, Hq, n_rows] in float64.

    q: [B, Hq, q_len, d]; k, v: [B, Hkv, kv_len, d] (any float dtype; bf16 is
    up-cast exactly).  ``mask`` is a rule of the menu, or a function
    mask(b, h_q, i, j) -> bool array over global query positions i (column) and key
    positions j (row).  ``rows``/``heads``/``batches`` optionally restrict the
    computed outputs to a subset (the result keeps the full B and Hq extents
    only when these are None; otherwise the leading axes follow the subsets).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Hq, q_len, d = q.shape
    Hkv, kv_len = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(q_len) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(Hq)) if heads is None else list(heads)
    batches = list(range(B)) if batches is None else list(batches)
    O = np.zeros((len(batches), len(heads), len(rows), v.shape[-1]))
    L = np.zeros((len(batches), len(heads), len(rows)))
    j = np.arange(kv_len, dtype=np.int64)[None, :]
    for bi, b in enumerate(batches):
        doc_row = masks.doc_row_for(doc_ids, b)
        for hi, h in enumerate(heads):
            hkv = h // g
            K = k[b, hkv]
            V = v[b, hkv]
            for s in range(0, len(rows), chunk):
                rr = rows[s:s + chunk]
                i = (rr + int(q_offset))[:, None]
                S = (q[b, h, rr] @ K.T) * scale
                S = score_mod(S, score, h, i, j, cap, slopes, table, radius)
                if callable(mask):      # an arbitrary allowed-pair function of (b, h, i, j)
                    M = np.broadcast_to(mask(b, h, i, j), S.shape)
                else:
                    M = np.broadcast_to(masks.evaluate(mask, i, j, doc_row), S.shape)
                S = np.where(M, S, -np.inf)
                empty = ~M.any(axis=1)
                mx = np.where(empty, 0.0, S.max(axis=1))
                P = np.exp(S - mx[:, None])
                l = P.sum(axis=1)
                lse = np.where(empty, -np.inf, mx + np.log(np.where(empty, 1.0, l)))
                out = (P @ V) / np.where(empty, 1.0, l)[:, None]
                out[empty] = 0.0
                O[bi, hi, s:s + len(rr)] = out
                L[bi, hi, s:s + len(rr)] = lse
    return O, L
