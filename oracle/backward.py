"""Gradients of the dense attention definition (test infrastructure).

Source: "FlexAttention: from rules to fused kernels", section 4 -- the backward of the
fused kernel recomputes the scores of each executed block from the saved row
log-sum-exp, differentiates score_mod, and accumulates dQ over a query row's KV list
and dK/dV over a KV column's query list (the transposed tables).  What it computes
is the gradient of the forward definition itself, which this module obtains by
float64 autograd of the plain dense formula (scaled scores, score_mod, mask to -inf,
softmax, weighted sum of V) for the scalar loss sum(O * dO).  A row with no allowed
key has O = 0 and passes no gradient.

Parity: pinned in tests/test_oracle_pins.py by central finite differences of the
forward oracle (numpy, no autograd) on tiny inputs for every score_mod -- of Q, K, V
and of the ALiBi slopes and the relative-position table -- and by torch's own
scaled-dot-product-attention backward on a causal case.
"""
from __future__ import annotations

import math

import numpy as np

from . import masks


def _t64(x):
    import torch
    if hasattr(x, "detach"):
        return x.detach().to("cpu").to(torch.float64)
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def attention_grads(q, k, v, do, mask, score="identity", cap=None, slopes=None, table=None,
                    radius=None, q_offset=0, doc_ids=None, scale=None, param_grads=False):
    """dQ [B, Hq, q_len, d], dK and dV [B, Hkv, kv_len, d] (float64 numpy) of
    loss = sum(O * dO), O the dense attention output.  With ``param_grads`` the
    gradient of the score_mod parameter follows: ALiBi slopes [Hq] or the relative-
    position table [Hq, 2R+1] (None for the other kinds)."""
    import torch
    Q = _t64(q).requires_grad_(True)
    K = _t64(k).requires_grad_(True)
    V = _t64(v).requires_grad_(True)
    dO = _t64(do)
    SL = _t64(slopes).requires_grad_(True) if score == "alibi" else None
    TB = _t64(table).requires_grad_(True) if score == "relpos" else None
    B, Hq, q_len, d = Q.shape
    Hkv, kv_len = K.shape[1], K.shape[2]
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    i_np = (np.arange(q_len, dtype=np.int64) + int(q_offset))[:, None]
    j_np = np.arange(kv_len, dtype=np.int64)[None, :]
    i_t = torch.as_tensor(i_np, dtype=torch.float64)
    j_t = torch.as_tensor(j_np, dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    for b in range(B):
        doc_row = masks.doc_row_for(doc_ids, b)
        if not callable(mask):
            M = torch.as_tensor(np.broadcast_to(masks.evaluate(mask, i_np, j_np, doc_row), (q_len, kv_len)).copy())
            empty = ~M.any(dim=1, keepdim=True)
        for h in range(Hq):
            if callable(mask):      # an arbitrary allowed-pair function of (b, h, i, j)
                M = torch.as_tensor(np.broadcast_to(mask(b, h, i_np, j_np), (q_len, kv_len)).copy())
                empty = ~M.any(dim=1, keepdim=True)
            hkv = h // g
            S = (Q[b, h] @ K[b, hkv].T) * scale
            if score == "softcap":
                S = cap * torch.tanh(S / cap)
            elif score == "alibi":
                S = S + SL[h] * (j_t - i_t)
            elif score == "relpos":
                R = int(radius)
                rel = torch.as_tensor(np.clip(i_np - j_np, -R, R) + R)
                S = S + TB[h][rel]
            elif score != "identity":
                raise ValueError(f"unknown score_mod {score!r}")
            S = S.masked_fill(~M, -math.inf)
            S = torch.where(empty, torch.zeros_like(S), S)      # empty rows: no -inf row
            P = torch.softmax(S, dim=1) * M                      # ... and zero weights
            loss = loss + ((P @ V[b, hkv]) * dO[b, h]).sum()
    loss.backward()
    out = (Q.grad.numpy(), K.grad.numpy(), V.grad.numpy())
    if param_grads:
        P = SL if SL is not None else TB
        grad = None if P is None else (P.grad.numpy() if P.grad is not None else np.zeros(tuple(P.shape)))
        out = out + (grad,)
    return out
