"""Merge law of partial softmax states (test infrastructure).

Source: "Kernels: turning logical sparsity into real speed", section 3 -- for a
processed key set A keep m_A = max s_j, l_A = sum exp(s_j - m_A) and
u_A = sum exp(s_j - m_A) v_j; merging with a set B uses m = max(m_A, m_B),
l = e^(m_A - m) l_A + e^(m_B - m) l_B, u likewise, and the output is u / l, in any
order.  "FlexAttention: compiler optimization of custom attention", section 6 --
split-KV outputs are combined with weights from each split's denominator, and an
empty split contributes zero.

Only used to pin the split-KV combination; the attention oracle itself never splits.
"""
from __future__ import annotations

import numpy as np


def partial_state(s, v):
    """(m, l, u) of one key subset: scores s [n] (may hold -inf), values v [n, d]."""
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if s.size == 0 or not np.isfinite(s).any():
        return -np.inf, 0.0, np.zeros(v.shape[1])
    m = s.max()
    w = np.exp(s - m)
    return m, w.sum(), w @ v


def merge(states):
    """Merge a list of (m, l, u) states; returns (O, LSE) with O = 0, LSE = -inf
    when every state is empty."""
    ms = np.array([st[0] for st in states], dtype=np.float64)
    if not np.isfinite(ms).any():
        d = len(states[0][2])
        return np.zeros(d), -np.inf
    m = ms.max()
    l = 0.0
    u = np.zeros_like(np.asarray(states[0][2], dtype=np.float64))
    for mi, li, ui in states:
        if not np.isfinite(mi):
            continue
        w = np.exp(mi - m)
        l += w * li
        u = u + w * np.asarray(ui, dtype=np.float64)
    return u / l, m + np.log(l)
