"""Shared helpers of the GPU parity tests (HIP path through the C ABI vs the oracle)."""
import math

import numpy as np
import torch

from oracle import attention as OA
from oracle import blockmask as OB

O_TOL = 2e-2      # max-abs on O (bf16 output, fp32 accumulation)
LSE_TOL = 1e-3    # max-abs on finite LSE values

TABLE_SIDES = ("kv", "full_kv", "q", "full_q")


def gpu_tables(mask, B, H, q_len, kv_len, bq, bk, q_offset=0, doc=None):
    import block_sparse_programmable_amd as fa
    docT = None if doc is None else torch.as_tensor(np.asarray(doc, np.int32)).cuda()
    bm = fa.create_block_mask(mask, B, H, q_len, kv_len, bq, bk, q_offset, docT)
    torch.cuda.synchronize()
    return bm, bm.compact()


def assert_tables_equal(got, want, ctx=""):
    for side in TABLE_SIDES:
        for part in ("num", "ptr", "idx"):
            k = f"{side}_{part}"
            g, w = np.asarray(got[k]), np.asarray(want[k])
            assert g.shape == w.shape and (g == w).all(), f"{ctx}: {k} differs\n got {g[:40]}\nwant {w[:40]}"


def check_tables(mask, B, H, q_len, kv_len, bq, bk, q_offset=0, doc=None):
    _, got = gpu_tables(mask, B, H, q_len, kv_len, bq, bk, q_offset, doc)
    want = OB.tables(mask, B, H, q_len, kv_len, bq, bk, q_offset,
                     None if doc is None else np.asarray(doc))
    assert_tables_equal(got, want, f"{mask} B={B} H={H} q={q_len} kv={kv_len} {bq}x{bk} off={q_offset}")
    return got


def run_forward(q, k, v, mask, bq, bk, score="identity", q_offset=0, doc=None, tB=1, tH=1,
                cap=0.0, slopes=None, table=None, radius=0, scale=None, tables=None):
    import block_sparse_programmable_amd as fa
    B, Hq, q_len, d = q.shape
    kv_len = k.shape[2]
    docT = None if doc is None else torch.as_tensor(np.asarray(doc, np.int32)).cuda()
    bm = fa.create_block_mask(mask, tB, tH, q_len, kv_len, bq, bk, q_offset, docT)
    if tables is not None:
        tables(bm)
    slT = None if slopes is None else torch.as_tensor(np.asarray(slopes, np.float32)).cuda()
    tbT = None if table is None else torch.as_tensor(np.asarray(table, np.float32)).cuda()
    o, lse = fa.forward(q, k, v, bm, score=score, softcap=cap, alibi_slopes=slT, relpos=tbT,
                        relpos_radius=radius, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def compare(o, lse, O, L, ctx="", o_tol=O_TOL, lse_tol=LSE_TOL):
    """o/lse: GPU tensors or arrays matching O/L (oracle float64)."""
    o = o.float().cpu().numpy() if hasattr(o, "cpu") else np.asarray(o, np.float64)
    lse = lse.float().cpu().numpy() if hasattr(lse, "cpu") else np.asarray(lse, np.float64)
    assert np.isfinite(o).all(), f"{ctx}: non-finite O"
    err_o = float(np.abs(o - O).max()) if O.size else 0.0
    finite = np.isfinite(L)
    assert (np.isneginf(lse) == ~finite).all(), f"{ctx}: empty-row pattern differs"
    err_l = float(np.abs(lse[finite] - L[finite]).max()) if finite.any() else 0.0
    assert err_o <= o_tol, f"{ctx}: O max-abs error {err_o:.3e} > {o_tol}"
    assert err_l <= lse_tol, f"{ctx}: LSE max-abs error {err_l:.3e} > {lse_tol}"
    return err_o, err_l


def randn_bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16)


def oracle_forward(q, k, v, mask, score="identity", q_offset=0, doc=None, cap=None, slopes=None,
                   table=None, radius=None, scale=None, rows=None, heads=None, batches=None):
    return OA.attention(q.cpu(), k.cpu(), v.cpu(), mask, score, cap=cap, slopes=slopes,
                        table=table, radius=radius, q_offset=q_offset,
                        doc_ids=None if doc is None else np.asarray(doc), scale=scale,
                        rows=rows, heads=heads, batches=batches)


def workload_block_mask(w, docT=None, order=False):
    """The block tables a workload's forward runs on: built from the rule, or from the
    workload's selector output (per-head tables) for selector workloads."""
    import block_sparse_programmable_amd as fa
    import workloads as W
    if w.selector:
        sel = torch.as_tensor(W.selector_indices(w)).cuda()
        return fa.block_mask_from_indices(sel, w.mask, w.B, w.Hq, w.q_len, w.kv_len, w.block_q, w.block_kv,
                                          w.q_offset, docT, order=order)
    return fa.create_block_mask(w.mask, 1, 1, w.q_len, w.kv_len, w.block_q, w.block_kv, w.q_offset, docT,
                                order=order)


def workload_oracle_mask(w, doc_ids=None, batches=None):
    """The rule, or for selector workloads a pair function (b, h, i, j) -> bool that
    evaluates the oracle's selected-pair matrix on the rows asked for; ``batches`` maps
    the oracle's batch index to the workload's when it runs on a subset of requests."""
    import workloads as W
    from oracle import selector as OS
    if not w.selector:
        return w.mask
    sets = OS.canonical_sets(W.selector_indices(w), -(-w.kv_len // w.block_kv))

    def fn(b, h, i, j):
        b = b if batches is None else batches[b]
        rows = np.asarray(i).reshape(-1) - w.q_offset
        M = OS.selected_mask(w.mask, sets, w.Hq, b, h, w.q_len, w.kv_len, w.block_q, w.block_kv, w.q_offset,
                             None if doc_ids is None else np.asarray(doc_ids)[0], rows=rows)
        return M[:, np.asarray(j).reshape(-1)]
    return fn
