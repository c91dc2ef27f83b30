#!/usr/bin/env python3
"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = fa_create_block_mask + fa_forward over one synthetic batch of the chosen
workload (default: the 64K prefix-LM with a relative-position table, B=1, Hq=16,
Hkv=2, N=65536, d=128, 128x128 blocks -- the largest single-GPU configuration).
Inputs are resident in HBM before the timed region starts.

Printed: ONE JSON line with the throughput over executed blocks (TFLOP/s for prefill
workloads, GB/s for decode workloads), the roofline position of the dominant kernel
(timed with HIP events on its launch stream inside the timed region) and the CPU oracle
timed on a bounded sample of the same workload.  The same line carries a "decode"
object (split-KV decode, B=64, KV 32768, GB/s against HBM) and an "extra" object with
the causal soft-cap and GQA document-window workloads, each with its own steps,
roofline and oracle baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "block-sparse attn fwd TFLOP/s (executed blocks), % bf16 MFMA peak; decode GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


KERNEL_SOURCES = {
    "prefill": ("prefill.hip", "prefill_common.hpp", "device_common.hpp", "fa_internal.hpp"),
    "decode": ("decode.hip", "prefill_common.hpp", "device_common.hpp", "fa_internal.hpp"),
}


def kernel_source_digest(kernel):
    """Digest of the source files a kernel is built from (a counter summary taken on
    other sources no longer describes it)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_programmable_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per dispatch from the committed rocprofv3 counter summary, or None
    if there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.lstrip().startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != kernel_source_digest(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


def accounting(w, tab, entries=1):
    """Executed blocks and algorithmic work of one step; ``entries`` = B' * H' of the
    tables (1: one table row set broadcast over every (batch, head))."""
    nf = int(tab["full_kv_ptr"][-1])
    npart = int(tab["kv_ptr"][-1])
    heads = w.B * w.Hq
    executed = nf + npart
    acc = {"full_blocks": nf, "partial_blocks": npart,
           "executed_blocks_per_head": executed if entries == 1 else None}
    if entries > 1:
        # per-(batch, head) tables: total executed blocks over all of them
        lens = tab["kv_num"] + tab["full_kv_num"]
        total = int(lens.sum()) * (heads // entries)
        acc["per_entry_executed"] = lens.reshape(entries, -1).sum(axis=1).tolist()
        if w.q_len == 1:
            # every query head reads the K and V of its own blocks (its group's KV head)
            acc["bytes"] = (total * w.block_kv * w.d * 2 * 2 + 2 * w.B * w.Hq * w.d * 2 + w.B * w.Hq * 4
                            + 4 * int(lens.size + lens.sum()))
            acc["flop"] = total * w.block_kv * 4 * w.d
        else:
            acc["flop"] = total * 4 * w.block_q * w.block_kv * w.d
        return acc
    if w.q_len == 1:
        kv_bytes = w.B * w.Hkv * executed * w.block_kv * w.d * 2 * 2
        q_bytes = w.B * w.Hq * w.q_len * w.d * 2
        idx_bytes = 4 * (executed + 4)
        if w.page_size:   # page-table entries of the executed blocks, per request
            idx_bytes += 4 * w.B * executed * (w.block_kv // w.page_size)
        acc["bytes"] = kv_bytes + 2 * q_bytes + w.B * w.Hq * w.q_len * 4 + idx_bytes
        acc["flop"] = heads * executed * w.block_kv * 4 * w.d * w.q_len
    else:
        acc["flop"] = heads * executed * 4 * w.block_q * w.block_kv * w.d
    return acc


def row_stats(tab):
    """Row lengths (executed blocks per table row): mean, P50, P95, max, and the
    full/partial split ("FlexAttention: from rules to fused kernels", section 6.3)."""
    import numpy as np
    lens = tab["kv_num"] + tab["full_kv_num"]
    return {"rows": int(lens.size), "mean": float(lens.mean()), "p50": float(np.percentile(lens, 50)),
            "p95": float(np.percentile(lens, 95)), "max": int(lens.max()),
            "full": int(tab["full_kv_ptr"][-1]), "partial": int(tab["kv_ptr"][-1])}


def _blas_threads():
    """BLAS threads numpy uses: os.cpu_count(), capped by OMP_NUM_THREADS when the
    environment sets it (a machine's CPU share can be smaller than its core count)."""
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def _spread(n):
    """0 .. n-1 in an order that samples the whole range early (stride coprime to n)."""
    if n <= 2:
        return list(range(n))
    step = max(1, int(n * 0.618))
    while math.gcd(step, n) != 1:
        step += 1
    return [(x * step) % n for x in range(n)]


def cpu_baseline(w, aux, q, k, v, acc, tab_host, budget_s):
    """The oracle, as is, on a bounded sample of the same workload, with numpy's BLAS
    on ``_blas_threads()`` threads.  Block tables: the whole grid, or for grids of more
    than 64 query blocks 16 query blocks (four runs of four, spread over the grid, each
    classified as the rows [r0 B_q, (r0 + 4) B_q) of the same rule) prorated to the grid.
    Attention: whole query blocks (prefill; spread over the rows, heads in turn) or whole
    requests (decode), until the time budget is used, each credited with its own
    executed-block FLOP (bytes for decode)."""
    import numpy as np
    from oracle import attention as OA
    from oracle import blockmask as OB
    threads = _blas_threads()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(threads)
    except Exception:   # pragma: no cover - threadpoolctl is part of the image
        limiter = None
    nqb = -(-w.q_len // w.block_q)
    mask_of = lambda b, h=None: w.mask   # noqa: E731
    t0 = time.perf_counter()
    if w.selector:
        # the selected-pair matrix is evaluated inside the attention, row chunk by chunk;
        # the oracle sees a one-request (and, for prefill, one-head) slice, so the global
        # request and head are bound here (h None: the slice holds every head)
        import workloads as W
        from oracle import selector as OS
        sets = OS.canonical_sets(W.selector_indices(w), -(-w.kv_len // w.block_kv))
        t_tab = time.perf_counter() - t0
        tab_sample = "selector candidate sets (canonicalised)"

        def mask_of(b, h=None):
            def fn(bb, hh, i, j):
                rows = np.asarray(i).reshape(-1) - w.q_offset
                M = OS.selected_mask(w.mask, sets, w.Hq, b, hh if h is None else h, w.q_len, w.kv_len,
                                     w.block_q, w.block_kv, w.q_offset, None, rows=rows)
                return M[:, np.asarray(j).reshape(-1)]
            return fn
    elif nqb <= 64:
        OB.tables(w.mask, 1, 1, w.q_len, w.kv_len, w.block_q, w.block_kv, w.q_offset, aux["doc_ids"])
        t_tab = time.perf_counter() - t0
        tab_sample = f"whole grid ({nqb} query blocks)"
    else:
        starts = [(nqb * x) // 4 for x in range(4)]
        for r0 in starts:
            n = min(4, nqb - r0)
            OB.tables(w.mask, 1, 1, min(n * w.block_q, w.q_len - r0 * w.block_q), w.kv_len, w.block_q,
                      w.block_kv, w.q_offset + r0 * w.block_q, aux["doc_ids"])
        t_tab = (time.perf_counter() - t0) * nqb / 16
        tab_sample = f"16 of {nqb} query blocks (rows from blocks {starts}, four each), prorated"
    kw = dict(cap=w.cap or None, radius=w.relpos_radius, doc_ids=aux["doc_ids"])
    done = 0
    t_attn = 0.0
    credited = 0.0
    if w.q_len == 1:
        units = w.B
        per_unit = acc["bytes"] / w.B
        while done < units and t_attn < budget_s:
            b = done
            qb, kb, vb = (OA._as_f64(t[b:b + 1]) for t in (q, k, v))
            t1 = time.perf_counter()
            OA.attention(qb, kb, vb, mask_of(b), w.score, slopes=aux["slopes"], table=aux["table"],
                         q_offset=w.q_offset, **kw)
            t_attn += time.perf_counter() - t1
            done += 1
            credited += per_unit
        value = credited / (t_attn + t_tab) / 1e9
        unit = "GB/s"
        sample = f"{done} of {units} requests (all {w.Hq} heads), credited with their bytes"
    else:
        lens = np.asarray(tab_host["kv_num"]) + np.asarray(tab_host["full_kv_num"])
        per_entry = "per_entry_executed" in acc
        blk_flop = 4 * w.block_q * w.block_kv * w.d
        units = w.B * w.Hq * nqb
        order = _spread(nqb)
        kvc, qc = {}, {}
        while done < units and t_attn < budget_s:
            r = order[done % nqb]
            b, h = divmod((done // nqb + done) % (w.B * w.Hq), w.Hq)
            hkv = h // w.g
            if (b, hkv) not in kvc:
                kvc = {(b, hkv): (OA._as_f64(k[b:b + 1, hkv:hkv + 1]), OA._as_f64(v[b:b + 1, hkv:hkv + 1]))}
            if (b, h) not in qc:
                qc = {(b, h): OA._as_f64(q[b:b + 1, h:h + 1])}
            kb, vb = kvc[(b, hkv)]
            r0, r1 = r * w.block_q, min((r + 1) * w.block_q, w.q_len)
            qb = qc[(b, h)][:, :, r0:r1]
            sl = None if aux["slopes"] is None else aux["slopes"][h:h + 1]
            tb = None if aux["table"] is None else aux["table"][h:h + 1]
            fn = mask_of(b, h)   # rules and pair functions both see global positions
            t1 = time.perf_counter()
            OA.attention(qb, kb, vb, fn, w.score, slopes=sl, table=tb, q_offset=w.q_offset + r0, **kw)
            t_attn += time.perf_counter() - t1
            row = (b * w.Hq + h) * nqb + r if per_entry else r
            credited += int(lens[row]) * blk_flop
            done += 1
        value = credited / (t_attn + t_tab * min(1.0, done / units)) / 1e12
        unit = "TFLOP/s"
        sample = (f"{done} of {units} (batch, head, query block) items, whole query blocks spread over "
                  f"the rows, each credited with its executed-block FLOP; block tables prorated to the "
                  f"sampled share")
    if limiter is not None:
        limiter.restore_original_limits()
    return {"value": value, "unit": unit, "cores": int(threads), "cpu_count": os.cpu_count(),
            "blas_threads": int(threads), "kind": "oracle", "sample": sample,
            "blockmask_oracle_s": round(t_tab, 3), "blockmask_sample": tab_sample,
            "attention_oracle_s": round(t_attn, 3), "seconds": round(t_attn + t_tab, 3)}


def run_workload(args, name, headline=True):
    """One workload: K timed steps (build + forward) after W warm-up steps, the forward
    timed with HIP events on its launch stream, the cold-cache legs, and the oracle on a
    bounded sample.  The optional legs (backward, prebuilt slices, the work-order
    comparison of selector tables) run for the headline workload only."""
    import numpy as np
    import torch

    import block_sparse_programmable_amd as fa
    import workloads as W

    w = W.WORKLOADS[name]
    torch.cuda.set_device(0)
    dev = "cuda"
    aux = W.aux_inputs(w)
    q, k, v = W.qkv(w, device=dev)
    docT = None if aux["doc_ids"] is None else torch.as_tensor(aux["doc_ids"]).to(dev)
    sl = None if aux["slopes"] is None else torch.as_tensor(aux["slopes"]).to(dev)
    tb = None if aux["table"] is None else torch.as_tensor(aux["table"]).to(dev)

    if w.selector:
        # selector workloads: per-head tables from the selector output, with the work order
        selT = torch.as_tensor(W.selector_indices(w)).to(dev)

        def build(tables=None, workspace=None, order=True):
            # the forward reads only the kv side; the backward leg needs the query side too
            return fa.block_mask_from_indices(selT, w.mask, w.B, w.Hq, w.q_len, w.kv_len, w.block_q,
                                              w.block_kv, w.q_offset, docT, tables=tables,
                                              workspace=workspace, order=order,
                                              q_side=bool(args.backward))
    else:
        # rule workloads: tables with the work order (longest rows first), which the
        # one-workgroup builder ranks in place for up to 256 query blocks; the forward
        # reads only the kv side, the backward leg needs the query side too
        def build(tables=None, workspace=None, order=True):
            return fa.create_block_mask(w.mask, 1, 1, w.q_len, w.kv_len, w.block_q, w.block_kv, w.q_offset,
                                        docT, tables=tables, workspace=workspace, order=order,
                                        q_side=bool(args.backward))
    bm = build()
    tables = bm.tensors
    bws = bm._keep[1]
    out = torch.empty(w.B, w.Hq, w.q_len, w.d, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(w.B, w.Hq, w.q_len, dtype=torch.float32, device=dev)
    fargs, _, _ = fa.forward_args(q, k, v, bm, w.score, w.cap, sl, tb, w.relpos_radius, None, out, lse)
    fws_bytes = fa.forward_workspace_size(fargs)
    fws = torch.empty(max(fws_bytes, 1), dtype=torch.uint8, device=dev)
    if w.page_size:
        # paged caches holding the same logical K/V through a fragmented page table
        pt_np = W.page_table(w)
        kc, vc = W.paged_caches(w, k, v, pt_np)
        ptT = torch.as_tensor(pt_np).to(dev)
    torch.cuda.synchronize()
    tab_host = bm.compact()
    acc = accounting(w, tab_host, bm.desc.B * bm.desc.H)

    def fwd(b):
        if w.page_size:
            fa.forward_paged(q, kc, vc, ptT, w.kv_len, b, score=w.score, softcap=w.cap, alibi_slopes=sl,
                             relpos=tb, relpos_radius=w.relpos_radius, out=out, lse=lse, workspace=fws)
        else:
            fa.forward(q, k, v, b, score=w.score, softcap=w.cap, alibi_slopes=sl, relpos=tb,
                       relpos_radius=w.relpos_radius, out=out, lse=lse, workspace=fws)

    def step(ev=None, i=0):
        b = build(tables=tables, workspace=bws)
        if ev is not None:
            ev[0][i].record()
        fwd(b)
        if ev is not None:
            ev[1][i].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = ([torch.cuda.Event(enable_timing=True) for _ in range(K)],
          [torch.cuda.Event(enable_timing=True) for _ in range(K)])
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(K):
        step(ev, i)
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K
    fwd_ms = [ev[0][i].elapsed_time(ev[1][i]) for i in range(K)]
    fwd_avg = float(np.mean(fwd_ms))

    # the builder and the forward alone, each with caches flushed before every
    # repetition (a 1 GiB read that is not timed; a read leaves clean lines, where a
    # write would leave dirty ones for the timed kernel to write back): the step loop
    # above runs back to back, where inputs that fit the last-level cache stay warm
    cold = {}
    if args.cold_reps > 0:
        flush = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        sink = torch.empty(2, dtype=torch.uint8, device=dev)
        e = [[torch.cuda.Event(enable_timing=True) for _ in range(args.cold_reps)] for _ in range(4)]
        for i in range(args.cold_reps):
            torch.amax(flush, dim=0, out=sink[0])
            e[0][i].record()
            b = build(tables=tables, workspace=bws)
            e[1][i].record()
            torch.amax(flush, dim=0, out=sink[1])
            e[2][i].record()
            fwd(b)
            e[3][i].record()
        torch.cuda.synchronize()
        bt = [e[0][i].elapsed_time(e[1][i]) for i in range(args.cold_reps)]
        ft = [e[2][i].elapsed_time(e[3][i]) for i in range(args.cold_reps)]
        cold = {"reps": args.cold_reps,
                "build_ms_median": float(np.median(bt)), "build_ms_p10": float(np.percentile(bt, 10)),
                "build_ms_p90": float(np.percentile(bt, 90)),
                "fwd_ms_median": float(np.median(ft)), "fwd_ms_p10": float(np.percentile(ft, 10)),
                "fwd_ms_p90": float(np.percentile(ft, 90))}
        del flush, sink

    # backward of the same step's forward (prefill workloads): dQ, dK, dV over the
    # block tables, credited with 5 products of 2 Bq Bk d FLOP per executed block
    bwd = None
    if headline and args.backward and w.q_len > 1:
        dout = W.randn_bf16(tuple(out.shape), w.seed + 7, device=dev)
        fwd(bm)
        gq = torch.empty(q.shape, dtype=torch.float32, device=dev)
        gk = torch.empty(k.shape, dtype=torch.float32, device=dev)
        gv = torch.empty(v.shape, dtype=torch.float32, device=dev)
        bkw = dict(score=w.score, softcap=w.cap, alibi_slopes=sl, relpos=tb, relpos_radius=w.relpos_radius,
                   dq=gq, dk=gk, dv=gv)
        # warm-up to the steady state: the first few tens of milliseconds of back-to-back
        # backward calls run up to 15% slower on MI355X (clocks ramping under the load)
        t_end = time.perf_counter() + 0.2
        while time.perf_counter() < t_end:
            for _ in range(10):
                fa.backward(q, k, v, out, lse, dout, bm, **bkw)
            torch.cuda.synchronize()
        nb = max(10, K)
        e = [[torch.cuda.Event(enable_timing=True) for _ in range(nb)] for _ in range(2)]
        for i in range(nb):
            e[0][i].record()
            fa.backward(q, k, v, out, lse, dout, bm, **bkw)
            e[1][i].record()
        torch.cuda.synchronize()
        bt = [e[0][i].elapsed_time(e[1][i]) for i in range(nb)]
        bflop = acc["flop"] * 5 // 2
        bwd = {"reps": nb, "ms_mean": float(np.mean(bt)), "ms_p10": float(np.percentile(bt, 10)),
               "ms_p90": float(np.percentile(bt, 90)), "algorithmic_flop": bflop,
               "tflops": bflop / (float(np.mean(bt)) * 1e-3) / 1e12,
               "frac_bf16_peak": bflop / (float(np.mean(bt)) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}

    # selector workloads: the forward over tables with and without the work order (the
    # latter hands query blocks out by descending index), alternating, back to back, to
    # show what the longest-first order buys
    no_order = None
    if headline and w.selector:
        bm_n = build(order=False)
        R = max(20, K)
        e = [[torch.cuda.Event(enable_timing=True) for _ in range(R)] for _ in range(4)]
        for _ in range(3):
            fwd(bm_n)
            fwd(bm)
        for i in range(R):
            e[0][i].record()
            fwd(bm_n)
            e[1][i].record()
            fwd(bm)
            e[2][i].record()
        torch.cuda.synchronize()
        nt = [e[0][i].elapsed_time(e[1][i]) for i in range(R)]
        ot = [e[1][i].elapsed_time(e[2][i]) for i in range(R)]
        no_order = {"reps": R, "fwd_ms_mean": float(np.mean(nt)), "fwd_ms_p10": float(np.percentile(nt, 10)),
                    "fwd_ms_p90": float(np.percentile(nt, 90)),
                    "with_order_fwd_ms_mean": float(np.mean(ot)),
                    "with_order_fwd_ms_p10": float(np.percentile(ot, 10))}
        del bm_n

    # decode from tables prebuilt once for the whole context: per step, slice the query
    # block of the current position (kv side only) instead of rebuilding; the forward
    # over the slice is timed beside the forward over rebuilt tables
    pre = None
    decode = w.q_len == 1
    if headline and args.prebuilt and decode:
        Lmax = w.kv_len
        eb = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        eb[0].record()
        src = fa.create_block_mask(w.mask, 1, 1, Lmax, Lmax, w.block_q, w.block_kv, 0, docT)
        eb[1].record()
        torch.cuda.synchronize()
        sl_bm = fa.slice_block_mask(src, w.q_len, w.kv_len, w.q_offset, q_side=False)
        R = max(20, K)
        e = [[torch.cuda.Event(enable_timing=True) for _ in range(R)] for _ in range(6)]
        for i in range(R):
            e[0][i].record()
            fa.slice_block_mask(src, w.q_len, w.kv_len, w.q_offset, q_side=False, tables=sl_bm.tensors,
                                workspace=sl_bm._keep[1])
            e[1][i].record()
            fa.create_block_mask(w.mask, 1, 1, w.q_len, w.kv_len, w.block_q, w.block_kv, w.q_offset,
                                 docT, tables=tables, workspace=bws)
            e[2][i].record()
        for i in range(R):
            e[3][i].record()
            fwd(sl_bm)
            e[4][i].record()
        torch.cuda.synchronize()
        o_slice = out.float().clone()
        fwd(bm)
        torch.cuda.synchronize()
        st = [e[0][i].elapsed_time(e[1][i]) for i in range(R)]
        rt = [e[1][i].elapsed_time(e[2][i]) for i in range(R)]
        ft = [e[3][i].elapsed_time(e[4][i]) for i in range(R)]
        sc = sl_bm.compact()
        pre = {"lmax": Lmax, "prebuild_ms": eb[0].elapsed_time(eb[1]), "reps": R,
               "slice_ms_median": float(np.median(st)), "rebuild_ms_median": float(np.median(rt)),
               "fwd_over_slice_ms_mean": float(np.mean(ft)), "fwd_over_rebuilt_ms_mean": fwd_avg,
               "slice_blocks": int(sc["kv_ptr"][-1] + sc["full_kv_ptr"][-1]),
               "rebuilt_blocks": acc["full_blocks"] + acc["partial_blocks"],
               "max_abs_o_diff": float((o_slice - out.float()).abs().max())}
        del src, sl_bm

    if decode:
        value = acc["bytes"] / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
        achieved = acc["bytes"] / (fwd_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": read_traffic("decode", w.name)}
    else:
        value = acc["flop"] / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = acc["flop"] / (fwd_avg * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": read_traffic("prefill", w.name)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, aux, q, k, v, acc, tab_host, args.cpu_seconds)

    cfg = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "q_len": w.q_len, "kv_len": w.kv_len,
           "d": w.d, "block_q": w.block_q, "block_kv": w.block_kv, "mask": repr(w.mask),
           "score_mod": w.score, "q_offset": w.q_offset, "seed": w.seed, "page_size": w.page_size or None,
           "selector": list(w.selector) if w.selector else None,
           "full_blocks": acc["full_blocks"], "partial_blocks": acc["partial_blocks"]}
    rec = {"value": value, "unit": unit, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
           "config": cfg, "roofline": roof, "cpu_baseline": cpu,
           "fwd_ms": fwd_avg, "fwd_ms_p10": float(np.percentile(fwd_ms, 10)),
           "fwd_ms_p90": float(np.percentile(fwd_ms, 90)),
           "algorithmic_flop": acc["flop"], "algorithmic_bytes": acc.get("bytes"),
           "cold_cache": cold or None,
           "backward": bwd,
           "prebuilt": pre,
           "row_lengths": row_stats(tab_host),
           "without_work_order": no_order,
           "kernel_source_digest": kernel_source_digest("decode" if decode else "prefill"),
           "gpu": torch.cuda.get_device_name(0),
           "torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    if decode:
        rec["forward_workspace_bytes"] = fws_bytes
    return rec


# Workloads timed beside the headline in the same line: the split-KV decode (GB/s
# against HBM) and the two shorter prefill workloads.
DECODE_WORKLOAD = "decode_swa_softcap"
EXTRA_WORKLOADS = ("causal_softcap", "gqa_doc_swa_alibi")


def run(args):
    import torch
    # the short workloads go first: right after seconds of the 64K prefill at full power
    # the memory-bound decode measured 7% slower than on its own
    decode, extra = None, {}
    if not args.no_extras:
        if args.workload != DECODE_WORKLOAD:
            decode = run_workload(args, DECODE_WORKLOAD, headline=False)
            torch.cuda.empty_cache()
        for name in EXTRA_WORKLOADS:
            if name != args.workload:
                extra[name] = run_workload(args, name, headline=False)
                torch.cuda.empty_cache()
    head = run_workload(args, args.workload, headline=True)
    torch.cuda.empty_cache()
    rec = {"metric": METRIC, "value": head.pop("value"), "unit": head.pop("unit"), "n_gpus": 1,
           "steps": head.pop("steps"), "warmup": head.pop("warmup"), "ms_per_step": head.pop("ms_per_step"),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic"}
    rec.update(head)
    rec["decode"] = decode
    rec["extra"] = extra
    return rec


def copy_calibration(mib):
    """A plain device-to-device copy of known size (for scaling HBM byte counters)."""
    import torch
    torch.cuda.set_device(0)
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_read": n, "copy_bytes_written": n, "copies": 3}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefix_relpos_64k")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the chosen workload only (no decode / extra prefill objects)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="time budget of the oracle's attention sample per workload")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward of the forward (prefill workloads)")
    ap.add_argument("--prebuilt", action="store_true",
                    help="decode workloads: also time slicing tables prebuilt for the whole context")
    ap.add_argument("--cold-reps", type=int, default=20,
                    help="repetitions of the separately timed build and forward with flushed caches")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args(argv)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(args.copy_calibration)))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path "
              f"(--gpus {args.gpus} requested); run with --gpus 1", file=sys.stderr)
        return 2
    rec = run(args)
    print(json.dumps(rec))
    return 0


if __name__ == "__main__":
    sys.exit(main())
