"""Host-side checks of the benchmark's bookkeeping (no GPU): the one-GPU contract and
the algorithmic work credited per step."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


def _tab(kv_num, full_kv_num):
    kv_num, full_kv_num = np.asarray(kv_num, np.int32), np.asarray(full_kv_num, np.int32)
    return {"kv_num": kv_num, "full_kv_num": full_kv_num,
            "kv_ptr": np.concatenate([[0], np.cumsum(kv_num)]).astype(np.int32),
            "full_kv_ptr": np.concatenate([[0], np.cumsum(full_kv_num)]).astype(np.int32)}


def test_accounting_broadcast_tables():
    w = W.WORKLOADS["causal_softcap"]
    nqb = w.q_len // w.block_q
    tab = _tab(np.ones(nqb), np.arange(nqb))            # causal: r full + 1 partial per row
    acc = bench.accounting(w, tab)
    executed = nqb + nqb * (nqb - 1) // 2
    assert acc["executed_blocks_per_head"] == executed == 528
    assert acc["flop"] == w.B * w.Hq * executed * 4 * w.block_q * w.block_kv * w.d


def test_accounting_per_head_tables():
    w = W.WORKLOADS["select_uniform"]
    nqb = w.q_len // w.block_q
    lens = np.full(w.B * w.Hq * nqb, 13)
    acc = bench.accounting(w, _tab(np.zeros_like(lens), lens), w.B * w.Hq)
    assert acc["flop"] == int(lens.sum()) * 4 * w.block_q * w.block_kv * w.d
    assert acc["per_entry_executed"] == [13 * nqb] * (w.B * w.Hq)
    # decode with per-head tables: every query head reads the K and V of its own blocks
    wd = W.WORKLOADS["decode_select"]
    lens = np.full(wd.B * wd.Hq, 32)
    accd = bench.accounting(wd, _tab(np.zeros_like(lens), lens), wd.B * wd.Hq)
    kv = wd.B * wd.Hq * 32 * wd.block_kv * wd.d * 2 * 2
    assert kv <= accd["bytes"] < kv * 1.01


def test_row_stats():
    st = bench.row_stats(_tab([0, 1, 0, 2], [3, 0, 1, 9]))
    assert st["rows"] == 4 and st["max"] == 11 and st["full"] == 13 and st["partial"] == 3
    assert abs(st["mean"] - 4.0) < 1e-12 and st["p50"] == 2.0
