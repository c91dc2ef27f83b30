"""GPU block-table builder vs the oracle: bit-exact tables (GPU, via the C ABI)."""
import itertools

import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import assert_tables_equal, check_tables, gpu_tables
from oracle import blockmask as OB

pytestmark = pytest.mark.gpu

LEAVES = [("causal",), ("swa", 1), ("swa", 37), ("swa", 200), ("prefix", 0), ("prefix", 50),
          ("prefix", 128), ("doc",)]
PAIRS = [(op, a, b) for op in ("and", "or")
         for a, b in itertools.combinations([("causal",), ("swa", 37), ("prefix", 50), ("doc",)], 2)]


def docs_for(n, kind, seed=0):
    rng = np.random.default_rng(seed)
    if kind == "packed":
        lens = []
        while sum(lens) < n:
            lens.append(int(rng.integers(1, 90)))
        return np.repeat(np.arange(len(lens)), lens)[:n].astype(np.int32)
    if kind == "nonmono":
        return rng.integers(0, 3, n).astype(np.int32)
    return np.zeros(n, np.int32)


@pytest.mark.parametrize("spec", LEAVES + PAIRS, ids=[str(s) for s in LEAVES + PAIRS])
def test_exhaustive_sweep(spec):
    torch.cuda.set_device(0)
    uses_doc = W.mask_uses_doc(spec)
    for bq, bk in ((64, 64), (128, 128), (64, 128), (128, 64)):
        Bm = min(bq, bk)
        lengths = sorted({1, 3, Bm - 1, Bm, Bm + 1, 2 * Bm + 3, 5 * 128 + 17})
        for L in lengths:
            for q_len, kv_len, q_off in ((L, L, 0), (max(1, L // 2), L, L - max(1, L // 2)),
                                         (L, L + 70, 5)):
                kinds = ("packed", "nonmono") if uses_doc else (None,)
                for kind in kinds:
                    doc = None
                    if kind:
                        n = max(q_off + q_len, kv_len)
                        doc = docs_for(n, kind, seed=L)[None]
                    check_tables(spec, 1, 1, q_len, kv_len, bq, bk, q_off, doc)


def test_broadcast_extents_and_per_batch_docs():
    rng = np.random.default_rng(3)
    q_len = kv_len = 700
    doc = np.stack([docs_for(kv_len, "packed", 1), docs_for(kv_len, "nonmono", 2)])
    for spec in (("and", ("doc",), ("causal",)), ("or", ("doc",), ("swa", 100))):
        check_tables(spec, 2, 3, q_len, kv_len, 128, 64, 0, doc)
    check_tables(("swa", 300), 1, 4, q_len, kv_len, 64, 128)
    check_tables(("causal",), 3, 1, q_len, kv_len, 128, 128)
    del rng


def test_positions_beyond_the_32_bit_fast_path():
    """Query positions at and above 2^30 take the one-workgroup builder's 64-bit
    classification (the 32-bit form covers positions below 2^30); the tables stay exact
    on both sides of that bound and near 2^31."""
    for q_off in ((1 << 30) - 400, (1 << 30) - 100, 1 << 30, (1 << 31) - 600):
        for spec in (("causal",), ("swa", 300), ("prefix", 700), ("swa", 1 << 30),
                     ("and", ("swa", (1 << 30) + 200), ("prefix", 500))):
            check_tables(spec, 1, 1, 300, 1000, 128, 128, q_off)


def test_deterministic_repeat():
    doc = docs_for(3000, "nonmono", 9)[None]
    spec = ("or", ("and", ("doc",), ("swa", 300)), ("prefix", 64))
    _, a = gpu_tables(spec, 1, 2, 3000, 3000, 128, 128, 0, doc)
    for _ in range(3):
        _, b = gpu_tables(spec, 1, 2, 3000, 3000, 128, 128, 0, doc)
        assert_tables_equal(b, a, "repeat")


def _grid_rows(got, nqb):
    """Per query block: (full list, partial list) of the kv side."""
    return [(list(got["full_kv_idx"][got["full_kv_ptr"][r]:got["full_kv_ptr"][r + 1]]),
             list(got["kv_idx"][got["kv_ptr"][r]:got["kv_ptr"][r + 1]])) for r in range(nqb)]


def _golden_row(line):
    return ([c for c, ch in enumerate(line) if ch == "F"], [c for c, ch in enumerate(line) if ch == "P"])


def test_worked_example_n8_w4_2x2(golden):
    """The teaching example at its own size ("FlexAttention: from rules to fused
    kernels", section 2.2, Fig. 1): length 8, window 4, 2 x 2 blocks, built by the GPU
    builder through the C ABI; bit-exact against the oracle and the fixture's grid."""
    kv, _ = golden("worked_n8_w4_2x2.txt")
    got = check_tables(("swa", kv["W"]), 1, 1, kv["q_len"], kv["kv_len"], kv["block_q"], kv["block_kv"])
    nqb = kv["q_len"] // kv["block_q"]
    assert _grid_rows(got, nqb) == [_golden_row(line) for line in kv["grid"]]
    executed = int(got["kv_ptr"][-1] + got["full_kv_ptr"][-1])
    assert executed == kv["executed_blocks"]
    assert nqb * (kv["kv_len"] // kv["block_kv"]) - executed == kv["empty_blocks"]
    # executed elements: every pair of the executed blocks
    assert executed * kv["block_q"] * kv["block_kv"] == kv["covered_elements"]


def test_worked_example_n16_w8_4x4_last_row(golden):
    """The N=16, W=8, 4 x 4 BlockMask example ("FlexAttention: compiler optimization of
    custom attention", section 4) at its own size: the last query block's row."""
    kv, _ = golden("worked_n16_w8_4x4_lastrow.txt")
    got = check_tables(("swa", kv["W"]), 1, 1, kv["q_len"], kv["kv_len"], kv["block_q"], kv["block_kv"])
    nqb = kv["q_len"] // kv["block_q"]
    assert _grid_rows(got, nqb)[-1] == _golden_row(kv["last_row"])


def test_worked_example_scaled_grid():
    # the same grid with every length and block x 64: the forward's block sizes
    got = check_tables(("swa", 4 * 64), 1, 1, 8 * 64, 8 * 64, 128, 128)
    assert _grid_rows(got, 4) == [([], [0]), ([0], [1]), ([1], [0, 2]), ([2], [1, 3])]


SMALL_BLOCKS = ((2, 2), (4, 4), (8, 8), (16, 16), (2, 8), (16, 4))


@pytest.mark.parametrize("spec", LEAVES + PAIRS, ids=[str(s) for s in LEAVES + PAIRS])
def test_exhaustive_sweep_small_blocks(spec):
    """Table writers accept power-of-two blocks below 64 (the pages' worked examples use
    2 x 2 and 4 x 4): the same sweep of rules, lengths, offsets and documents."""
    torch.cuda.set_device(0)
    uses_doc = W.mask_uses_doc(spec)
    for bq, bk in SMALL_BLOCKS:
        Bm = min(bq, bk)
        for L in sorted({1, 3, Bm - 1 if Bm > 1 else 2, Bm, Bm + 1, 2 * Bm + 3, 97, 257}):
            for q_len, kv_len, q_off in ((L, L, 0), (max(1, L // 2), L, L - max(1, L // 2)),
                                         (L, L + 70, 5)):
                for kind in (("packed", "nonmono") if uses_doc else (None,)):
                    doc = None
                    if kind:
                        doc = docs_for(max(q_off + q_len, kv_len), kind, seed=L)[None]
                    check_tables(spec, 1, 1, q_len, kv_len, bq, bk, q_off, doc)


@pytest.mark.parametrize("name", [n for n in W.WORKLOADS if W.WORKLOADS[n].selector])
def test_selector_workload_tables(name):
    """Full-size selector workloads: every row of three heads against the oracle's
    per-row lists, the work order of those heads, and the totals in closed form (under
    the causal rule with equal block sizes each row keeps its diagonal block PARTIAL and
    its other chosen blocks FULL; under a rule allowing every pair all are FULL)."""
    from oracle import selector as OS
    from tests.helpers import workload_block_mask
    w = W.WORKLOADS[name]
    bm = workload_block_mask(w, order=True)
    torch.cuda.synchronize()
    got = bm.compact()
    nqb, nkb = -(-w.q_len // w.block_q), -(-w.kv_len // w.block_kv)
    sets = OS.canonical_sets(W.selector_indices(w), nkb)
    if w.q_len == w.kv_len:
        n_part = w.B * w.Hq * nqb if w.mask == ("causal",) else 0
        assert w.mask == ("causal",) or w.mask == ("prefix", w.kv_len)
    else:
        n_part = 0   # decode: the one row sees every key up to its own, all chosen blocks FULL
        assert w.q_len == 1 and w.q_offset == w.kv_len - 1 and w.mask == ("causal",)
    assert int(got["kv_ptr"][-1]) == n_part
    assert int(got["full_kv_ptr"][-1]) == sum(len(x) for x in sets) - n_part
    for h in (0, w.Hq // 2, w.Hq - 1):
        for r in range(nqb):
            row = h * nqb + r
            p, f = OS.row_lists(w.mask, sets, w.Hq, 0, h, r, w.q_len, w.kv_len, w.block_q, w.block_kv, w.q_offset)
            assert np.array_equal(got["kv_idx"][got["kv_ptr"][row]:got["kv_ptr"][row + 1]], p), (h, r)
            assert np.array_equal(got["full_kv_idx"][got["full_kv_ptr"][row]:got["full_kv_ptr"][row + 1]], f), (h, r)
        part = {k: got[k][h * nqb:(h + 1) * nqb] for k in ("kv_num", "full_kv_num")}
        assert np.array_equal(got["order"][h * nqb:(h + 1) * nqb], OS.work_order(part, 1, 1, w.q_len, w.block_q))


@pytest.mark.parametrize("case", ["causal_softcap", "gqa_doc_swa_alibi", "prefix_relpos_64k", "groups"])
def test_rule_tables_work_order(case):
    """The longest-first work order of rule tables: ranked in place by the one-workgroup
    builder for groups of up to 256 rows (several batch and head groups included), by
    its own kernel for longer groups (512 rows), against the oracle's ranking of the
    tables' own row lengths (ties by descending index)."""
    import block_sparse_programmable_amd as fa
    from oracle import selector as OS
    if case == "groups":
        rng = np.random.default_rng(41)
        doc = np.stack([np.repeat(np.arange(40), rng.integers(20, 200, 40))[:1500] for _ in range(2)]).astype(np.int32)
        spec, B, H, q_len, kv_len, bq, bk, off = ("or", ("and", ("doc",), ("swa", 300)), ("prefix", 64)), 2, 3, 1500, 1500, 64, 64, 0
    else:
        w = W.WORKLOADS[case]
        doc = W.aux_inputs(w)["doc_ids"]
        spec, B, H, q_len, kv_len, bq, bk, off = w.mask, 1, 1, w.q_len, w.kv_len, w.block_q, w.block_kv, w.q_offset
    docT = None if doc is None else torch.as_tensor(np.asarray(doc, np.int32)).cuda()
    bm = fa.create_block_mask(spec, B, H, q_len, kv_len, bq, bk, off, docT, order=True)
    torch.cuda.synchronize()
    got = bm.compact()
    want = OS.work_order({k: np.asarray(got[k]) for k in ("kv_num", "full_kv_num")}, B, H, q_len, bq)
    assert np.array_equal(np.asarray(got["order"]), want)


@pytest.mark.parametrize("name", ["gqa_doc_swa_alibi", "prefix_relpos_64k"])
def test_kv_side_only_tables(name):
    """Tables built without the query side (the one-workgroup builder, and the
    multi-launch builder for the 512 x 512 grid) equal the kv side and the work order of
    tables built with it."""
    import block_sparse_programmable_amd as fa
    w = W.WORKLOADS[name]
    doc = W.aux_inputs(w)["doc_ids"]
    docT = None if doc is None else torch.as_tensor(np.asarray(doc, np.int32)).cuda()
    args = (w.mask, 1, 1, w.q_len, w.kv_len, w.block_q, w.block_kv, w.q_offset, docT)
    both = fa.create_block_mask(*args, order=True).compact()
    kv = fa.create_block_mask(*args, order=True, q_side=False)
    torch.cuda.synchronize()
    assert "q_num" not in kv.tensors
    got = kv.compact()
    for k in ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx", "order"):
        assert np.array_equal(np.asarray(got[k]), np.asarray(both[k])), k


@pytest.mark.parametrize("name", [n for n in W.WORKLOADS if not W.WORKLOADS[n].selector])
def test_workload_tables(name):
    w = W.WORKLOADS[name]
    aux = W.aux_inputs(w)
    tB = 1
    got = check_tables(w.mask, tB, 1, w.q_len, w.kv_len, w.block_q, w.block_kv, w.q_offset, aux["doc_ids"])
    nf = int(got["full_kv_ptr"][-1])
    npart = int(got["kv_ptr"][-1])
    expected = {"tiny_swa": (7, 14), "causal_softcap": (496, 32), "gqa_doc_swa_alibi": (175, 160),
                "prefix_relpos_64k": (131344, 480), "decode_swa_softcap": (32, 0),
                "decode_paged_swa_softcap": (32, 0)}[name]
    assert (nf, npart) == expected


@pytest.mark.parametrize("spec", [("and", ("doc",), ("swa", 700)), ("or", ("doc",), ("prefix", 300)),
                                  ("causal",), ("and", ("prefix", 1000), ("doc",))],
                         ids=["doc&swa", "doc|prefix", "causal", "prefix&doc"])
def test_large_grid_multi_launch_path(spec):
    # more than 16384 blocks: the five-launch build path (the small grids above use the
    # single-workgroup path); per-batch documents, replicated heads, ragged tail
    n = 64 * 130 + 17
    doc = np.stack([docs_for(n, "packed", 11), docs_for(n, "nonmono", 12)])
    if W.mask_uses_doc(spec):
        check_tables(spec, 2, 2, n, n, 64, 64, 0, doc)
    else:
        check_tables(spec, 1, 3, n, n, 64, 64, 0, None)


def test_empty_sides_are_written():
    """q_len = 0 (or kv_len = 0): every count and pointer is still written (zeros), on
    both the one-launch and the multi-launch builder paths."""
    import block_sparse_programmable_amd as fa
    from block_sparse_programmable_amd.api import TABLE_NAMES
    for B, H, q_len, kv_len in ((1, 2, 0, 300), (2, 1, 300, 0), (1, 1, 0, 0), (1, 1, 0, 64 * 3000)):
        n_rows = B * H * -(-q_len // 64)
        n_cols = B * H * -(-kv_len // 64)
        tables = {}
        for side, n in (("kv", n_rows), ("full_kv", n_rows), ("q", n_cols), ("full_q", n_cols)):
            tables[f"{side}_num"] = torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
            tables[f"{side}_ptr"] = torch.full((n + 1,), -7, dtype=torch.int32, device="cuda")
            tables[f"{side}_idx"] = torch.full((1,), -7, dtype=torch.int32, device="cuda")
        assert set(tables) == set(TABLE_NAMES)
        fa.create_block_mask(("causal",), B, H, q_len, kv_len, 64, 64, 0, tables=tables)
        torch.cuda.synchronize()
        for side, n in (("kv", n_rows), ("full_kv", n_rows), ("q", n_cols), ("full_q", n_cols)):
            assert (tables[f"{side}_num"][:n] == 0).all(), (B, H, q_len, kv_len, side)
            assert (tables[f"{side}_ptr"] == 0).all(), (B, H, q_len, kv_len, side)
