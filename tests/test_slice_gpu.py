"""Row slices of prebuilt block tables (fa_block_mask_slice) on the GPU, via the C ABI.

"FlexAttention: from rules to fused kernels", section 5.2: tables built once for the
longest context; each decode step takes the query block of its position, the rule still
seeing global positions.  Section 2.2: a crop is reused only for rules whose rebuilt
tables, for several target lengths, equal the crop in block indices and in element
adjacency (the whitelist test below).

Bars: the sliced tables equal, bit for bit, the oracle's tables built directly for the
new geometry (a slice re-decides only blocks whose rows or keys were cut, so it must
reach the same exact classification), and list no block the prebuilt tables leave out;
the forward over sliced tables meets the forward bars against the float64 oracle."""
import numpy as np
import pytest
import torch

from oracle import blockmask as OB
from oracle import masks as OM
from tests.helpers import assert_tables_equal, compare, oracle_forward, randn_bf16

pytestmark = pytest.mark.gpu

MENU = [("causal",), ("swa", 100), ("prefix", 70), ("and", ("causal",), ("swa", 300)),
        ("or", ("swa", 60), ("prefix", 130)), ("and", ("doc",), ("causal",)),
        ("and", ("doc",), ("swa", 200))]


def packed_docs(n, B, seed):
    rng = np.random.default_rng(seed)
    rows = []
    for _ in range(B):
        lens = []
        while sum(lens) < n:
            lens.append(int(rng.integers(30, 400)))
        rows.append(np.repeat(np.arange(len(lens)), lens)[:n])
    return np.stack(rows).astype(np.int32)


def prebuilt(spec, B, H, L, bq, bk, doc):
    import block_sparse_programmable_amd as fa
    uses_doc = "doc" in str(spec)
    docT = torch.as_tensor(doc).cuda() if uses_doc else None
    bm = fa.create_block_mask(spec, B if uses_doc else 1, H, L, L, bq, bk, 0, docT)
    want = OB.tables(spec, B if uses_doc else 1, H, L, L, bq, bk, 0, doc if uses_doc else None)
    return bm, want, (B if uses_doc else 1), docT


def sliced(bm, q_len, kv_len, q_offset, q_side=True):
    import block_sparse_programmable_amd as fa
    s = fa.slice_block_mask(bm, q_len, kv_len, q_offset, q_side=q_side)
    torch.cuda.synchronize()
    return s, s.compact()


def check_slice(bm, src, spec, tB, H, L_src, bq, bk, q_len, kv_len, q_off, doc, src_off=0, kv_src=None):
    """GPU slice == oracle tables at the new geometry; both sides and the kv-only form;
    tightened from the conservative slice of the prebuilt tables (never more blocks)."""
    ctx = f"{spec} slice q={q_len} kv={kv_len} off={q_off}"
    kv_src = L_src if kv_src is None else kv_src
    want = OB.tables(spec, tB, H, q_len, kv_len, bq, bk, q_off, doc if "doc" in str(spec) else None)
    _, got = sliced(bm, q_len, kv_len, q_off)
    assert_tables_equal(got, want, ctx)
    _, got_kv = sliced(bm, q_len, kv_len, q_off, q_side=False)
    assert_kv_equal(got_kv, want, ctx + " kv side only")
    loose = OB.slice_rows(src, tB, H, L_src, kv_src, bq, bk, src_off, q_len, kv_len, q_off)
    rows = tB * H * OB.n_blocks(q_len, bq)
    for r in range(rows):
        lst = lambda t, key: set(t[f"{key}_idx"][t[f"{key}_ptr"][r]:t[f"{key}_ptr"][r + 1]].tolist())
        assert lst(want, "kv") | lst(want, "full_kv") <= lst(loose, "kv") | lst(loose, "full_kv"), ctx
        assert lst(loose, "full_kv") <= lst(want, "full_kv"), ctx


def assert_kv_equal(got, want, ctx):
    for side in ("kv", "full_kv"):
        for part in ("num", "ptr", "idx"):
            k = f"{side}_{part}"
            assert np.array_equal(got[k], want[k]), f"{ctx}: {k} differs"


@pytest.mark.parametrize("spec", MENU, ids=[str(s) for s in MENU])
def test_slices_match_oracle(spec):
    """Decode rows (one and three positions, at block edges and inside), aligned crops,
    an offset multi-block slice and empty slices, both sides, one-launch path."""
    L, bq, bk = 1000, 64, 128
    doc = packed_docs(L, 2, seed=3)
    bm, src, tB, _ = prebuilt(spec, 2, 3, L, bq, bk, doc)
    cases = [(1, t + 1, t) for t in (0, 63, 64, 127, 128, 500, 999)]
    cases += [(3, t + 3, t) for t in (0, 61, 64, 900)]
    cases += [(1, 1000, 640), (5, 700, 130)]                 # keys past the position
    cases += [(512, 512, 0), (1000, 1000, 0), (448, 1000, 0), (300, 700, 128), (64, 1000, 896), (40, 1000, 960)]
    cases += [(0, 300, 128), (2, 0, 64), (0, 0, 1000)]
    for q_len, kv_len, q_off in cases:
        check_slice(bm, src, spec, tB, 3, L, bq, bk, q_len, kv_len, q_off, doc)
    # rejected on both sides: straddling rows, unaligned multi-block rows, past the end
    import block_sparse_programmable_amd as fa
    for q_len, kv_len, q_off in ((2, 100, 63), (100, 1000, 32), (1, 1001, 999), (2, 1000, 999)):
        with pytest.raises(ValueError):
            OB.slice_rows(src, tB, 3, L, L, bq, bk, 0, q_len, kv_len, q_off)
        with pytest.raises(fa.FAError):
            fa.slice_block_mask(bm, q_len, kv_len, q_off)


@pytest.mark.parametrize("spec", [("causal",), ("and", ("doc",), ("swa", 500)), ("or", ("swa", 60), ("prefix", 130))],
                         ids=str)
def test_large_slices_match_oracle(spec):
    """More than 16384 new blocks or 4096 new lines: the three-launch path."""
    L, bq, bk = 4096, 64, 64
    doc = packed_docs(L, 2, seed=4)
    bm, src, tB, _ = prebuilt(spec, 2, 16, L, bq, bk, doc)
    for q_len, kv_len, q_off in ((3000, 3000, 0), (2000, 3500, 640), (1, 4096, 4095), (4096, 4096, 0),
                                 (3, 3001, 2998)):
        check_slice(bm, src, spec, tB, 16, L, bq, bk, q_len, kv_len, q_off, doc)


def test_slice_of_offset_tables():
    """Tables prebuilt for rows [256, 2304): slices keep global positions."""
    import block_sparse_programmable_amd as fa
    spec, bq, bk, off0 = ("swa", 333), 128, 64, 256
    bm = fa.create_block_mask(spec, 1, 2, 2048, 2304, bq, bk, off0)
    src = OB.tables(spec, 1, 2, 2048, 2304, bq, bk, off0)
    for q_len, kv_len, q_off in ((1, 1001, 1000), (128, 1500, 1280), (700, 2304, 1024), (2, 2304, 2302)):
        check_slice(bm, src, spec, 1, 2, 2048, bq, bk, q_len, kv_len, q_off, None, src_off=off0, kv_src=2304)


def test_crop_whitelist():
    """Section 2.2's procedure on the GPU: for each rule of the menu, crop tables prebuilt
    at L_max to several target lengths and compare with tables rebuilt at that length,
    in block indices and in element adjacency (partial blocks under the exact rule).  Every rule of the menu reads global positions only, so
    every one must pass; the CPU pins show the same check rejecting a rule that reads the
    total length."""
    import block_sparse_programmable_amd as fa
    Lmax, bq, bk = 2048, 128, 128
    doc = packed_docs(Lmax, 1, seed=5)
    whitelist = []
    for spec in MENU:
        bm, _, tB, docT = prebuilt(spec, 1, 1, Lmax, bq, bk, doc)
        ok = True
        for L in (256, 1024, 1536, 2048, 300, 1000, 1999):
            _, crop = sliced(bm, L, L, 0)
            re_bm = fa.create_block_mask(spec, tB, 1, L, L, bq, bk, 0, docT)
            torch.cuda.synchronize()
            rebuilt = re_bm.compact()
            ok &= all(np.array_equal(crop[k], rebuilt[k]) for k in rebuilt)
            d = doc[:, :L] if tB == 1 and "doc" in str(spec) else None
            dr = OM.doc_row_for(d, 0) if d is not None else None
            M = OM.dense(spec, L, L, 0, dr)
            ok &= np.array_equal(OB.expand(crop, 1, 1, L, L, bq, bk, spec, 0, d), M)
            ok &= np.array_equal(OB.expand(rebuilt, 1, 1, L, L, bq, bk, spec, 0, d), M)
        if ok:
            whitelist.append(spec)
    assert whitelist == MENU


def decode_inputs(B, Hq, Hkv, L, d, seed):
    q = randn_bf16((B, Hq, L, d), seed).cuda()
    k = randn_bf16((B, Hkv, L, d), seed + 1).cuda()
    v = randn_bf16((B, Hkv, L, d), seed + 2).cuda()
    return q, k, v


@pytest.mark.parametrize("spec", [("causal",), ("swa", 700), ("and", ("doc",), ("causal",)),
                                  ("or", ("swa", 200), ("prefix", 300))], ids=str)
def test_decode_forward_over_sliced_tables(spec):
    """Token-by-token decode: one prebuilt L_max table, sliced per step; the forward over
    the slice (split-KV decode path, GQA) against the oracle at the step's geometry."""
    import block_sparse_programmable_amd as fa
    B, Hq, Hkv, d, Lmax, bq, bk = 2, 8, 1, 128, 3000, 128, 128
    doc = packed_docs(Lmax, B, seed=6)
    bm, _, tB, docT = prebuilt(spec, B, 1, Lmax, bq, bk, doc)
    q_all, k_all, v_all = decode_inputs(B, Hq, Hkv, Lmax, d, seed=31)
    for t in (0, 127, 128, 1000, 2047, 2999):
        s, _ = sliced(bm, 1, t + 1, t, q_side=False)
        q = q_all[:, :, t:t + 1].contiguous()
        k = k_all[:, :, :t + 1].contiguous()
        v = v_all[:, :, :t + 1].contiguous()
        o, lse = fa.forward(q, k, v, s, score="softcap", softcap=30.0)
        # the slice equals the rebuilt tables, so the forward is the same, bit for bit
        rb = fa.create_block_mask(spec, tB, 1, 1, t + 1, bq, bk, t, docT)
        o2, lse2 = fa.forward(q, k, v, rb, score="softcap", softcap=30.0)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, lse2), f"{spec} t={t}: slice and rebuild differ"
        O, Lo = oracle_forward(q, k, v, spec, "softcap", t, doc if tB > 1 else None, cap=30.0)
        compare(o, lse, O, Lo, f"{spec} decode t={t} over sliced tables")


def test_slice_writes_the_work_order():
    """A slice asked for the work order writes the order of its own (new) rows."""
    import block_sparse_programmable_amd as fa
    from oracle import selector as OS
    L, bq, bk = 1500, 64, 64
    bm = fa.create_block_mask(("swa", 400), 1, 2, L, L, bq, bk)
    for q_len, kv_len, q_off in ((1000, 1000, 0), (320, 1400, 640), (1, 1200, 1199)):
        s = fa.slice_block_mask(bm, q_len, kv_len, q_off, order=True)
        torch.cuda.synchronize()
        got = s.compact()
        want = OB.tables(("swa", 400), 1, 2, q_len, kv_len, bq, bk, q_off)
        assert_tables_equal(got, want, f"slice order q={q_len}")
        assert np.array_equal(got["order"], OS.work_order(want, 1, 2, q_len, bq)), (q_len, kv_len, q_off)
