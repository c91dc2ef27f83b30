"""GPU forward (prefill and split-KV decode) vs the float64 oracle, via the C ABI.

Bars: O max-abs <= 2e-2, LSE max-abs <= 1e-3 on finite rows, and identical empty-row
patterns (O = 0, LSE = -inf)."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from tests.helpers import compare, oracle_forward, randn_bf16, run_forward, workload_block_mask, workload_oracle_mask

pytestmark = pytest.mark.gpu


def qkv(B, Hq, Hkv, q_len, kv_len, d, seed, qscale=1.0):
    q = randn_bf16((B, Hq, q_len, d), seed, qscale).cuda()
    k = randn_bf16((B, Hkv, kv_len, d), seed + 1).cuda()
    v = randn_bf16((B, Hkv, kv_len, d), seed + 2).cuda()
    return q, k, v


def score_kw(kind, Hq, seed=0):
    rng = np.random.default_rng(seed)
    if kind == "alibi":
        return dict(slopes=np.exp2(-8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32))
    if kind == "softcap":
        return dict(cap=20.0)
    if kind == "relpos":
        R = 40
        return dict(table=(rng.standard_normal((Hq, 2 * R + 1)) * 0.5).astype(np.float32), radius=R)
    return {}


def check(q, k, v, mask, bq, bk, score="identity", q_offset=0, doc=None, tB=1, tH=1, scale=None,
          ctx="", **skw):
    o, lse = run_forward(q, k, v, mask, bq, bk, score, q_offset, doc, tB, tH, scale=scale,
                         cap=skw.get("cap", 0.0), slopes=skw.get("slopes"), table=skw.get("table"),
                         radius=skw.get("radius", 0))
    O, L = oracle_forward(q, k, v, mask, score, q_offset, doc, cap=skw.get("cap"),
                          slopes=skw.get("slopes"), table=skw.get("table"), radius=skw.get("radius"),
                          scale=scale)
    return compare(o, lse, O, L, ctx)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("score", ["identity", "alibi", "softcap", "relpos"])
def test_small_shapes_all_scores(d, score):
    for (bq, bk) in ((128, 128), (64, 64), (64, 128), (128, 64)):
        for (Hq, Hkv) in ((4, 4), (4, 2), (4, 1)):       # MHA, GQA, MQA
            q, k, v = qkv(1, Hq, Hkv, 300, 300, d, seed=d + bq + bk + Hkv)
            for mask in (("causal",), ("swa", 70), ("prefix", 45)):
                check(q, k, v, mask, bq, bk, score, ctx=f"d{d} {bq}x{bk} {Hq}/{Hkv} {mask} {score}",
                      **score_kw(score, Hq))


@pytest.mark.parametrize("score", ["identity", "alibi", "softcap", "relpos"])
def test_doc_and_compositions(score):
    rng = np.random.default_rng(5)
    n = 777
    lens = []
    while sum(lens) < n:
        lens.append(int(rng.integers(20, 250)))
    doc = np.repeat(np.arange(len(lens)), lens)[:n].astype(np.int32)[None]
    q, k, v = qkv(2, 8, 2, n, n, 128, seed=11)
    for mask in (("and", ("doc",), ("swa", 100)), ("and", ("doc",), ("causal",)),
                 ("or", ("swa", 64), ("prefix", 130)), ("and", ("prefix", 200), ("doc",))):
        check(q, k, v, mask, 128, 128, score, doc=doc, ctx=f"{mask} {score}", **score_kw(score, 8))


def _chain(leaves, ops, right):
    """Eight-leaf and/or chain: left-deep (((a b) c) d)... or right-deep a (b (c (d ...)))."""
    t = leaves[-1] if right else leaves[0]
    rest = leaves[-2::-1] if right else leaves[1:]
    for leaf, op in zip(rest, ops):
        t = (op, leaf, t) if right else (op, t, leaf)
    return t


@pytest.mark.parametrize("score", ["identity", "softcap"])
def test_eight_leaf_programs(score):
    """Sixteen-node-limit programs mixing every leaf with and/or: the kernels evaluate
    them with a four-value stack after the host reorders operands, which the
    right-deep chain needs (it would reach depth eight in the order written)."""
    rng = np.random.default_rng(8)
    n = 530
    lens = []
    while sum(lens) < n:
        lens.append(int(rng.integers(15, 160)))
    doc = np.repeat(np.arange(len(lens)), lens)[:n].astype(np.int32)[None]
    q, k, v = qkv(1, 4, 2, n, n, 128, seed=18)
    leaves = [("doc",), ("swa", 90), ("prefix", 40), ("causal",), ("swa", 300), ("doc",),
              ("prefix", 333), ("swa", 17)]
    ops = ["or", "and", "or", "and", "or", "and", "or"]
    for right in (False, True):
        mask = _chain(leaves, ops, right)
        check(q, k, v, mask, 128, 128, score, doc=doc, ctx=f"chain right={right} {score}",
              **score_kw(score, 4))
    bal = ("or", ("and", ("or", ("doc",), ("swa", 50)), ("or", ("prefix", 64), ("causal",))),
           ("and", ("or", ("swa", 200), ("doc",)), ("or", ("prefix", 7), ("swa", 400))))
    check(q, k, v, bal, 64, 128, score, doc=doc, ctx=f"balanced {score}", **score_kw(score, 4))


@pytest.mark.parametrize("R", [1536, 1537, 2500])
def test_relpos_large_radius(R):
    """Position tables around and beyond the size staged whole in LDS (2R + 1 <= 3073
    entries): larger tables travel as per-tile windows.  Lengths past R on both sides
    (a bidirectional prefix) reach both saturated ends; the decode path reads the same
    table."""
    rng = np.random.default_rng(R)
    n = 3300
    table = (rng.standard_normal((2, 2 * R + 1)) * 0.5).astype(np.float32)
    q, k, v = qkv(1, 2, 1, n, n, 64, seed=19)
    check(q, k, v, ("prefix", 2100), 128, 128, "relpos", table=table, radius=R, ctx=f"prefix R={R}")
    check(q, k, v, ("causal",), 64, 128, "relpos", table=table, radius=R, ctx=f"causal R={R}")
    qd = q[:, :, -3:].contiguous()
    check(qd, k, v, ("prefix", 2100), 128, 128, "relpos", q_offset=n - 3, table=table, radius=R,
          ctx=f"decode R={R}")


def test_nonmonotone_docs_per_batch():
    rng = np.random.default_rng(6)
    n = 400
    doc = np.stack([rng.integers(0, 4, n), rng.integers(0, 2, n)]).astype(np.int32)
    q, k, v = qkv(2, 4, 4, n, n, 128, seed=12)
    check(q, k, v, ("and", ("doc",), ("causal",)), 64, 128, "identity", doc=doc, tB=2,
          ctx="per-batch docs")


def test_ragged_and_offsets_and_empty_rows():
    # q shorter than kv with an offset, kv tail inside a block, rows with no key
    q, k, v = qkv(1, 2, 2, 77, 333, 128, seed=13)
    check(q, k, v, ("causal",), 128, 128, q_offset=256, ctx="offset causal")
    check(q, k, v, ("swa", 50), 64, 128, q_offset=300, ctx="window beyond kv: empty rows")
    q, k, v = qkv(1, 2, 2, 200, 130, 64, seed=14)
    check(q, k, v, ("causal",), 128, 128, ctx="q longer than kv")
    check(q, k, v, ("prefix", 3), 64, 64, ctx="prefix 3")
    q, k, v = qkv(1, 2, 2, 1, 1, 128, seed=15)
    check(q, k, v, ("causal",), 128, 128, ctx="single element")


def test_large_scores_and_single_key_rows():
    q, k, v = qkv(1, 2, 1, 256, 256, 128, seed=16, qscale=6.0)
    check(q, k, v, ("causal",), 128, 128, ctx="large scores")
    check(q, k, v, ("causal",), 128, 128, "softcap", cap=5.0, ctx="large scores softcap")
    check(q, k, v, ("swa", 1), 64, 64, ctx="single-key rows")


@pytest.mark.parametrize("cap", [0.5, 5.0, 34.0, 35.0, 200.0])
def test_softcap_reference_both_sides_of_the_fixed_bound(cap):
    """Soft-cap kernels fix the softmax reference at cap * log2(e) for caps up to 34.6
    (every weight then lies in [2^(-2 cap log2 e), 1]) and keep a running maximum above;
    both sides, a tiny cap and a cap far above the scores, on causal and window masks
    with large scores, all blocks partial and full."""
    q, k, v = qkv(1, 4, 2, 384, 384, 128, seed=31, qscale=4.0)
    for mask in (("causal",), ("swa", 100)):
        for bq, bk in ((128, 128), (64, 64)):
            check(q, k, v, mask, bq, bk, "softcap", cap=cap, ctx=f"softcap {cap} {mask} {bq}x{bk}")


def test_explicit_scale():
    q, k, v = qkv(1, 2, 2, 200, 200, 64, seed=17)
    check(q, k, v, ("causal",), 64, 64, scale=0.3, ctx="scale 0.3")


def test_three_way_degradation():
    """Normal tables vs the same rule with every listed block forced to partial
    (mask evaluated everywhere) vs every block listed as partial (dense)."""
    import block_sparse_programmable_amd as fa
    rng = np.random.default_rng(7)
    n = 640
    doc = np.repeat(np.arange(6), [100, 90, 150, 120, 80, 100]).astype(np.int32)[None]
    q, k, v = qkv(1, 4, 2, n, n, 128, seed=18)
    mask = ("and", ("doc",), ("swa", 200))
    base = run_forward(q, k, v, mask, 128, 128, "alibi", doc=doc, slopes=score_kw("alibi", 4)["slopes"])

    def all_partial(bm):
        t = bm.compact()
        nqb = len(t["kv_num"])
        num, idx = [], []
        for r in range(nqb):
            cols = sorted(list(t["kv_idx"][t["kv_ptr"][r]:t["kv_ptr"][r + 1]]) +
                          list(t["full_kv_idx"][t["full_kv_ptr"][r]:t["full_kv_ptr"][r + 1]]))
            num.append(len(cols))
            idx += cols
        _write(bm, num, idx)

    def dense(bm):
        nqb = len(bm.compact()["kv_num"])
        nkb = (n + 127) // 128
        _write(bm, [nkb] * nqb, list(range(nkb)) * nqb)

    def _write(bm, num, idx):
        num = np.asarray(num, np.int32)
        ptr = np.concatenate([[0], np.cumsum(num)]).astype(np.int32)
        bm.tensors["kv_num"][: len(num)] = torch.from_numpy(num).cuda()
        bm.tensors["kv_ptr"][: len(ptr)] = torch.from_numpy(ptr).cuda()
        bm.tensors["kv_idx"][: len(idx)] = torch.as_tensor(np.asarray(idx, np.int32)).cuda()
        bm.tensors["full_kv_num"].zero_()
        bm.tensors["full_kv_ptr"].zero_()

    sl = score_kw("alibi", 4)["slopes"]
    forced = run_forward(q, k, v, mask, 128, 128, "alibi", doc=doc, slopes=sl, tables=all_partial)
    dense_r = run_forward(q, k, v, mask, 128, 128, "alibi", doc=doc, slopes=sl, tables=dense)
    O, L = oracle_forward(q, k, v, mask, "alibi", doc=doc, slopes=sl)
    for name, (o, lse) in (("normal", base), ("forced partial", forced), ("dense", dense_r)):
        compare(o, lse, O, L, name)
    # the three lowerings agree with each other more tightly than with the oracle
    assert float((base[0].float() - forced[0].float()).abs().max()) <= 1e-2
    assert float((base[1] - dense_r[1]).abs().max()) <= 1e-4
    del rng


def test_gqa_matches_expanded_kv():
    q, k, v = qkv(1, 8, 2, 256, 256, 128, seed=19)
    sl = score_kw("alibi", 8)["slopes"]
    o1, l1 = run_forward(q, k, v, ("causal",), 128, 128, "alibi", slopes=sl)
    ke = k.repeat_interleave(4, dim=1).contiguous()
    ve = v.repeat_interleave(4, dim=1).contiguous()
    o2, l2 = run_forward(q, ke, ve, ("causal",), 128, 128, "alibi", slopes=sl)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("score", ["identity", "softcap", "alibi", "relpos"])
def test_decode_shapes(score):
    # single query (and a few) against long KV through the split-KV path
    # (g * q_len columns: up to 16 take the split-KV kernel, 32 the prefill kernel)
    for (B, Hq, Hkv, q_len, kv_len, mask, d) in (
            (3, 8, 2, 1, 2000, ("swa", 700), 128),
            (2, 4, 4, 1, 1024, ("causal",), 128),
            (2, 8, 1, 4, 900, ("causal",), 128),
            (1, 32, 8, 1, 4096, ("swa", 4096), 128),
            (2, 4, 2, 3, 513, ("prefix", 100), 128),
            (1, 16, 1, 1, 3000, ("swa", 1500), 128),
            (2, 8, 1, 2, 1500, ("causal",), 128),
            (3, 8, 2, 1, 1100, ("swa", 600), 64)):
        q, k, v = qkv(B, Hq, Hkv, q_len, kv_len, d, seed=20 + kv_len)
        check(q, k, v, mask, 128, 128, score, q_offset=kv_len - q_len,
              ctx=f"decode {B}x{Hq}/{Hkv} q{q_len} kv{kv_len} d{d} {mask} {score}", **score_kw(score, Hq))


@pytest.mark.parametrize("B,Hkv,kv_len", [(128, 8, 700), (64, 4, 1100), (16, 2, 1500)],
                         ids=["one_split", "splits_in_workgroup", "split_merge_kernel"])
def test_decode_split_paths(B, Hkv, kv_len):
    # enough (batch, KV head) pairs for one split per unit, splits merged in LDS, and
    # splits merged by the second kernel (on a 256-CU device: 1, 4 and 12 splits)
    Hq = 2 * Hkv
    q, k, v = qkv(B, Hq, Hkv, 1, kv_len, 128, seed=40 + B)
    check(q, k, v, ("swa", 600), 128, 128, "softcap", q_offset=kv_len - 1,
          ctx=f"decode split path B{B} Hkv{Hkv} kv{kv_len}", **score_kw("softcap", Hq))


def test_decode_long_rows():
    # one (batch, KV head) pair over 4200 listed blocks: 64 splits of 65-66 blocks, so a
    # split's block list spans more than one 64-entry register chunk (with the rotated
    # stage order the chunk is reloaded going forward and back)
    kv_len = 128 * 4200
    q, k, v = qkv(1, 2, 1, 1, kv_len, 128, seed=50)
    check(q, k, v, ("causal",), 128, 128, "identity", q_offset=kv_len - 1, ctx="decode long rows")


def test_decode_empty_and_offsets():
    q, k, v = qkv(2, 4, 2, 1, 700, 128, seed=30)
    check(q, k, v, ("swa", 100), 128, 128, q_offset=1000, ctx="decode window past the cache (empty)")
    check(q, k, v, ("swa", 100), 128, 128, q_offset=650, ctx="decode window partly past the cache")
    check(q, k, v, ("causal",), 128, 128, q_offset=0, ctx="decode first position")


def sample_rows(n, block, count, seed):
    rng = np.random.default_rng(seed)
    edges = {0, n - 1, block - 1, block, n // 2}
    picks = set(int(x) for x in rng.integers(0, n, count))
    return np.array(sorted(x for x in edges | picks if 0 <= x < n))


@pytest.mark.parametrize("name", list(W.WORKLOADS))
def test_workload_full_size_sampled(name):
    """Full-size workloads in the launch configuration the bench times; the oracle
    computes a sample of rows (all heads or a head subset) one by one."""
    import block_sparse_programmable_amd as fa
    w = W.WORKLOADS[name]
    aux = W.aux_inputs(w)
    q, k, v = W.qkv(w, device="cuda")
    docT = None if aux["doc_ids"] is None else torch.as_tensor(aux["doc_ids"]).cuda()
    bm = workload_block_mask(w, docT, order=bool(w.selector))
    sl = None if aux["slopes"] is None else torch.as_tensor(aux["slopes"]).cuda()
    tb = None if aux["table"] is None else torch.as_tensor(aux["table"]).cuda()
    if w.page_size:
        # the same logical K/V through the workload's fragmented page table
        pt = W.page_table(w)
        kcache, vcache = W.paged_caches(w, k, v, pt)
        o, lse = fa.forward_paged(q, kcache, vcache, torch.as_tensor(pt).cuda(), w.kv_len, bm,
                                  score=w.score, softcap=w.cap, alibi_slopes=sl, relpos=tb,
                                  relpos_radius=w.relpos_radius)
        torch.cuda.synchronize()
        del kcache, vcache
    else:
        o, lse = fa.forward(q, k, v, bm, score=w.score, softcap=w.cap, alibi_slopes=sl, relpos=tb,
                            relpos_radius=w.relpos_radius)
        torch.cuda.synchronize()
    if w.q_len == 1:
        batches = [0, w.B // 2, w.B - 1]
        heads = list(range(w.Hq))
        rows = np.array([0])
    else:
        batches = list(range(w.B))
        heads = sorted({0, w.Hq // 2, w.Hq - 1})
        rows = sample_rows(w.q_len, w.block_q, 40 if w.q_len > 10000 else 64, seed=w.seed)
    # indices are checked on the host before any device indexing
    assert max(batches) < w.B and max(heads) < w.Hq and int(rows.max()) < w.q_len
    bi = torch.as_tensor(batches)
    hi = torch.as_tensor(heads)
    ri = torch.as_tensor(rows)
    # all indexing happens on host copies; the oracle gets the full K/V of each batch entry
    bid = bi.cuda()
    qc, kc, vc = (t.index_select(0, bid).cpu() for t in (q, k, v))
    O, L = oracle_forward(qc, kc, vc, workload_oracle_mask(w, aux["doc_ids"], batches), w.score, w.q_offset,
                          aux["doc_ids"],
                          cap=w.cap or None, slopes=aux["slopes"], table=aux["table"],
                          radius=w.relpos_radius, rows=rows, heads=heads)
    got_o = o.index_select(0, bid).cpu()[:, hi][:, :, ri]
    got_l = lse.index_select(0, bid).cpu()[:, hi][:, :, ri]
    compare(got_o, got_l, O, L, name)
