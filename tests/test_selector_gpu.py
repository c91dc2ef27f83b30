"""Block tables from selector output (fa_block_mask_from_indices) and the longest-row-
first work order, on the GPU via the C ABI.

"FlexAttention: from rules to fused kernels", sections 5.2 and 6.3: candidate KV blocks
per query block are range-checked, sorted and de-duplicated into each row's list, and
row lengths drive the scheduling of query tiles; "Kernels: turning logical sparsity
into real speed", section 3: repeats must not reach the kernel.

Bars: tables and work orders bit-exact against the oracle; the forward over selector
tables within the forward bars, and the backward within the backward bar, against the
float64 oracle evaluated on the selected-pair matrix; outputs with and without the
work order identical bit for bit."""
import numpy as np
import pytest
import torch

from oracle import backward as OBW
from oracle import blockmask as OB
from oracle import selector as OS
from tests.helpers import assert_tables_equal, compare, oracle_forward, randn_bf16

pytestmark = pytest.mark.gpu

G_TOL = 2e-2


def random_selection(B, H, nqb, nkb, k, seed, extra_bad=True):
    """Candidate lists with repeats, -1 padding and out-of-range values."""
    rng = np.random.default_rng(seed)
    sel = rng.integers(0, max(nkb, 1), size=(B, H, nqb, k))
    if extra_bad and k >= 4:
        sel[..., 0] = -1
        sel[..., 1] = sel[..., 2]                       # a repeat
        bad = rng.random((B, H, nqb)) < 0.3
        sel[..., 3] = np.where(bad, nkb + rng.integers(0, 5, size=(B, H, nqb)), sel[..., 3])
    return sel.astype(np.int32)


def gpu_select(spec, sel, B, H, q_len, kv_len, bq, bk, q_offset=0, doc=None, order=True):
    import block_sparse_programmable_amd as fa
    docT = None if doc is None else torch.as_tensor(np.asarray(doc, np.int32)).cuda()
    bm = fa.block_mask_from_indices(torch.as_tensor(sel).cuda(), spec, B, H, q_len, kv_len, bq, bk, q_offset,
                                    docT, order=order)
    torch.cuda.synchronize()
    return bm, bm.compact()


RULES = [("causal",), ("prefix", 1 << 20), ("swa", 200), ("or", ("swa", 60), ("prefix", 130)),
         ("and", ("doc",), ("causal",))]


@pytest.mark.parametrize("spec", RULES, ids=str)
def test_selector_tables_match_oracle(spec):
    rng = np.random.default_rng(7)
    doc = np.repeat(np.arange(8), rng.integers(60, 200, 8))[:1000].astype(np.int32)
    doc = np.stack([doc, np.sort(rng.integers(0, 5, 1000))]).astype(np.int32)
    for (B, H, q_len, kv_len, bq, bk, k, off) in ((2, 3, 700, 900, 64, 128, 8, 0),
                                                  (1, 4, 333, 1000, 128, 64, 12, 400),
                                                  (2, 1, 1000, 1000, 64, 64, 20, 0),
                                                  (1, 2, 1, 1000, 128, 128, 6, 999),
                                                  (2, 2, 256, 256, 128, 128, 0, 0)):
        nqb, nkb = OB.n_blocks(q_len, bq), OB.n_blocks(kv_len, bk)
        sel = random_selection(B, H, nqb, nkb, k, seed=q_len + k)
        uses_doc = "doc" in str(spec)
        d = doc[:B] if uses_doc else None
        _, got = gpu_select(spec, sel, B, H, q_len, kv_len, bq, bk, off, d)
        want = OS.tables_from_selection(spec, sel, B, H, q_len, kv_len, bq, bk, off, d)
        ctx = f"{spec} B={B} H={H} q={q_len} kv={kv_len} {bq}x{bk} k={k} off={off}"
        assert_tables_equal(got, want, ctx)
        import block_sparse_programmable_amd as fa
        docT = None if d is None else torch.as_tensor(d).cuda()
        kv_only = fa.block_mask_from_indices(torch.as_tensor(sel).cuda(), spec, B, H, q_len, kv_len, bq, bk, off,
                                             docT, q_side=False).compact()
        for key in ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx"):
            assert np.array_equal(kv_only[key], want[key]), ctx + " kv side only: " + key
        assert np.array_equal(got["order"], OS.work_order(want, B, H, q_len, bq)), ctx + ": order"


def test_selector_large_grid():
    """More than 16384 blocks: the multi-launch path, per-head selections."""
    B, H, L, bq, bk, k = 1, 32, 2048, 64, 64, 10
    nqb = nkb = L // 64
    sel = random_selection(B, H, nqb, nkb, k, seed=11)
    for spec in (("causal",), ("or", ("swa", 60), ("prefix", 130))):
        _, got = gpu_select(spec, sel, B, H, L, L, bq, bk)
        want = OS.tables_from_selection(spec, sel, B, H, L, L, bq, bk)
        assert_tables_equal(got, want, f"large {spec}")
        assert np.array_equal(got["order"], OS.work_order(want, B, H, L, bq))


def test_builder_work_order():
    """The plain builder writes the same order when asked, on both of its paths."""
    import block_sparse_programmable_amd as fa
    for (spec, B, H, L, bq, bk) in ((("causal",), 1, 2, 1000, 64, 64), (("swa", 300), 1, 1, 700, 128, 64),
                                    (("prefix", 500), 1, 3, 1500, 64, 64), (("causal",), 1, 1, 16384, 128, 128)):
        bm = fa.create_block_mask(spec, B, H, L, L, bq, bk, order=True)
        torch.cuda.synchronize()
        got = bm.compact()
        want = OB.tables(spec, B, H, L, L, bq, bk)
        assert_tables_equal(got, want, f"builder {spec}")
        assert np.array_equal(got["order"], OS.work_order(want, B, H, L, bq)), f"builder order {spec}"


def selected_fn(spec, sel, B, H, q_len, kv_len, bq, bk, off, doc=None):
    sets = OS.canonical_sets(sel, OB.n_blocks(kv_len, bk))
    mats = {}
    for b in range(B):
        for h in range(H):
            dr = None if doc is None else doc[b]
            mats[(b, h)] = OS.selected_mask(spec, sets, H, b, h, q_len, kv_len, bq, bk, off, dr)

    def fn(b, h, i, j):
        M = mats[(b if B > 1 else 0, h if H > 1 else 0)]
        return M[np.asarray(i).reshape(-1) - off][:, np.asarray(j).reshape(-1)]
    return fn


@pytest.mark.parametrize("score", ["identity", "softcap"])
def test_forward_and_backward_over_selector_tables(score):
    """Per-head top-k selection inside a causal rule (GQA, ragged lengths): the forward
    and the backward over the selector tables against the oracle on the selected-pair
    matrix; the work order changes nothing in the outputs."""
    import block_sparse_programmable_amd as fa
    B, Hq, Hkv, q_len, kv_len, d, bq, bk, k = 1, 4, 2, 700, 700, 128, 128, 64, 5
    nqb, nkb = OB.n_blocks(q_len, bq), OB.n_blocks(kv_len, bk)
    rng = np.random.default_rng(3)
    # each query block picks its diagonal block plus k - 1 random earlier ones
    sel = rng.integers(0, nkb, size=(B, Hq, nqb, k)).astype(np.int32)
    sel[..., 0] = (np.arange(nqb) * bq // bk)[None, None, :]
    spec = ("causal",)
    q = randn_bf16((B, Hq, q_len, d), 41).cuda()
    kk = randn_bf16((B, Hkv, kv_len, d), 42).cuda()
    v = randn_bf16((B, Hkv, kv_len, d), 43).cuda()
    do = randn_bf16((B, Hq, q_len, d), 44).cuda()
    fkw = dict(score=score, softcap=20.0 if score == "softcap" else 0.0)
    selT = torch.as_tensor(sel).cuda()
    bm_o = fa.block_mask_from_indices(selT, spec, B, Hq, q_len, kv_len, bq, bk, order=True)
    bm_n = fa.block_mask_from_indices(selT, spec, B, Hq, q_len, kv_len, bq, bk, order=False)
    o, lse = fa.forward(q, kk, v, bm_o, **fkw)
    o2, lse2 = fa.forward(q, kk, v, bm_n, **fkw)
    dq, dk, dv = fa.backward(q, kk, v, o, lse, do, bm_o, **fkw)
    dq2, dk2, dv2 = fa.backward(q, kk, v, o, lse, do, bm_n, **fkw)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2), "forward depends on the work order"
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2), "backward depends on the order"
    fn = selected_fn(spec, sel, B, Hq, q_len, kv_len, bq, bk, 0)
    cap = 20.0 if score == "softcap" else None
    O, L = oracle_forward(q, kk, v, fn, score, cap=cap)
    compare(o, lse, O, L, f"selector forward {score}")
    kw = {"cap": cap} if cap else {}
    DQ, DK, DV = OBW.attention_grads(q.cpu(), kk.cpu(), v.cpu(), do.cpu(), fn, score, **kw)
    for name, g, G in (("dq", dq, DQ), ("dk", dk, DK), ("dv", dv, DV)):
        g = g.cpu().numpy()
        err = float(np.abs(g - G).max())
        bound = G_TOL * max(1.0, float(np.abs(G).max()))
        assert err <= bound, f"selector {score}: {name} max-abs error {err:.3e} > {bound:.3e}"


def test_order_on_causal_tables_changes_nothing():
    """Builder tables with and without the work order: identical forward outputs."""
    import block_sparse_programmable_amd as fa
    q = randn_bf16((1, 8, 1000, 128), 51).cuda()
    k = randn_bf16((1, 8, 1000, 128), 52).cuda()
    v = randn_bf16((1, 8, 1000, 128), 53).cuda()
    for spec in (("causal",), ("swa", 256)):
        a = fa.forward(q, k, v, fa.create_block_mask(spec, 1, 1, 1000, 1000, 128, 128, order=True))
        b = fa.forward(q, k, v, fa.create_block_mask(spec, 1, 1, 1000, 1000, 128, 128))
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), spec


def test_decode_over_per_head_tables():
    """One query per request under GQA with per-head selections: the query heads of a KV
    head walk different rows, so each becomes a split-KV unit of its own (reading its
    group's KV head); the result matches the oracle, MHA with the same tables too, and
    the paged cache gives the contiguous result bit for bit."""
    import block_sparse_programmable_amd as fa
    B, Hq, Hkv, d, L, bq, bk, k = 2, 8, 2, 128, 1500, 128, 128, 4
    nkb = OB.n_blocks(L, bk)
    rng = np.random.default_rng(9)
    sel = rng.integers(-1, nkb, size=(B, Hq, 1, k)).astype(np.int32)
    t = L - 1
    q = randn_bf16((B, Hq, 1, d), 61).cuda()
    kk = randn_bf16((B, Hkv, L, d), 62).cuda()
    v = randn_bf16((B, Hkv, L, d), 63).cuda()
    bm = fa.block_mask_from_indices(torch.as_tensor(sel).cuda(), ("causal",), B, Hq, 1, L, bq, bk, t)
    o, lse = fa.forward(q, kk, v, bm, score="softcap", softcap=30.0)
    torch.cuda.synchronize()
    fn = selected_fn(("causal",), sel, B, Hq, 1, L, bq, bk, t)
    O, Lo = oracle_forward(q, kk, v, fn, "softcap", q_offset=t, cap=30.0)
    compare(o, lse, O, Lo, "decode over per-head selector tables")
    # the same tables with MHA (one query head per KV head) stay on the split-KV path
    kk2 = randn_bf16((B, Hq, L, d), 64).cuda()
    v2 = randn_bf16((B, Hq, L, d), 65).cuda()
    o2, lse2 = fa.forward(q, kk2, v2, bm, score="softcap", softcap=30.0)
    torch.cuda.synchronize()
    O2, L2 = oracle_forward(q, kk2, v2, fn, "softcap", q_offset=t, cap=30.0)
    compare(o2, lse2, O2, L2, "MHA decode over per-head selector tables")
    # paged: one random permutation of 16-key pages holding the same logical K/V
    npg = -(-L // 16)
    perm = torch.as_tensor(np.random.default_rng(10).permutation(B * npg).astype(np.int32))
    pt = perm.reshape(B, npg).cuda()
    caches = []
    for t in (kk, v):
        c = torch.zeros(B * npg, Hkv, 16, d, dtype=torch.bfloat16, device="cuda")
        src = torch.nn.functional.pad(t, (0, 0, 0, npg * 16 - L)).view(B, Hkv, npg, 16, d)
        c.index_copy_(0, perm.long().cuda(), src.permute(0, 2, 1, 3, 4).reshape(B * npg, Hkv, 16, d))
        caches.append(c)
    o3, lse3 = fa.forward_paged(q, caches[0], caches[1], pt, L, bm, score="softcap", softcap=30.0)
    torch.cuda.synchronize()
    assert torch.equal(o3, o) and torch.equal(lse3, lse), "paged per-head decode differs from contiguous"


def test_slices_of_selector_tables():
    """Per-head selector tables built once for a 1500-token context, sliced for decode
    steps and a crop: each slice equals the oracle's tables for the new geometry from the
    same candidates (the rows the slice keeps)."""
    import block_sparse_programmable_amd as fa
    B, H, L, bq, bk, k = 1, 4, 1500, 128, 64, 6
    nqb, nkb = OB.n_blocks(L, bq), OB.n_blocks(L, bk)
    sel = random_selection(B, H, nqb, nkb, k, seed=21)
    spec = ("causal",)
    src = fa.block_mask_from_indices(torch.as_tensor(sel).cuda(), spec, B, H, L, L, bq, bk)
    for q_len, kv_len, q_off in ((1, 1001, 1000), (2, 1500, 1498), (1, 1, 0), (640, 1200, 0), (256, 1500, 1024)):
        s = fa.slice_block_mask(src, q_len, kv_len, q_off)
        torch.cuda.synchronize()
        r0 = q_off // bq
        sub = sel[:, :, r0:r0 + OB.n_blocks(q_len, bq)]
        want = OS.tables_from_selection(spec, sub, B, H, q_len, kv_len, bq, bk, q_off)
        assert_tables_equal(s.compact(), want, f"selector slice q={q_len} kv={kv_len} off={q_off}")


def test_work_order_at_its_largest():
    """The work order at its limit of 4096 query blocks (a 262144-token causal square in
    64-token blocks, tables built by the multi-launch builder): a permutation of every
    table row set, by non-increasing executed-block count, ties by descending index;
    one more query block is refused."""
    import block_sparse_programmable_amd as fa
    L = 4096 * 64
    bm = fa.create_block_mask(("swa", 20000), 1, 1, L, L, 64, 64, order=True)
    torch.cuda.synchronize()
    order = bm.tensors["order"][:4096].cpu().numpy()
    lens = (bm.tensors["kv_num"][:4096] + bm.tensors["full_kv_num"][:4096]).cpu().numpy()
    assert np.array_equal(np.sort(order), np.arange(4096))
    key = lens[order].astype(np.int64) * 8192 + order        # (length, index), both descending
    assert (np.diff(key) < 0).all()
    with pytest.raises(fa.FAError):
        fa.create_block_mask(("swa", 20000), 1, 1, L + 64, L + 64, 64, 64, order=True)
