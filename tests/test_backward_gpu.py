"""GPU backward (dQ, dK, dV) vs the float64 autograd oracle, via the C ABI
("FlexAttention: from rules to fused kernels", section 4).

Bar: for each gradient tensor G (oracle) and g (GPU, fp32), max |g - G| <= 2e-2 *
max(1, max |G|).  The GPU path rounds P and dS to bf16 before the MFMAs (relative
error <= 2^-9 per term) and accumulates in fp32; with N(0,1) inputs the gradient
entries are O(1) sums of such terms."""
import numpy as np
import pytest
import torch

from oracle import backward as OBW
from tests.helpers import randn_bf16

pytestmark = pytest.mark.gpu

G_TOL = 2e-2


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


def run_case(B, Hq, Hkv, q_len, kv_len, d, mask, bq, bk, score, q_offset=0, doc=None, qscale=1.0, seed=0,
             ctx=""):
    import block_sparse_programmable_amd as fa
    q = randn_bf16((B, Hq, q_len, d), seed, qscale).cuda()
    k = randn_bf16((B, Hkv, kv_len, d), seed + 1).cuda()
    v = randn_bf16((B, Hkv, kv_len, d), seed + 2).cuda()
    do = randn_bf16((B, Hq, q_len, d), seed + 3).cuda()
    kw = score_kw(score, Hq, seed)
    docT = None if doc is None else torch.as_tensor(np.asarray(doc, np.int32)).cuda()
    bm = fa.create_block_mask(mask, 1, 1, q_len, kv_len, bq, bk, q_offset, docT)
    fkw = dict(score=score, softcap=kw.get("cap", 0.0),
               alibi_slopes=None if "slopes" not in kw else torch.as_tensor(kw["slopes"]).cuda(),
               relpos=None if "table" not in kw else torch.as_tensor(kw["table"]).cuda(),
               relpos_radius=kw.get("radius", 0))
    o, lse = fa.forward(q, k, v, bm, **fkw)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, bm, **fkw)
    torch.cuda.synchronize()
    DQ, DK, DV = OBW.attention_grads(q.cpu(), k.cpu(), v.cpu(), do.cpu(), mask, score, q_offset=q_offset,
                                     doc_ids=None if doc is None else np.asarray(doc), **kw)
    for name, g, G in (("dq", dq, DQ), ("dk", dk, DK), ("dv", dv, DV)):
        g = g.cpu().numpy()
        assert np.isfinite(g).all(), f"{ctx}: non-finite {name}"
        err = float(np.abs(g - G).max()) if G.size else 0.0
        bound = G_TOL * max(1.0, float(np.abs(G).max()) if G.size else 0.0)
        assert err <= bound, f"{ctx}: {name} max-abs error {err:.3e} > {bound:.3e}"


@pytest.mark.parametrize("score", ["identity", "softcap", "alibi", "relpos"])
def test_backward_scores_and_masks(score):
    for (B, Hq, Hkv, ql, kl, d, mask, bq, bk) in (
            (1, 4, 2, 256, 256, 128, ("causal",), 128, 128),
            (1, 4, 2, 300, 300, 128, ("causal",), 128, 128),   # ragged last block, two heads per KV head
            (2, 2, 1, 300, 300, 64, ("swa", 90), 64, 64),
            (1, 4, 4, 200, 333, 128, ("prefix", 70), 128, 64),
            (1, 2, 2, 190, 190, 128, ("or", ("swa", 40), ("prefix", 20)), 64, 128)):
        run_case(B, Hq, Hkv, ql, kl, d, mask, bq, bk, score, seed=ql + kl,
                 ctx=f"bwd {B}x{Hq}/{Hkv} q{ql} kv{kl} d{d} {mask} {bq}x{bk} {score}")


def test_backward_documents_gqa_and_offsets():
    n = 400
    doc = np.repeat(np.arange(4), [90, 150, 60, 100]).astype(np.int32)[None]
    run_case(1, 8, 2, n, n, 128, ("and", ("doc",), ("causal",)), 128, 128, "alibi", doc=doc, seed=5,
             ctx="bwd doc&causal gqa")
    # decode-like shapes (offset rows) and rows with no allowed key (window past kv)
    run_case(2, 4, 1, 3, 500, 128, ("causal",), 128, 128, "softcap", q_offset=497, seed=6, ctx="bwd offset rows")
    run_case(1, 2, 2, 64, 100, 64, ("swa", 10), 64, 64, "identity", q_offset=150, seed=7, ctx="bwd empty rows")


@pytest.mark.parametrize("bq,bk", [(128, 128), (64, 128), (128, 64)])
def test_backward_eight_leaf_programs(bq, bk):
    """Programs at the 16-node limit mixing every leaf with and/or, with documents: the
    dQ kernel evaluates them per row over a block's keys, the dK/dV kernel per key over
    a block's rows, both on words after the host's operand reordering (the right-deep
    chain would need eight stack values in the order written)."""
    from tests.test_forward_gpu import _chain
    rng = np.random.default_rng(bq + bk)
    n = 420
    lens = []
    while sum(lens) < n:
        lens.append(int(rng.integers(15, 140)))
    doc = np.repeat(np.arange(len(lens)), lens)[:n].astype(np.int32)[None]
    leaves = [("doc",), ("swa", 90), ("prefix", 40), ("causal",), ("swa", 300), ("doc",),
              ("prefix", 333), ("swa", 17)]
    ops = ["or", "and", "or", "and", "or", "and", "or"]
    for right in (False, True):
        run_case(1, 4, 2, n, n, 64, _chain(leaves, ops, right), bq, bk, "softcap", doc=doc,
                 seed=30 + right, ctx=f"bwd chain right={right} {bq}x{bk}")
    run_case(1, 2, 2, 150, n, 64, _chain(leaves, ops, True), bq, bk, "identity", q_offset=n - 150,
             doc=doc, seed=32, ctx=f"bwd chain offset rows {bq}x{bk}")


def test_backward_large_scores():
    run_case(1, 2, 1, 256, 256, 128, ("causal",), 128, 128, "softcap", qscale=6.0, seed=8, ctx="bwd large softcap")
    run_case(1, 2, 1, 256, 256, 128, ("causal",), 128, 128, "identity", qscale=3.0, seed=9, ctx="bwd large identity")


@pytest.mark.parametrize("score", ["alibi", "relpos"])
def test_parameter_gradients(score):
    """Gradients of the ALiBi slopes and of the relative-position table (sums over all
    allowed pairs, accumulated with atomic adds) against the autograd oracle."""
    import block_sparse_programmable_amd as fa
    for (B, Hq, Hkv, n, mask, bq, bk, R) in ((2, 4, 2, 300, ("causal",), 128, 64, 40),
                                             (1, 2, 1, 400, ("or", ("swa", 50), ("prefix", 30)), 64, 128, 1024),
                                             (1, 4, 4, 260, ("swa", 90), 64, 64, 3)):
        q = randn_bf16((B, Hq, n, 128), 71).cuda()
        k = randn_bf16((B, Hkv, n, 128), 72).cuda()
        v = randn_bf16((B, Hkv, n, 128), 73).cuda()
        do = randn_bf16((B, Hq, n, 128), 74).cuda()
        rng = np.random.default_rng(75)
        slopes = np.exp2(-8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32)
        table = (rng.standard_normal((Hq, 2 * R + 1)) * 0.5).astype(np.float32)
        kw = dict(alibi_slopes=torch.as_tensor(slopes).cuda()) if score == "alibi" else \
            dict(relpos=torch.as_tensor(table).cuda(), relpos_radius=R)
        bm = fa.create_block_mask(mask, 1, 1, n, n, bq, bk)
        o, lse = fa.forward(q, k, v, bm, score=score, **kw)
        dq, dk, dv, gp = fa.backward(q, k, v, o, lse, do, bm, score=score, param_grad=True, **kw)
        torch.cuda.synchronize()
        okw = dict(slopes=slopes) if score == "alibi" else dict(table=table, radius=R)
        DQ, DK, DV, GP = OBW.attention_grads(q.cpu(), k.cpu(), v.cpu(), do.cpu(), mask, score, param_grads=True,
                                             **okw)
        ctx = f"{score} B={B} {Hq}/{Hkv} n={n} {mask} R={R}"
        for name, g, G in (("dq", dq, DQ), ("dk", dk, DK), ("dv", dv, DV), ("dparam", gp, GP)):
            g = g.cpu().numpy()
            assert g.shape == G.shape, (ctx, name)
            err = float(np.abs(g - G).max())
            bound = G_TOL * max(1.0, float(np.abs(G).max()))
            assert err <= bound, f"{ctx}: {name} max-abs error {err:.3e} > {bound:.3e}"


def test_backward_full_size_causal_softcap():
    """The causal soft-cap workload at full size (B=2, H=16, N=4096, d=128, cap 20,
    128-blocks): the whole backward on the GPU, dQ, dK and dV compared element by
    element with the float64 autograd oracle on three sampled (batch, head) pairs (with
    Hkv = Hq every KV head's gradient comes from its own query head only)."""
    import block_sparse_programmable_amd as fa
    import workloads as W
    w = W.WORKLOADS["causal_softcap"]
    assert w.Hq == w.Hkv
    q, k, v = W.qkv(w, device="cuda")
    do = W.randn_bf16((w.B, w.Hq, w.q_len, w.d), w.seed + 7, device="cuda")
    bm = fa.create_block_mask(w.mask, 1, 1, w.q_len, w.kv_len, w.block_q, w.block_kv, w.q_offset)
    o, lse = fa.forward(q, k, v, bm, score=w.score, softcap=w.cap)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, bm, score=w.score, softcap=w.cap)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 7), (1, w.Hq - 1)):
        print(f"full-size backward: oracle for batch {b}, head {h}", flush=True)
        sl = lambda t: t[b:b + 1, h:h + 1].cpu()   # noqa: E731
        DQ, DK, DV = OBW.attention_grads(sl(q), sl(k), sl(v), sl(do), w.mask, w.score, cap=w.cap)
        for name, g, G in (("dq", dq, DQ), ("dk", dk, DK), ("dv", dv, DV)):
            g = g[b:b + 1, h:h + 1].cpu().numpy()
            assert np.isfinite(g).all(), f"({b},{h}): non-finite {name}"
            err = float(np.abs(g - G).max())
            bound = G_TOL * max(1.0, float(np.abs(G).max()))
            assert err <= bound, f"({b},{h}): {name} max-abs error {err:.3e} > {bound:.3e}"


def test_stored_and_recomputed_gradients_agree():
    """The dQ pass over the per-pair gradients stored by the dK/dV pass (the full
    workspace, 128 x 128 blocks at d = 128) against the dQ pass that recomputes them
    (the minimum workspace): dK and dV are the same computation, so they match exactly;
    dQ sums the same bf16 gradients (up to the rounding of a recomputed score), and both
    match the oracle within the bar of the other tests."""
    import block_sparse_programmable_amd as fa
    n = 640
    doc = np.repeat(np.arange(6), [100, 200, 90, 150, 100, 60]).astype(np.int32)[None]
    for (B, Hq, Hkv, ql, kl, mask, score, q_offset) in (
            (2, 4, 2, n, n, ("causal",), "softcap", 0),
            (1, 4, 1, 300, 700, ("and", ("doc",), ("swa", 200)), "identity", 400),
            (1, 2, 2, n, n, ("or", ("swa", 100), ("prefix", 64)), "alibi", 0)):
        q = randn_bf16((B, Hq, ql, 128), 81).cuda()
        k = randn_bf16((B, Hkv, kl, 128), 82).cuda()
        v = randn_bf16((B, Hkv, kl, 128), 83).cuda()
        do = randn_bf16((B, Hq, ql, 128), 84).cuda()
        kw = score_kw(score, Hq, 85)
        fkw = dict(score=score, softcap=kw.get("cap", 0.0),
                   alibi_slopes=None if "slopes" not in kw else torch.as_tensor(kw["slopes"]).cuda())
        docT = torch.as_tensor(doc[:, :kl]).cuda() if "doc" in str(mask) else None
        bm = fa.create_block_mask(mask, 1, 1, ql, kl, 128, 128, q_offset, docT)
        o, lse = fa.forward(q, k, v, bm, **fkw)
        a = fa.backward(q, k, v, o, lse, do, bm, store_grads=True, **fkw)
        r = fa.backward(q, k, v, o, lse, do, bm, store_grads=False, **fkw)
        torch.cuda.synchronize()
        ctx = f"{B}x{Hq}/{Hkv} q{ql} kv{kl} {mask} {score} off{q_offset}"
        assert torch.equal(a[1], r[1]) and torch.equal(a[2], r[2]), ctx
        scale = max(1.0, float(r[0].abs().max()))
        assert float((a[0] - r[0]).abs().max()) <= 2.0 ** -7 * scale, ctx
        DQ, _, _ = OBW.attention_grads(q.cpu(), k.cpu(), v.cpu(), do.cpu(), mask, score, q_offset=q_offset,
                                       doc_ids=None if docT is None else doc[:, :kl], **kw)
        for g in (a[0], r[0]):
            err = float(np.abs(g.cpu().numpy() - DQ).max())
            assert err <= G_TOL * max(1.0, float(np.abs(DQ).max())), f"{ctx}: dq {err:.3e}"
