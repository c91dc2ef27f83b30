"""Seeded random sweep over the forward's inputs (rule, geometry, heads, block sizes,
head dim, score_mod, offsets, table extents, work order) against the float64 oracle,
and over the backward on a subset.  Every case is valid input; the seeds are fixed,
so the sweep is the same every run."""
import numpy as np
import pytest
import torch

from oracle import backward as OBW
from tests.helpers import compare, oracle_forward, randn_bf16

pytestmark = pytest.mark.gpu

LEAVES = [("causal",), ("swa", 1), ("swa", 45), ("swa", 300), ("prefix", 0), ("prefix", 90), ("doc",)]


def random_rule(rng, depth=0):
    if depth < 2 and rng.random() < 0.45:
        return (("and", "or")[int(rng.integers(0, 2))], random_rule(rng, depth + 1), random_rule(rng, depth + 1))
    return LEAVES[int(rng.integers(0, len(LEAVES)))]


def uses_doc(spec):
    return spec[0] == "doc" or (spec[0] in ("and", "or") and (uses_doc(spec[1]) or uses_doc(spec[2])))


def random_case(seed):
    rng = np.random.default_rng(seed)
    Hkv = int(rng.choice([1, 2]))
    g = int(rng.choice([1, 2, 4]))
    c = dict(B=int(rng.integers(1, 3)), Hq=Hkv * g, Hkv=Hkv, d=int(rng.choice([64, 128])),
             bq=int(rng.choice([64, 128])), bk=int(rng.choice([64, 128])), spec=random_rule(rng),
             score=str(rng.choice(["identity", "alibi", "softcap", "relpos"])))
    if rng.random() < 0.25:   # short queries at the end of a longer context
        c["kv_len"] = int(rng.integers(1, 900))
        c["q_len"] = int(rng.integers(1, min(c["kv_len"], 4) + 1))
        c["q_off"] = c["kv_len"] - c["q_len"]
    else:
        c["q_len"] = int(rng.integers(1, 700))
        c["kv_len"] = int(rng.integers(1, 800))
        c["q_off"] = int(rng.integers(0, 300))
    n = c["q_off"] + max(c["q_len"], c["kv_len"])
    c["doc"] = None
    if uses_doc(c["spec"]):
        rows = []
        for _ in range(c["B"]):
            lens = []
            while sum(lens) < n:
                lens.append(int(rng.integers(1, 200)))
            rows.append(np.repeat(np.arange(len(lens)), lens)[:n])
        c["doc"] = np.stack(rows).astype(np.int32)
    c["tB"] = c["B"] if c["doc"] is not None else int(rng.choice([1, c["B"]]))
    c["tH"] = int(rng.choice([1, c["Hq"]]))
    c["order"] = bool(rng.random() < 0.5)
    c["seed"] = seed
    return c


def score_args(c, rng):
    Hq = c["Hq"]
    if c["score"] == "alibi":
        return dict(slopes=np.exp2(-8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32))
    if c["score"] == "softcap":
        return dict(cap=float(rng.choice([5.0, 20.0])))
    if c["score"] == "relpos":
        R = int(rng.integers(0, 60))
        return dict(table=(rng.standard_normal((Hq, 2 * R + 1)) * 0.5).astype(np.float32), radius=R)
    return {}


def run(c, backward=False):
    import block_sparse_programmable_amd as fa
    rng = np.random.default_rng(c["seed"] + 1)
    skw = score_args(c, rng)
    q = randn_bf16((c["B"], c["Hq"], c["q_len"], c["d"]), c["seed"] * 7 + 1).cuda()
    k = randn_bf16((c["B"], c["Hkv"], c["kv_len"], c["d"]), c["seed"] * 7 + 2).cuda()
    v = randn_bf16((c["B"], c["Hkv"], c["kv_len"], c["d"]), c["seed"] * 7 + 3).cuda()
    docT = None if c["doc"] is None else torch.as_tensor(c["doc"]).cuda()
    bm = fa.create_block_mask(c["spec"], c["tB"], c["tH"], c["q_len"], c["kv_len"], c["bq"], c["bk"], c["q_off"],
                              docT, order=c["order"])
    fkw = dict(score=c["score"], softcap=skw.get("cap", 0.0),
               alibi_slopes=None if "slopes" not in skw else torch.as_tensor(skw["slopes"]).cuda(),
               relpos=None if "table" not in skw else torch.as_tensor(skw["table"]).cuda(),
               relpos_radius=skw.get("radius", 0))
    o, lse = fa.forward(q, k, v, bm, **fkw)
    torch.cuda.synchronize()
    ctx = {key: c[key] for key in ("seed", "B", "Hq", "Hkv", "d", "bq", "bk", "q_len", "kv_len", "q_off", "spec",
                                   "score", "tB", "tH", "order")}
    O, L = oracle_forward(q, k, v, c["spec"], c["score"], c["q_off"], c["doc"], **skw)
    compare(o, lse, O, L, str(ctx))
    if backward:
        do = randn_bf16(tuple(o.shape), c["seed"] * 7 + 4).cuda()
        dq, dk, dv = fa.backward(q, k, v, o, lse, do, bm, **fkw)
        torch.cuda.synchronize()
        G = OBW.attention_grads(q.cpu(), k.cpu(), v.cpu(), do.cpu(), c["spec"], c["score"], q_offset=c["q_off"],
                                doc_ids=c["doc"], **skw)
        for name, g, Gt in zip(("dq", "dk", "dv"), (dq, dk, dv), G):
            g = g.cpu().numpy()
            err = float(np.abs(g - Gt).max()) if Gt.size else 0.0
            bound = 2e-2 * max(1.0, float(np.abs(Gt).max()) if Gt.size else 0.0)
            assert err <= bound, f"{ctx}: {name} max-abs error {err:.3e} > {bound:.3e}"


@pytest.mark.parametrize("chunk", range(4))
def test_random_forward(chunk):
    for seed in range(1000 + 12 * chunk, 1000 + 12 * (chunk + 1)):
        run(random_case(seed))


def test_random_backward():
    for seed in range(2000, 2010):
        c = random_case(seed)
        # shorter lengths (the document IDs drawn for the longer ones still cover them)
        c["q_len"] = min(c["q_len"], 300)
        c["kv_len"] = max(min(c["kv_len"], 300), c["q_off"] + c["q_len"] if c["q_len"] <= 4 else 1)
        run(c, backward=True)
