"""fa_forward_noalloc (the forward whose split-KV partial states live in the library's
static device scratch) against fa_forward with a caller workspace: identical results on
two calls in a row, the second smaller, plus the oracle's tolerance (GPU, C ABI)."""
import numpy as np
import pytest
import torch

import block_sparse_programmable_amd as fa
from tests.helpers import compare, oracle_forward, randn_bf16

pytestmark = pytest.mark.gpu

# short-query shapes whose split-KV path needs partial states (the splits of a KV head
# do not fit one workgroup), then a smaller one, then a prefill shape (no scratch)
CASES = [
    dict(B=1, Hq=8, Hkv=2, q_len=1, kv_len=5000, mask=("swa", 3000), score="softcap", cap=30.0, seed=1),
    dict(B=2, Hq=4, Hkv=1, q_len=3, kv_len=1500, mask=("causal",), score="identity", cap=0.0, seed=2),
    dict(B=1, Hq=2, Hkv=2, q_len=300, kv_len=300, mask=("causal",), score="identity", cap=0.0, seed=3),
]


def _run(c, noalloc):
    torch.cuda.set_device(0)
    d = 128
    q = randn_bf16((c["B"], c["Hq"], c["q_len"], d), c["seed"]).cuda()
    k = randn_bf16((c["B"], c["Hkv"], c["kv_len"], d), c["seed"] + 100).cuda()
    v = randn_bf16((c["B"], c["Hkv"], c["kv_len"], d), c["seed"] + 200).cuda()
    q_off = c["kv_len"] - c["q_len"]
    bm = fa.create_block_mask(c["mask"], 1, 1, c["q_len"], c["kv_len"], 128, 128, q_off)
    out = torch.full((c["B"], c["Hq"], c["q_len"], d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((c["B"], c["Hq"], c["q_len"]), float("nan"), dtype=torch.float32, device="cuda")
    args, _, _ = fa.forward_args(q, k, v, bm, c["score"], c["cap"], out=out, lse=lse)
    ws = fa.forward_workspace_size(args)
    if noalloc:
        fa.forward_noalloc(q, k, v, bm, out, lse, score=c["score"], softcap=c["cap"])
    else:
        fa.forward(q, k, v, bm, score=c["score"], softcap=c["cap"], out=out, lse=lse)
    torch.cuda.synchronize()
    return q, k, v, q_off, out, lse, ws


def test_noalloc_matches_workspace_forward_twice():
    got = []
    for i, c in enumerate(CASES):
        print(f"noalloc case {i}: {c}", flush=True)
        q, k, v, q_off, o_ref, l_ref, ws = _run(c, noalloc=False)
        _, _, _, _, o, l, _ = _run(c, noalloc=True)
        if i < 2:
            assert ws > 0, "the case must use split-KV partial states"
        assert torch.equal(o, o_ref), f"case {i}: O differs from fa_forward"
        assert torch.equal(l, l_ref), f"case {i}: LSE differs from fa_forward"
        O, L = oracle_forward(q, k, v, c["mask"], c["score"], q_offset=q_off, cap=c["cap"] or None)
        compare(o, l, O, L, f"noalloc case {i}")
        got.append(ws)
    assert got[1] < got[0], "the second call must be the smaller one"
