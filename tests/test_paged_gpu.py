"""Paged-KV decode ("FlexAttention: from rules to fused kernels", section 5) vs the
oracle on the gathered logical K/V, through fa_forward_paged.

Caches are filled from random logical K/V through random, fragmented page tables
(pages shuffled among unused ones, some requests sharing prefix pages).  Each case
checks the paged result against the oracle (O max-abs <= 2e-2, LSE <= 1e-3) and
against the contiguous-cache forward on the same logical K/V, which must agree bit
for bit (the same kernel reads the same keys in the same order)."""
import numpy as np
import pytest
import torch

from oracle import paged as OP
from tests.helpers import compare, oracle_forward, randn_bf16

pytestmark = pytest.mark.gpu


def paged_case(B, Hkv, kv_len, d, page_size, seed, share=0, spare=7):
    """Logical K/V [B, Hkv, kv_len, d] and caches + table holding them; requests 1.. share
    their first `share` pages with request 0 (their logical keys there are request 0's)."""
    rng = np.random.default_rng(seed)
    k = randn_bf16((B, Hkv, kv_len, d), seed + 1)
    v = randn_bf16((B, Hkv, kv_len, d), seed + 2)
    npg = -(-kv_len // page_size)
    share = min(share, npg)
    for b in range(1, B):
        k[b, :, :share * page_size] = k[0, :, :share * page_size]
        v[b, :, :share * page_size] = v[0, :, :share * page_size]
    own = [npg if b == 0 else npg - share for b in range(B)]
    num_pages = sum(own) + spare
    perm = rng.permutation(num_pages)                  # fragmented placement
    table = np.zeros((B, npg + 3), dtype=np.int32)     # pt_stride > pages needed
    kc = torch.zeros((num_pages, Hkv, page_size, d), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    nxt = 0
    for b in range(B):
        for lp in range(npg):
            if b > 0 and lp < share:
                table[b, lp] = table[0, lp]
                continue
            pg = int(perm[nxt])
            nxt += 1
            table[b, lp] = pg
            j0 = lp * page_size
            n = min(page_size, kv_len - j0)
            kc[pg, :, :n] = k[b, :, j0:j0 + n]
            vc[pg, :, :n] = v[b, :, j0:j0 + n]
    table[:, npg:] = 10 ** 6                          # never read
    # the oracle's gather reproduces the logical K/V from the caches
    assert torch.equal(torch.as_tensor(OP.gather_logical_kv(kc.float().numpy(), table, kv_len)), k.float())
    return k, v, kc, vc, table


def run_both(q, k, v, kc, vc, table, mask, q_offset, score, **kw):
    import block_sparse_programmable_amd as fa
    kv_len = k.shape[2]
    bm = fa.create_block_mask(mask, 1, 1, q.shape[2], kv_len, 128, 128, q_offset)
    o_p, l_p = fa.forward_paged(q, kc.cuda(), vc.cuda(), torch.as_tensor(table).cuda(), kv_len, bm,
                                score=score, **kw)
    o_c, l_c = fa.forward(q, k.cuda(), v.cuda(), bm, score=score, **kw)
    torch.cuda.synchronize()
    return o_p, l_p, o_c, l_c


def score_args(kind, Hq):
    if kind == "softcap":
        return dict(softcap=30.0), dict(cap=30.0)
    if kind == "alibi":
        s = np.exp2(-8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32)
        return dict(alibi_slopes=torch.as_tensor(s).cuda()), dict(slopes=s)
    if kind == "relpos":
        R = 50   # rows reach past R on the far side, so both table ends are used
        t = (np.random.default_rng(Hq).standard_normal((Hq, 2 * R + 1)) * 0.5).astype(np.float32)
        return dict(relpos=torch.as_tensor(t).cuda(), relpos_radius=R), dict(table=t, radius=R)
    return {}, {}


@pytest.mark.parametrize("page_size", [16, 32, 128, 256])
@pytest.mark.parametrize("score", ["identity", "softcap", "alibi", "relpos"])
def test_paged_decode_matches_oracle_and_contiguous(page_size, score):
    for (B, Hq, Hkv, q_len, kv_len, mask, d, share) in (
            (3, 8, 2, 1, 2000, ("swa", 700), 128, 5),
            (2, 8, 1, 2, 777, ("causal",), 128, 0),
            (4, 16, 4, 1, 1300, ("causal",), 64, 3),
            (2, 4, 2, 2, 129, ("prefix", 40), 128, 1)):
        seed = 100 + kv_len + page_size
        k, v, kc, vc, table = paged_case(B, Hkv, kv_len, d, page_size, seed, share)
        q = randn_bf16((B, Hq, q_len, d), seed + 3).cuda()
        q_off = kv_len - q_len
        fkw, okw = score_args(score, Hq)
        o_p, l_p, o_c, l_c = run_both(q, k, v, kc, vc, table, mask, q_off, score, **fkw)
        ctx = f"paged ps{page_size} {B}x{Hq}/{Hkv} q{q_len} kv{kv_len} d{d} {mask} {score}"
        assert torch.equal(o_p, o_c) and torch.equal(l_p, l_c), f"{ctx}: paged != contiguous"
        O, L = oracle_forward(q, k, v, mask, score, q_offset=q_off, **okw)
        compare(o_p, l_p, O, L, ctx)


@pytest.mark.parametrize("B,Hkv,kv_len", [(64, 4, 1100), (16, 2, 1500)],
                         ids=["splits_in_workgroup", "split_merge_kernel"])
def test_paged_decode_split_paths(B, Hkv, kv_len):
    # the split counts of the contiguous split-path tests, over 16-key pages
    k, v, kc, vc, table = paged_case(B, Hkv, kv_len, 128, 16, seed=7 + B, share=10)
    Hq = 2 * Hkv
    q = randn_bf16((B, Hq, 1, 128), 9 + B).cuda()
    o_p, l_p, o_c, l_c = run_both(q, k, v, kc, vc, table, ("swa", 600), kv_len - 1, "softcap",
                                  softcap=30.0)
    assert torch.equal(o_p, o_c) and torch.equal(l_p, l_c)
    O, L = oracle_forward(q, k, v, ("swa", 600), "softcap", q_offset=kv_len - 1, cap=30.0)
    compare(o_p, l_p, O, L, f"paged split path B{B}")


def test_paged_out_of_range_entries_stay_in_bounds():
    # table entries outside [0, num_pages) are clamped into the cache: the call
    # completes and only the rows that use them are unspecified
    import block_sparse_programmable_amd as fa
    k, v, kc, vc, table = paged_case(2, 2, 300, 128, 16, seed=3)
    table[1, 2] = 10 ** 7
    table[1, 3] = -5
    q = randn_bf16((2, 8, 1, 128), 4).cuda()
    bm = fa.create_block_mask(("causal",), 1, 1, 1, 300, 128, 128, 299)
    o, lse = fa.forward_paged(q, kc.cuda(), vc.cuda(), torch.as_tensor(table).cuda(), 300, bm)
    torch.cuda.synchronize()
    O, L = oracle_forward(q, k, v, ("causal",), q_offset=299)
    compare(o[:1], lse[:1], O[:1], L[:1], "request with valid pages")
    assert torch.isfinite(o).all()
