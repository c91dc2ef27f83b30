"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Every check here compares the oracle with something other than itself: values
printed on the pages (tests/golden, each file cites its passage), closed forms,
invariants, special cases that reduce to a library routine (torch SDPA, torch's
own CPU FlexAttention), and brute force on tiny inputs.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import blockmask as OB
from oracle import masks as OM
from oracle import merge as OMG

CHARS = {OB.EMPTY: ".", OB.PARTIAL: "P", OB.FULL: "F"}


def grid_str(grid):
    return ["".join(CHARS[int(x)] for x in row) for row in grid]


# ---------------------------------------------------------------- worked examples

def test_worked_n8_w4_grid(golden):
    kv, _ = golden("worked_n8_w4_2x2.txt")
    spec = ("swa", kv["W"])
    grid = OB.classify(spec, kv["q_len"], kv["kv_len"], kv["block_q"], kv["block_kv"])
    assert grid_str(grid) == kv["grid"]
    M = OM.dense(spec, kv["q_len"], kv["kv_len"])
    assert int(M.sum()) == kv["valid_edges"]
    executed = int((grid != OB.EMPTY).sum())
    assert executed == kv["executed_blocks"]
    assert executed * kv["block_q"] * kv["block_kv"] == kv["covered_elements"]
    assert int((grid == OB.EMPTY).sum()) == kv["empty_blocks"]
    # block (queries 4-5, keys 0-1) holds only the edge (4, 1)
    sub = M[4:6, 0:2]
    assert sub.tolist() == [[False, True], [False, False]]
    assert M[4:6, 2:4].all()


def test_worked_n16_w8_last_row(golden):
    kv, _ = golden("worked_n16_w8_4x4_lastrow.txt")
    grid = OB.classify(("swa", kv["W"]), kv["q_len"], kv["kv_len"], kv["block_q"], kv["block_kv"])
    assert grid_str(grid)[-1] == kv["last_row"]


def test_interval_example(golden):
    kv, _ = golden("interval_a4_b7_w4.txt")
    spec = ("swa", kv["W"])
    M = OM.dense(spec, 8, 8)
    rows = M[kv["a"]:kv["b"] + 1]
    union = np.nonzero(rows.any(axis=0))[0]
    inter = np.nonzero(rows.all(axis=0))[0]
    assert (union.min(), union.max()) == (kv["union_lo"], kv["union_hi"])
    assert len(union) == union.max() - union.min() + 1
    assert (inter.min(), inter.max()) == (kv["inter_lo"], kv["inter_hi"])
    grid = OB.classify(spec, 8, 8, kv["b"] - kv["a"] + 1, kv["block_kv"])
    assert grid_str(grid)[1] == kv["row_classes"]


def test_pair_counts_n8192(golden):
    kv, _ = golden("pair_counts_n8192_w1024.txt")
    N, W = kv["N"], kv["W"]
    assert int(OM.dense(("swa", W), N, N).sum()) == kv["window_pairs"]
    assert int(OM.dense(("causal",), N, N).sum()) == kv["causal_pairs"]
    # prefix over the whole sequence allows every pair
    assert int(OM.dense(("prefix", N), N, N).sum()) == kv["dense_pairs"]
    # the page's verbal formula: 1 + ... + W for the first W rows, W for the rest
    assert W * (W + 1) // 2 + (N - W) * W == kv["window_pairs"]


def test_causal_skip_fraction_table(golden):
    _, rows = golden("causal_skip_fraction_b64.txt")
    for N, pct, n_empty, n_full, n_bnd in rows:
        N = int(N)
        grid = OB.classify(("causal",), N, N, 64, 64)
        e, f, p = [int((grid == c).sum()) for c in (OB.EMPTY, OB.FULL, OB.PARTIAL)]
        assert (e, f, p) == (int(n_empty), int(n_full), int(n_bnd))
        exact = 100.0 * e / grid.size
        assert math.floor(exact * 10) / 10 == float(pct)


def test_causal_geometric_rule_matches_classes():
    # "Causal block geometric pruning", section 1: empty iff (i+1)Br-1 < jBc, full iff
    # iBr >= (j+1)Bc-1, otherwise boundary (rectangular blocks included).
    for Br, Bc, N in ((64, 64, 1024), (32, 64, 512), (64, 32, 512), (16, 48, 480)):
        grid = OB.classify(("causal",), N, N, Br, Bc)
        for i in range(grid.shape[0]):
            for j in range(grid.shape[1]):
                if (i + 1) * Br - 1 < j * Bc:
                    want = OB.EMPTY
                elif i * Br >= (j + 1) * Bc - 1:
                    want = OB.FULL
                else:
                    want = OB.PARTIAL
                assert grid[i, j] == want, (Br, Bc, i, j)


def test_grid_size_64k():
    # "FlexAttention: from rules to fused kernels", section 2.1: a 64K sequence with
    # 128 x 128 blocks has 262,144 blocks and about 4.2e9 elements.
    nqb = OB.n_blocks(65536, 128)
    assert nqb * nqb == 262144
    assert 65536 * 65536 == 4294967296


# ---------------------------------------------------------------- closed-form counts

@pytest.mark.parametrize("T,w,B", [(8, 2, 64), (64, 8, 16), (16, 1, 8), (16, 16, 4), (12, 5, 8)])
def test_swa_block_counts_closed_form(T, w, B):
    N, W = T * B, w * B
    grid = OB.classify(("swa", W), N, N, B, B)
    full = w * (w - 1) // 2 + (T - w) * (w - 1)
    part = 2 * T - w
    assert int((grid == OB.FULL).sum()) == full
    assert int((grid == OB.PARTIAL).sum()) == part


def test_swa_counts_at_workload_sizes():
    # tiny workload: T = 8, w = 2 gives 7 full / 14 partial; the window of the
    # document workload without documents: T = 64, w = 8 gives 420 / 120.
    for T, w, want in ((8, 2, (7, 14)), (64, 8, (420, 120))):
        full = w * (w - 1) // 2 + (T - w) * (w - 1)
        part = 2 * T - w
        assert (full, part) == want
    grid = OB.classify(("swa", 128), 512, 512, 64, 64)
    assert (int((grid == OB.FULL).sum()), int((grid == OB.PARTIAL).sum())) == (7, 14)


@pytest.mark.parametrize("T,p,B", [(16, 4, 8), (32, 2, 4), (8, 8, 16), (10, 0, 8)])
def test_prefix_block_counts_closed_form(T, p, B):
    N, P = T * B, p * B
    grid = OB.classify(("prefix", P), N, N, B, B)
    full = p * p + (T * (T - 1) - p * (p - 1)) // 2 if p > 0 else T * (T - 1) // 2
    part = T - p
    assert int((grid == OB.FULL).sum()) == full
    assert int((grid == OB.PARTIAL).sum()) == part
    # the 64K prefix-LM workload: T = 512, p = 32
    assert 32 * 32 + (512 * 511 - 32 * 31) // 2 == 131344


@pytest.mark.parametrize("T,w,B", [(256, 32, 128), (64, 8, 16), (16, 3, 8)])
def test_decode_window_counts(T, w, B):
    # one query at the last position; window of w whole blocks ends at it
    N = T * B
    grid = OB.classify(("swa", w * B), 1, N, B, B, q_offset=N - 1)
    assert int((grid == OB.FULL).sum()) == w
    assert int((grid == OB.PARTIAL).sum()) == 0
    assert list(np.nonzero(grid[0])[0]) == list(range(T - w, T))


def test_pair_count_closed_forms_prefix_doc():
    N, P = 1024, 96
    assert int(OM.dense(("prefix", P), N, N).sum()) == N * (N + 1) // 2 + P * (P - 1) // 2
    lens = np.array([300, 17, 1, 256, 450])
    doc = np.repeat(np.arange(len(lens)), lens).astype(np.int32)
    n = int(lens.sum())
    got = int(OM.dense(("and", ("doc",), ("causal",)), n, n, 0, doc).sum())
    assert got == int(sum(L * (L + 1) // 2 for L in lens))
    W = 100
    got = int(OM.dense(("and", ("doc",), ("swa", W)), n, n, 0, doc).sum())
    want = sum(W * (W + 1) // 2 + (L - W) * W if L >= W else L * (L + 1) // 2 for L in lens)
    assert got == want


# ---------------------------------------------------------------- brute force on tiny inputs

def brute_allowed(spec, i, j, doc):
    op = spec[0]
    if op == "causal":
        return j <= i
    if op == "swa":
        return j <= i and i - j < spec[1]
    if op == "prefix":
        return j < spec[1] or j <= i
    if op == "doc":
        return doc[i] == doc[j]
    a = brute_allowed(spec[1], i, j, doc)
    b = brute_allowed(spec[2], i, j, doc)
    return (a and b) if op == "and" else (a or b)


LEAVES = [("causal",), ("swa", 3), ("prefix", 2), ("doc",)]
SPECS = LEAVES + [(op, a, b) for op in ("and", "or") for a, b in itertools.combinations(LEAVES, 2)]


def brute_tables(spec, q_len, kv_len, bq, bk, q_off, doc):
    nqb, nkb = -(-q_len // bq), -(-kv_len // bk)
    cls = {}
    for r in range(nqb):
        for c in range(nkb):
            pairs = [(i, j) for i in range(r * bq, min((r + 1) * bq, q_len))
                     for j in range(c * bk, min((c + 1) * bk, kv_len))]
            vals = [brute_allowed(spec, i + q_off, j, doc) for i, j in pairs]
            cls[r, c] = "F" if all(vals) else ("P" if any(vals) else ".")
    rows_p = [[c for c in range(nkb) if cls[r, c] == "P"] for r in range(nqb)]
    rows_f = [[c for c in range(nkb) if cls[r, c] == "F"] for r in range(nqb)]
    cols_p = [[r for r in range(nqb) if cls[r, c] == "P"] for c in range(nkb)]
    cols_f = [[r for r in range(nqb) if cls[r, c] == "F"] for c in range(nkb)]
    return rows_p, rows_f, cols_p, cols_f


def unpack(num, ptr, idx):
    out = []
    for r in range(len(num)):
        assert ptr[r + 1] - ptr[r] == num[r]
        out.append([int(x) for x in idx[ptr[r]:ptr[r + 1]]])
    return out


@pytest.mark.parametrize("spec", SPECS, ids=[str(s) for s in SPECS])
def test_exhaustive_tiny(spec):
    B = 4
    rng = np.random.default_rng(7)
    docs = [np.array([0, 0, 0, 1, 1, 2, 2, 2, 2, 3, 3, 3, 3, 3, 4, 4, 5, 5, 5, 5], np.int32),
            rng.integers(0, 3, 20).astype(np.int32)]          # non-monotone IDs
    for doc in docs:
        for q_len, kv_len, q_off in [(1, 1, 0), (3, 3, 0), (B - 1, B - 1, 0), (B, B, 0),
                                     (B + 1, B + 1, 0), (2 * B + 3, 2 * B + 3, 0),
                                     (3, 2 * B + 3, 8), (2 * B + 3, 5, 0), (5, 9, 4)]:
            i = np.arange(q_len)[:, None] + q_off
            j = np.arange(kv_len)[None, :]
            M = OM.dense(spec, q_len, kv_len, q_off, doc)
            for ii in range(q_len):
                for jj in range(kv_len):
                    assert M[ii, jj] == brute_allowed(spec, ii + q_off, jj, doc)
            del i, j
            for bq, bk in ((B, B), (2, B), (B, 3)):
                tab = OB.tables(spec, 1, 2, q_len, kv_len, bq, bk, q_off, doc[None])
                rp, rf, cp, cf = brute_tables(spec, q_len, kv_len, bq, bk, q_off, doc)
                assert unpack(tab["kv_num"], tab["kv_ptr"], tab["kv_idx"]) == rp + rp
                assert unpack(tab["full_kv_num"], tab["full_kv_ptr"], tab["full_kv_idx"]) == rf + rf
                assert unpack(tab["q_num"], tab["q_ptr"], tab["q_idx"]) == cp + cp
                assert unpack(tab["full_q_num"], tab["full_q_ptr"], tab["full_q_idx"]) == cf + cf
                # expanding the tables reproduces the element mask exactly
                E = OB.expand(tab, 1, 2, q_len, kv_len, bq, bk, spec, q_off, doc[None], h=1)
                assert (E == M).all()


def test_per_batch_doc_tables():
    doc = np.array([[0, 0, 1, 1, 1, 2, 2, 2], [0, 1, 1, 1, 1, 1, 1, 2]], np.int32)
    tab = OB.tables(("and", ("doc",), ("causal",)), 2, 1, 8, 8, 2, 2, 0, doc)
    for b in range(2):
        rp, rf, _, _ = brute_tables(("and", ("doc",), ("causal",)), 8, 8, 2, 2, 0, doc[b])
        got_p = unpack(tab["kv_num"], tab["kv_ptr"], tab["kv_idx"])[4 * b:4 * b + 4]
        got_f = unpack(tab["full_kv_num"], tab["full_kv_ptr"], tab["full_kv_idx"])[4 * b:4 * b + 4]
        assert got_p == rp and got_f == rf


# ---------------------------------------------------------------- attention special cases

def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa(q, k, v, mask=None, causal=False, bias=None):
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)) for x in (q, k, v))
    attn = None
    if mask is not None:
        attn = torch.from_numpy(mask)
    if bias is not None:
        attn = torch.from_numpy(bias)
    return torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=attn, is_causal=causal).numpy()


def test_identity_causal_matches_sdpa():
    q, k, v = rand((2, 3, 37, 16), 1), rand((2, 3, 37, 16), 2), rand((2, 3, 37, 16), 3)
    O, _ = OA.attention(q, k, v, ("causal",))
    assert np.abs(O - sdpa(q, k, v, causal=True)).max() < 1e-12


def test_identity_window_gqa_matches_sdpa_expanded():
    q, k, v = rand((1, 4, 29, 8), 4), rand((1, 2, 29, 8), 5), rand((1, 2, 29, 8), 6)
    spec = ("swa", 5)
    O, _ = OA.attention(q, k, v, spec)
    M = OM.dense(spec, 29, 29)
    ke, ve = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)   # repeat_interleave of heads
    assert np.abs(O - sdpa(q, ke, ve, mask=M)).max() < 1e-12


def test_gqa_distinct_slopes_equals_expanded():
    # two query heads share a KV head but carry different ALiBi slopes
    q, k, v = rand((1, 4, 19, 8), 7), rand((1, 2, 19, 8), 8), rand((1, 2, 19, 8), 9)
    slopes = np.array([0.5, 0.125, 0.25, 0.0625])
    O, L = OA.attention(q, k, v, ("causal",), "alibi", slopes=slopes)
    Oe, Le = OA.attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), ("causal",),
                          "alibi", slopes=slopes)
    assert np.abs(O - Oe).max() < 1e-13 and np.abs(L - Le).max() < 1e-13
    # h_kv = h_q // g, not h_q % Hkv: a modular mapping gives a different answer
    k_alt = k[:, [0, 1, 0, 1]]
    v_alt = v[:, [0, 1, 0, 1]]
    Oa, _ = OA.attention(q, k_alt, v_alt, ("causal",), "alibi", slopes=slopes)
    assert np.abs(O - Oa).max() > 1e-3


def test_single_key_row_and_uniform_rows():
    q, k, v = rand((1, 1, 12, 8), 10), rand((1, 1, 12, 8), 11), rand((1, 1, 12, 8), 12)
    for kind, kw in (("identity", {}), ("softcap", dict(cap=2.0)),
                     ("alibi", dict(slopes=[0.7])),
                     ("relpos", dict(table=rand((1, 7), 13), radius=3))):
        O, L = OA.attention(q, k, v, ("causal",), kind, **kw)
        # row 0 of a causal mask has exactly one key: O = V_0 and LSE = the modified score
        assert np.abs(O[0, 0, 0] - v[0, 0, 0]).max() < 1e-14
        s = float(q[0, 0, 0] @ k[0, 0, 0]) / math.sqrt(8)
        want = {"identity": s, "softcap": 2.0 * math.tanh(s / 2.0), "alibi": s,
                "relpos": s + kw.get("table", np.zeros((1, 7)))[0][3]}[kind]
        assert abs(L[0, 0, 0] - want) < 1e-12
    # Q = 0 with identity: uniform weights over the allowed keys
    z = np.zeros_like(q)
    for spec in (("causal",), ("swa", 4), ("prefix", 5)):
        O, L = OA.attention(z, k, v, spec)
        M = OM.dense(spec, 12, 12)
        for i in range(12):
            n = M[i].sum()
            assert abs(L[0, 0, i] - math.log(n)) < 1e-13
            assert np.abs(O[0, 0, i] - v[0, 0][M[i]].mean(axis=0)).max() < 1e-13


def test_alibi_geometric_closed_form():
    # zero scores: causal row i weighs key j by exp(slope (j - i)), a geometric
    # series; the weights and the log-normaliser have closed forms.  One-hot
    # values expose each weight.
    n, slope = 24, 0.3
    z = np.zeros((1, 1, n, n))
    eye = np.eye(n)[None, None]
    O, L = OA.attention(z, z, eye, ("causal",), "alibi", slopes=[slope])
    for i in range(n):
        Z = (1 - math.exp(-slope * (i + 1))) / (1 - math.exp(-slope))
        assert abs(L[0, 0, i] - math.log(Z)) < 1e-12
        for j in range(i + 1):
            assert abs(O[0, 0, i, j] - math.exp(-slope * (i - j)) / Z) < 1e-12
        assert np.abs(O[0, 0, i, i + 1:]).max(initial=0.0) == 0.0


def test_relpos_offset_sign_and_clip():
    n, R, big = 20, 4, 5.0
    z = np.zeros((1, 1, n, n))
    eye = np.eye(n)[None, None]
    # bias only for i - j = 1 (table index R + 1): the previous token is preferred
    tab = np.zeros((1, 2 * R + 1))
    tab[0, R + 1] = big
    O, L = OA.attention(z, z, eye, ("prefix", n), "relpos", table=tab, radius=R)
    for i in range(1, n):
        Z = math.exp(big) + (n - 1)
        assert abs(O[0, 0, i, i - 1] - math.exp(big) / Z) < 1e-12
        assert abs(L[0, 0, i] - math.log(Z)) < 1e-12
    # bias at the clip end (index 2R): every key with i - j >= R gets it
    tab = np.zeros((1, 2 * R + 1))
    tab[0, 2 * R] = big
    O, L = OA.attention(z, z, eye, ("causal",), "relpos", table=tab, radius=R)
    for i in range(n):
        far = max(0, i - R + 1)          # keys j <= i - R
        Z = far * math.exp(big) + (i + 1 - far)
        assert abs(L[0, 0, i] - math.log(Z)) < 1e-12
    # the negative clip end (index 0) is reached by keys ahead of the query (j - i >= R)
    tab = np.zeros((1, 2 * R + 1))
    tab[0, 0] = big
    O, L = OA.attention(z, z, eye, ("prefix", n), "relpos", table=tab, radius=R)
    for i in range(n):
        ahead = max(0, n - (i + R))       # keys j >= i + R
        Z = ahead * math.exp(big) + (n - ahead)
        assert abs(L[0, 0, i] - math.log(Z)) < 1e-12


def test_softcap_limits_and_bounds():
    q, k, v = rand((1, 2, 16, 8), 14) * 3, rand((1, 2, 16, 8), 15) * 3, rand((1, 2, 16, 8), 16)
    O0, L0 = OA.attention(q, k, v, ("causal",))
    O1, L1 = OA.attention(q, k, v, ("causal",), "softcap", cap=1e7)   # |tanh x - x| <= |x|^3/3
    assert np.abs(O0 - O1).max() < 1e-9 and np.abs(L0 - L1).max() < 1e-9
    cap = 0.5
    _, L = OA.attention(q, k, v, ("causal",), "softcap", cap=cap)
    n = np.arange(1, 17)
    assert (L[0, 0] <= np.log(n) + cap + 1e-12).all()
    assert (L[0, 0] >= np.log(n) - cap - 1e-12).all()


def test_mask_after_softcap_order():
    # Correct order: modify, then mask -> masked keys carry exactly zero weight.
    # The wrong order (mask to -inf, then soft-cap) turns -inf into -CAP and
    # gives each masked key a weight proportional to exp(-CAP).
    n, cap = 10, 3.0
    q, k = rand((1, 1, n, 8), 17), rand((1, 1, n, 8), 18)
    eye = np.eye(n)[None, None]
    O, _ = OA.attention(q, k, eye, ("causal",), "softcap", cap=cap)
    M = OM.dense(("causal",), n, n)
    assert (O[0, 0][~M] == 0.0).all()
    S = (q[0, 0] @ k[0, 0].T) / math.sqrt(8)
    wrong = cap * np.tanh(np.where(M, S, -np.inf) / cap)
    P = np.exp(wrong - wrong.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    assert (P[~M] > 0).all()
    assert np.abs(P - O[0, 0]).max() > 1e-3


def test_finite_bias_leak_mass():
    # "FlexAttention: from rules to fused kernels", section 6.3: replacing the mask
    # by a finite -C leaks m e^-C / (Z + m e^-C) of the probability mass.
    n, C = 16, 6.0
    z = np.zeros((1, 1, n, n))
    eye = np.eye(n)[None, None]
    M = OM.dense(("causal",), n, n)
    bias = np.where(M, 0.0, -C)[None, None]
    Ob = sdpa(z, z, eye, bias=bias)
    O, _ = OA.attention(z, z, eye, ("causal",))
    for i in range(n):
        m = n - (i + 1)
        Z = i + 1
        leak = m * math.exp(-C) / (Z + m * math.exp(-C))
        assert abs(Ob[0, 0, i][~M[i]].sum() - leak) < 1e-12
        assert O[0, 0, i][~M[i]].sum() == 0.0


def test_empty_rows():
    q, k, v = rand((1, 1, 3, 8), 19), rand((1, 1, 4, 8), 20), rand((1, 1, 4, 8), 21)
    # window of 3 ending at global positions 10..12 never reaches keys 0..3
    O, L = OA.attention(q, k, v, ("swa", 3), q_offset=10)
    assert (O == 0).all() and np.isneginf(L).all()
    # rows at global 5, 6, 7: row 5 keeps key 3 only, rows 6 and 7 are empty
    O, L = OA.attention(q, k, v, ("swa", 3), q_offset=5)
    assert np.abs(O[0, 0, 0] - v[0, 0, 3]).max() < 1e-14
    assert abs(L[0, 0, 0] - float(q[0, 0, 0] @ k[0, 0, 3]) / math.sqrt(8)) < 1e-13
    assert (O[0, 0, 1:] == 0).all() and np.isneginf(L[0, 0, 1:]).all()


@pytest.mark.parametrize("cuts", [[3], [1, 7], [0, 0, 5, 20], [2, 4, 6, 8, 10]])
def test_split_merge_equals_unsplit(cuts):
    rng = np.random.default_rng(22)
    n, d = 24, 5
    s = rng.standard_normal(n) * 4
    s[[2, 9, 10, 11]] = -np.inf                               # masked keys
    v = rng.standard_normal((n, d))
    bounds = [0] + cuts + [n]
    states = [OMG.partial_state(s[a:b], v[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
    O, L = OMG.merge(states)
    w = np.exp(s - s[np.isfinite(s)].max())
    assert np.abs(O - (w @ v) / w.sum()).max() < 1e-13
    assert abs(L - (s[np.isfinite(s)].max() + math.log(w.sum()))) < 1e-13
    O, L = OMG.merge([OMG.partial_state(s[[2, 9]], v[[2, 9]])])
    assert (O == 0).all() and L == -np.inf


# ---------------------------------------------------------------- torch's CPU FlexAttention

def _torch_flex(q, k, v, mask_spec, kind, q_off=0, doc=None, cap=None, slopes=None,
                table=None, radius=None):
    from torch.nn.attention.flex_attention import create_block_mask, flex_attention
    T = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    docT = T(doc) if doc is not None else None

    def pred(spec, i, j):
        op = spec[0]
        if op == "causal":
            return j <= i
        if op == "swa":
            return (j <= i) & (i - j < spec[1])
        if op == "prefix":
            return (j < spec[1]) | (j <= i)
        if op == "doc":
            return docT[i] == docT[j]
        a, b = pred(spec[1], i, j), pred(spec[2], i, j)
        return (a & b) if op == "and" else (a | b)

    def mask_mod(b, h, qi, ki):
        return pred(mask_spec, qi + q_off, ki)

    slT = T(np.asarray(slopes, np.float64)) if slopes is not None else None
    tbT = T(np.asarray(table, np.float64)) if table is not None else None

    def score_mod(s, b, h, qi, ki):
        i = qi + q_off
        if kind == "softcap":
            return cap * torch.tanh(s / cap)
        if kind == "alibi":
            return s + slT[h] * (ki - i)
        if kind == "relpos":
            return s + tbT[h, torch.clamp(i - ki, -radius, radius) + radius]
        return s

    Lq, Lk = q.shape[2], k.shape[2]
    bm = create_block_mask(mask_mod, None, None, Lq, Lk, device="cpu", BLOCK_SIZE=8)
    o, lse = flex_attention(T(q), T(k), T(v), score_mod=score_mod, block_mask=bm,
                            return_lse=True, enable_gqa=q.shape[1] != k.shape[1])
    return o.numpy(), lse.numpy()


@pytest.mark.parametrize("case", [
    dict(spec=("causal",), kind="softcap", cap=1.5),
    dict(spec=("and", ("doc",), ("swa", 9)), kind="alibi", slopes=[0.5, 0.25, 0.125, 0.0625]),
    dict(spec=("prefix", 16), kind="relpos", radius=6),
    dict(spec=("or", ("swa", 5), ("prefix", 8)), kind="identity", q_off=0),
])
def test_oracle_matches_torch_cpu_flexattention(case):
    pytest.importorskip("torch.nn.attention.flex_attention")
    q = rand((1, 4, 48, 16), 30) * 2
    k = rand((1, 2, 48, 16), 31) * 2
    v = rand((1, 2, 48, 16), 32)
    doc = np.repeat(np.arange(5), [7, 13, 3, 20, 5]).astype(np.int32)
    table = rand((4, 2 * case.get("radius", 1) + 1), 33)
    kw = dict(cap=case.get("cap"), slopes=case.get("slopes"), table=table,
              radius=case.get("radius"))
    O, L = OA.attention(q, k, v, case["spec"], case["kind"], doc_ids=doc[None], **kw)
    Ot, Lt = _torch_flex(q, k, v, case["spec"], case["kind"], doc=doc, **kw)
    assert np.abs(O - Ot).max() < 1e-10
    assert np.abs(L - Lt).max() < 1e-10


# ---- paged KV gather ("FlexAttention: from rules to fused kernels", section 5)

def test_paged_gather_worked_example():
    from oracle import paged as OP
    # two requests, page size 2, one KV head of width 1; physical pages hold the values
    # 10+p, 20+p (rows 0 and 1 of page p)
    cache = np.array([[[[10 + p], [20 + p]]] for p in range(4)], dtype=np.float64)
    table = np.array([[3, 0, 2], [1, 1, 0]], dtype=np.int32)
    got = OP.gather_logical_kv(cache, table, kv_len=5)
    want0 = [13, 23, 10, 20, 12]       # pages 3, 0, 2 (the last page holds one key)
    want1 = [11, 21, 11, 21, 10]       # page 1 twice: a shared page read twice
    assert got.shape == (2, 1, 5, 1)
    assert got[0, 0, :, 0].tolist() == want0
    assert got[1, 0, :, 0].tolist() == want1


def test_paged_gather_identity_table_and_shared_prefix():
    from oracle import paged as OP
    rng = np.random.default_rng(5)
    B, H, T, d, ps = 3, 2, 50, 4, 16
    k = rng.standard_normal((B, H, T, d))
    npg = -(-T // ps)
    cache = np.zeros((B * npg, H, ps, d))
    for b in range(B):
        for lp in range(npg):
            n = min(ps, T - lp * ps)
            cache[b * npg + lp, :, :n] = k[b, :, lp * ps:lp * ps + n]
    ident = np.arange(B * npg, dtype=np.int32).reshape(B, npg)
    assert np.array_equal(OP.gather_logical_kv(cache, ident, T), k)
    # request 2 reuses request 0's first two pages: its first 32 keys become request 0's
    shared = ident.copy()
    shared[2, :2] = shared[0, :2]
    g = OP.gather_logical_kv(cache, shared, T)
    assert np.array_equal(g[2, :, :32], k[0, :, :32])
    assert np.array_equal(g[2, :, 32:], k[2, :, 32:])
    with pytest.raises(ValueError):
        OP.gather_logical_kv(cache, np.full((1, npg), B * npg, dtype=np.int32), T)


# ---- backward: gradients of the dense definition ("FlexAttention: from rules to fused
# kernels", section 4), pinned by finite differences of the forward oracle

@pytest.mark.parametrize("kind", ["identity", "softcap", "alibi", "relpos"])
def test_backward_matches_finite_differences(kind):
    from oracle import backward as OBW
    rng = np.random.default_rng(11)
    B, Hq, Hkv, ql, kl, d = 1, 2, 1, 5, 7, 3
    q = rng.standard_normal((B, Hq, ql, d))
    k = rng.standard_normal((B, Hkv, kl, d))
    v = rng.standard_normal((B, Hkv, kl, d))
    do = rng.standard_normal((B, Hq, ql, d))
    # causal with q_offset=-... : row 0 sees key 0 only; a window rule leaves one row empty
    spec = ("and", ("causal",), ("swa", 3))
    kw = dict(cap=0.7, slopes=[0.5, 0.25], table=rng.standard_normal((Hq, 5)), radius=2)
    kw = {"identity": {}, "softcap": dict(cap=kw["cap"]), "alibi": dict(slopes=kw["slopes"]),
          "relpos": dict(table=kw["table"], radius=kw["radius"])}[kind]
    dq, dk, dv = OBW.attention_grads(q, k, v, do, spec, kind, q_offset=1, **kw)

    def loss(q_, k_, v_):
        O, _ = OA.attention(q_, k_, v_, spec, kind, q_offset=1, **kw)
        return float((O * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [tuple(rng.integers(0, n) for n in x.shape) for _ in range(6)]:
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[idx]) < 1e-6 * max(1.0, abs(fd)), (kind, name, idx, fd, g[idx])


def test_backward_matches_sdpa_causal():
    from oracle import backward as OBW
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 2, 9, 4))
    k = rng.standard_normal((1, 2, 9, 4))
    v = rng.standard_normal((1, 2, 9, 4))
    do = rng.standard_normal((1, 2, 9, 4))
    dq, dk, dv = OBW.attention_grads(q, k, v, do, ("causal",))
    Q, K, V = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    O = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True)
    (O * torch.tensor(do)).sum().backward()
    for a, b in ((dq, Q.grad), (dk, K.grad), (dv, V.grad)):
        assert np.abs(a - b.numpy()).max() < 1e-12


# ---- prebuilt maximum-length tables and their slices ("FlexAttention: from rules to
# fused kernels", section 5.2 for decode rows, section 2.2 for crops): block-aligned
# crops of a rule on global positions equal the rebuilt tables, decode-row slices expand
# to exactly the rule, and the crop check rejects a rule that reads the total length

SLICE_SPECS = [("causal",), ("swa", 100), ("prefix", 70), ("and", ("causal",), ("swa", 150)),
               ("or", ("swa", 60), ("prefix", 40)), ("and", ("doc",), ("causal",))]


@pytest.mark.parametrize("spec", SLICE_SPECS, ids=[str(s) for s in SLICE_SPECS])
def test_slice_block_aligned_crop_equals_rebuilt(spec):
    Lmax, bq, bk = 768, 64, 128
    doc = np.repeat(np.arange(6), [100, 200, 68, 150, 150, 100]).astype(np.int32)[None]
    src = OB.tables(spec, 1, 2, Lmax, Lmax, bq, bk, 0, doc)
    for L in (128, 256, 640):
        got = OB.slice_rows(src, 1, 2, Lmax, Lmax, bq, bk, 0, L, L, 0)
        want = OB.tables(spec, 1, 2, L, L, bq, bk, 0, doc)
        for k in got:
            assert np.array_equal(got[k], want[k]), (spec, L, k)


@pytest.mark.parametrize("spec", SLICE_SPECS, ids=[str(s) for s in SLICE_SPECS])
def test_slice_decode_rows_expand_to_the_rule(spec):
    Lmax, bq, bk = 700, 128, 64
    doc = np.repeat(np.arange(5), [130, 170, 100, 200, 100]).astype(np.int32)[None]
    src = OB.tables(spec, 1, 1, Lmax, Lmax, bq, bk, 0, doc)
    for t in (0, 63, 64, 127, 128, 300, 699):
        for ql in (1, 3):
            if t + ql > Lmax or t // bq != (t + ql - 1) // bq:
                continue
            got = OB.slice_rows(src, 1, 1, Lmax, Lmax, bq, bk, 0, ql, t + ql, t)
            # the slice's tables, expanded with the exact rule on partial blocks, give the rule
            M_hat = OB.expand(got, 1, 1, ql, t + ql, bq, bk, spec, t, doc)
            M = OM.dense(spec, ql, t + ql, t, OM.doc_row_for(doc, 0))
            assert np.array_equal(M_hat, M), (spec, t, ql)
            # and every block the rebuilt decode tables list is listed by the slice
            want = OB.tables(spec, 1, 1, ql, t + ql, bq, bk, t, doc)
            listed = lambda tab: set(tab["kv_idx"].tolist()) | set(tab["full_kv_idx"].tolist())
            assert listed(want) <= listed(got)
            assert set(want["full_kv_idx"].tolist()) >= set(got["full_kv_idx"].tolist())


def test_slice_rejects_straddling_rows():
    src = OB.tables(("causal",), 1, 1, 512, 512, 128, 128)
    with pytest.raises(ValueError):
        OB.slice_rows(src, 1, 1, 512, 512, 128, 128, 0, 2, 200, 127)      # rows 127..128
    with pytest.raises(ValueError):
        OB.slice_rows(src, 1, 1, 512, 512, 128, 128, 0, 200, 200, 64)     # 64 is not aligned
    with pytest.raises(ValueError):
        OB.slice_rows(src, 1, 1, 512, 512, 128, 128, 0, 1, 600, 100)      # keys past the prebuilt


def _crop_ok(spec_at, Lmax, lengths, bq, bk):
    """Section 2.2's whitelist check: crops of tables built at Lmax against tables rebuilt
    at each length, in block indices and in element adjacency."""
    src = OB.tables(spec_at(Lmax), 1, 1, Lmax, Lmax, bq, bk)
    for L in lengths:
        crop = OB.slice_rows(src, 1, 1, Lmax, Lmax, bq, bk, 0, L, L, 0)
        rebuilt = OB.tables(spec_at(L), 1, 1, L, L, bq, bk)
        same_idx = all(np.array_equal(crop[k], rebuilt[k]) for k in crop)
        M = OM.dense(spec_at(L), L, L)
        if not (same_idx and np.array_equal(OB.expand(crop, 1, 1, L, L, bq, bk, spec_at(L)), M)):
            return False
    return True


def test_crop_whitelist_rejects_a_length_dependent_rule(monkeypatch):
    # the pages' counterexample: a token wired to the end block of the sequence.  The rule
    # ("tail", L) lets every query see the last 64 keys of a length-L sequence, plus causal
    base = OM.evaluate

    def evaluate(spec, i, j, doc_row=None):
        if spec[0] == "tail":
            return (j >= spec[1] - 64) | (j <= i)
        return base(spec, i, j, doc_row)
    monkeypatch.setattr(OM, "evaluate", evaluate)
    assert _crop_ok(lambda L: ("causal",), 512, (128, 256, 384), 64, 64)
    assert _crop_ok(lambda L: ("swa", 90), 512, (128, 256, 384), 64, 64)
    assert not _crop_ok(lambda L: ("tail", L), 512, (128, 256, 384), 64, 64)


# ---- selector output into block tables ("FlexAttention: from rules to fused kernels",
# sections 5.2 and 6.3; "Kernels: turning logical sparsity into real speed", section 3)

from oracle import selector as OS  # noqa: E402


def test_selector_canonical_sets_hand_example():
    # range check, sort and repeat removal of one candidate row, NKB = 8
    sets = OS.canonical_sets(np.array([[5, -1, 3, 5, 99, 0, 8, 7]]), 8)
    assert [s.tolist() for s in sets] == [[0, 3, 5, 7]]
    assert [s.tolist() for s in OS.canonical_sets(np.full((2, 3), -1), 8)] == [[], []]


def test_selector_choosing_every_block_is_the_plain_rule():
    # selecting all blocks of every row reduces to the rule's own tables
    q_len = kv_len = 333
    bq, bk = 64, 32
    nqb, nkb = OB.n_blocks(q_len, bq), OB.n_blocks(kv_len, bk)
    sel = np.tile(np.arange(nkb)[::-1], (1, 2, nqb, 1))          # reversed order on purpose
    for spec in (("causal",), ("swa", 50), ("or", ("swa", 20), ("prefix", 40))):
        got = OS.tables_from_selection(spec, sel, 1, 2, q_len, kv_len, bq, bk)
        want = OB.tables(spec, 1, 2, q_len, kv_len, bq, bk)
        for k in got:
            assert np.array_equal(got[k], want[k]), (spec, k)


def test_selector_under_an_all_allowing_rule_lists_exactly_the_choice():
    # PREFIX(P >= KV_LEN) allows every pair, so each chosen block is FULL and nothing else
    rng = np.random.default_rng(0)
    q_len, kv_len, bq, bk = 200, 300, 64, 64
    nqb, nkb = OB.n_blocks(q_len, bq), OB.n_blocks(kv_len, bk)
    sel = rng.integers(-2, nkb + 2, size=(2, 1, nqb, 6))
    tab = OS.tables_from_selection(("prefix", kv_len), sel, 2, 1, q_len, kv_len, bq, bk)
    sets = OS.canonical_sets(sel, nkb)
    assert tab["kv_ptr"][-1] == 0
    for r, S in enumerate(sets):
        got = tab["full_kv_idx"][tab["full_kv_ptr"][r]:tab["full_kv_ptr"][r + 1]]
        assert got.tolist() == S.tolist()


def test_selector_mask_brute_force():
    # pair by pair: (i, j) allowed iff the rule allows it and j's block was chosen for
    # i's query block; and the tables expand back to that matrix
    rng = np.random.default_rng(1)
    q_len, kv_len, bq, bk, off = 70, 90, 16, 16, 20
    nqb, nkb = OB.n_blocks(q_len, bq), OB.n_blocks(kv_len, bk)
    sel = rng.integers(-1, nkb + 1, size=(1, 1, nqb, 4))
    spec = ("swa", 30)
    sets = OS.canonical_sets(sel, nkb)
    M = OS.selected_mask(spec, sets, 1, 0, 0, q_len, kv_len, bq, bk, off)
    for i in range(q_len):
        for j in range(kv_len):
            ig = i + off
            want = (j <= ig and ig - j < 30) and (j // bk) in set(sets[i // bq].tolist())
            assert M[i, j] == want
    tab = OS.tables_from_selection(spec, sel, 1, 1, q_len, kv_len, bq, bk, off)
    hat = np.zeros_like(M)
    for r in range(nqb):
        for c in tab["full_kv_idx"][tab["full_kv_ptr"][r]:tab["full_kv_ptr"][r + 1]]:
            hat[r * bq:(r + 1) * bq, c * bk:(c + 1) * bk] = True
        for c in tab["kv_idx"][tab["kv_ptr"][r]:tab["kv_ptr"][r + 1]]:
            sl = np.s_[r * bq:(r + 1) * bq, c * bk:(c + 1) * bk]
            hat[sl] = M[sl]
            assert M[sl].any() and not M[sl].all()
    assert np.array_equal(hat, M)
    # the q side is the transpose
    for c in range(nkb):
        rows = tab["q_idx"][tab["q_ptr"][c]:tab["q_ptr"][c + 1]].tolist()
        assert rows == [r for r in range(nqb) if c in tab["kv_idx"][tab["kv_ptr"][r]:tab["kv_ptr"][r + 1]]]


def test_work_order_is_longest_first_permutation():
    tab = {"kv_num": np.array([1, 0, 3, 1, 2, 2, 0, 5], np.int32),
           "full_kv_num": np.array([0, 4, 0, 0, 1, 0, 0, 0], np.int32)}
    # two table entries of four query blocks; lengths [1, 4, 3, 1] and [3, 2, 0, 5]
    order = OS.work_order(tab, 1, 2, 4 * 64, 64)
    assert order.tolist() == [1, 2, 3, 0, 3, 0, 1, 2]


def test_attention_oracle_accepts_a_pair_function():
    # the function form of the mask gives the same result as the rule it spells out
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 40, 16))
    k = rng.standard_normal((1, 1, 50, 16))
    v = rng.standard_normal((1, 1, 50, 16))
    O1, L1 = OA.attention(q, k, v, ("swa", 9), q_offset=10)
    O2, L2 = OA.attention(q, k, v, lambda b, h, i, j: (j <= i) & (i - j < 9), q_offset=10)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_backward_oracle_accepts_a_pair_function():
    from oracle import backward as OBW
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 2, 12, 8))
    k = rng.standard_normal((1, 1, 15, 8))
    v = rng.standard_normal((1, 1, 15, 8))
    do = rng.standard_normal((1, 2, 12, 8))
    a = OBW.attention_grads(q, k, v, do, ("swa", 5), q_offset=3)
    b = OBW.attention_grads(q, k, v, do, lambda bb, h, i, j: (j <= i) & (i - j < 5), q_offset=3)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("kind", ["alibi", "relpos"])
def test_parameter_gradients_match_finite_differences(kind):
    # gradients of the ALiBi slopes and of every relative-position table entry, against
    # central differences of the forward oracle
    from oracle import backward as OBW
    rng = np.random.default_rng(13)
    B, Hq, Hkv, ql, kl, d = 2, 2, 1, 6, 9, 3
    q = rng.standard_normal((B, Hq, ql, d))
    k = rng.standard_normal((B, Hkv, kl, d))
    v = rng.standard_normal((B, Hkv, kl, d))
    do = rng.standard_normal((B, Hq, ql, d))
    spec = ("or", ("swa", 3), ("prefix", 2))
    par = np.array([0.5, -0.3]) if kind == "alibi" else rng.standard_normal((Hq, 7))
    key = "slopes" if kind == "alibi" else "table"
    extra = {} if kind == "alibi" else {"radius": 3}
    out = OBW.attention_grads(q, k, v, do, spec, kind, q_offset=2, param_grads=True, **{key: par}, **extra)
    g = out[3]
    assert g.shape == par.shape

    def loss(pv):
        O, _ = OA.attention(q, k, v, spec, kind, q_offset=2, **{key: pv}, **extra)
        return float((O * do).sum())

    h = 1e-6
    for idx in np.ndindex(par.shape):
        pp, pm = par.copy(), par.copy()
        pp[idx] += h
        pm[idx] -= h
        fd = (loss(pp) - loss(pm)) / (2 * h)
        assert abs(fd - g[idx]) < 1e-6 * max(1.0, abs(fd)), (kind, idx, fd, g[idx])
    if kind == "relpos":
        # entries no pair reaches (here none: |i - j| spans every offset) would be zero
        assert np.abs(g).max() > 0
