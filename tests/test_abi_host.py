"""C-ABI checks that need no GPU: the library loads, exports every function that
include/fa.h declares, the ctypes structures match the C layout, and argument
validation rejects bad inputs before any device work (no compute calls)."""
import ctypes as C
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    from block_sparse_programmable_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        from block_sparse_programmable_amd import build
        build.build()
    return L.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(fa_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    from block_sparse_programmable_amd import _lib as L
    names = declared_functions()
    assert set(names) == set(L.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


LAYOUT_C = r"""
#include <stdio.h>
#include <stddef.h>
#include "fa.h"
#define P(T, F) printf(#T "." #F " %zu\n", offsetof(T, F));
int main(void) {
  printf("fa_mask_desc %zu\nfa_block_mask %zu\nfa_score_desc %zu\nfa_fwd_args %zu\nfa_bwd_args %zu\n",
         sizeof(fa_mask_desc), sizeof(fa_block_mask), sizeof(fa_score_desc), sizeof(fa_fwd_args),
         sizeof(fa_bwd_args));
  P(fa_mask_desc, doc_ids) P(fa_mask_desc, doc_batch) P(fa_mask_desc, doc_len)
  P(fa_block_mask, B) P(fa_block_mask, q_len) P(fa_block_mask, q_offset) P(fa_block_mask, block_kv)
  P(fa_block_mask, kv_num) P(fa_block_mask, full_q_idx) P(fa_block_mask, order)
  P(fa_score_desc, softcap) P(fa_score_desc, relpos) P(fa_score_desc, relpos_radius)
  P(fa_fwd_args, lse) P(fa_fwd_args, d) P(fa_fwd_args, q_len) P(fa_fwd_args, scale)
  P(fa_fwd_args, score) P(fa_fwd_args, bm) P(fa_fwd_args, ws_bytes)
  P(fa_bwd_args, ws_bytes) P(fa_bwd_args, dslopes) P(fa_bwd_args, dtable)
  return 0;
}
"""


def test_struct_layout_matches_header():
    from block_sparse_programmable_amd import _lib as L
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "layout.c")
        exe = os.path.join(d, "layout")
        open(src, "w").write(LAYOUT_C)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(l.rsplit(" ", 1) for l in lines if l)
    structs = {"fa_mask_desc": L.fa_mask_desc, "fa_block_mask": L.fa_block_mask,
               "fa_score_desc": L.fa_score_desc, "fa_fwd_args": L.fa_fwd_args, "fa_bwd_args": L.fa_bwd_args}
    for k, v in got.items():
        if "." in k:
            s, f = k.split(".")
            assert getattr(structs[s], f).offset == int(v), k
        else:
            assert C.sizeof(structs[k]) == int(v), k


def _bm(L, **kw):
    from block_sparse_programmable_amd.api import block_mask_desc
    args = dict(mask=("causal",), B=1, H=1, q_len=256, kv_len=256, block_q=128, block_kv=128)
    args.update(kw)
    d, _ = block_mask_desc(**args)
    return d


def test_block_mask_sizes(lib):
    from block_sparse_programmable_amd import _lib as L
    from block_sparse_programmable_amd.api import block_mask_sizes
    d = _bm(L, B=2, H=3, q_len=300, kv_len=1000, block_q=64, block_kv=128)
    rows, cols, cap, ws = block_mask_sizes(d)
    assert rows == 2 * 3 * 5 and cols == 2 * 3 * 8 and cap == 2 * 3 * 5 * 8 and ws > 0
    # table writers take any power-of-two block from 1 to 128 (the worked 2 x 2 example)
    d = _bm(L, q_len=8, kv_len=8, block_q=2, block_kv=2)
    rows, cols, cap, ws = block_mask_sizes(d)
    assert (rows, cols, cap) == (4, 4, 16) and ws > 0


def _status(fn, *a):
    return fn(*a)


def test_validation_errors_before_any_launch(lib):
    from block_sparse_programmable_amd import _lib as L
    # builder: bad block size, bad program, missing doc IDs, missing tables, workspace
    d = _bm(L, block_q=96)
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_UNSUPPORTED
    assert b"powers of two from 1 to 128" in lib.fa_last_error_message()
    for bad in (0, 256, 3):
        d = _bm(L, block_kv=bad)
        assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_UNSUPPORTED
    # 32-bit list positions: B * H * NQB * NKB must stay below 2^31
    d = _bm(L, B=4, H=2, q_len=2 ** 15, kv_len=2 ** 15, block_q=1, block_kv=1)
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_SHAPE
    assert b"32-bit" in lib.fa_last_error_message()
    d = _bm(L)
    d.mask.n = 2                                  # causal, causal: two values left
    d.mask.node[1].op = L.FA_M_CAUSAL
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_MASK_SPEC
    d = _bm(L, mask=("swa", 0))
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_MASK_SPEC
    d = _bm(L, mask=("prefix", -1))
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_MASK_SPEC
    d = _bm(L)
    d.mask.node[0].op = 99
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_MASK_SPEC
    d = _bm(L)
    d.mask.n = 1
    d.mask.node[0].op = L.FA_M_AND
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_MASK_SPEC
    d = _bm(L, mask=("doc",))
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_NULL
    d = _bm(L)
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_NULL   # no tables
    for name in ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx"):
        setattr(d, name, 0x1000)                  # never dereferenced: rejected first
    # the q side: all six pointers or none
    d.q_num = 0x1000
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_NULL
    assert b"q-side" in lib.fa_last_error_message()
    d.q_num = None
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_WORKSPACE   # kv side only
    for name in ("q_num", "q_ptr", "q_idx", "full_q_num", "full_q_ptr", "full_q_idx"):
        setattr(d, name, 0x1000)
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_WORKSPACE
    assert lib.fa_create_block_mask(C.byref(d), C.c_void_p(0x2000), 1, None) == L.FA_ERR_WORKSPACE
    d = _bm(L, q_len=-1)
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_SHAPE
    d = _bm(L, q_offset=2 ** 31 - 10, q_len=100)
    assert lib.fa_create_block_mask(C.byref(d), None, 0, None) == L.FA_ERR_SHAPE


def _fwd(L, bm, **kw):
    a = L.fa_fwd_args()
    a.q = a.k = a.v = a.o = a.lse = 0x1000
    a.B, a.Hq, a.Hkv, a.d = 1, 4, 2, 128
    a.q_len, a.kv_len = 256, 256
    a.bm = C.pointer(bm)
    for k, v in kw.items():
        if k.startswith("score_"):
            setattr(a.score, k[6:], v)
        else:
            setattr(a, k, v)
    return a


def test_forward_validation(lib):
    from block_sparse_programmable_amd import _lib as L
    bm = _bm(L)
    for name in ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx"):
        setattr(bm, name, 0x1000)
    F = lambda a: lib.fa_forward(C.byref(a), None)
    assert lib.fa_forward(None, None) == L.FA_ERR_NULL
    assert F(_fwd(L, bm, q=None)) == L.FA_ERR_NULL
    assert F(_fwd(L, bm, d=96)) == L.FA_ERR_UNSUPPORTED
    assert F(_fwd(L, bm, Hkv=3)) == L.FA_ERR_SHAPE
    assert F(_fwd(L, bm, q_len=128)) == L.FA_ERR_MASK_MISMATCH
    assert F(_fwd(L, bm, kv_len=512)) == L.FA_ERR_MASK_MISMATCH
    assert F(_fwd(L, bm, score_kind=7)) == L.FA_ERR_UNSUPPORTED
    assert F(_fwd(L, bm, score_kind=L.FA_S_ALIBI)) == L.FA_ERR_NULL
    assert F(_fwd(L, bm, score_kind=L.FA_S_SOFTCAP, score_softcap=0.0)) == L.FA_ERR_UNSUPPORTED
    assert F(_fwd(L, bm, score_kind=L.FA_S_RELPOS)) == L.FA_ERR_NULL
    assert F(_fwd(L, bm, score_kind=L.FA_S_RELPOS, score_relpos=0x1000,
                  score_relpos_radius=-1)) == L.FA_ERR_UNSUPPORTED
    # 2R + 1 table entries per head must stay below 2^31
    assert F(_fwd(L, bm, score_kind=L.FA_S_RELPOS, score_relpos=0x1000,
                  score_relpos_radius=2 ** 30)) == L.FA_ERR_UNSUPPORTED
    assert b"relpos_radius" in lib.fa_last_error_message()
    # tables of blocks below 64 are valid tables but not a forward geometry
    for bq, bk in ((32, 128), (128, 16), (2, 2)):
        bms = _bm(L, block_q=bq, block_kv=bk)
        for name in ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx"):
            setattr(bms, name, 0x1000)
        assert F(_fwd(L, bms)) == L.FA_ERR_UNSUPPORTED, (bq, bk)
        assert b"64- or 128-blocks" in lib.fa_last_error_message()
    assert F(_fwd(L, bm, scale=float("nan"))) == L.FA_ERR_SHAPE
    # rows move in 16-byte chunks: q, k, v, o 16-byte aligned, lse 4-byte aligned
    for name in ("q", "k", "v", "o"):
        assert F(_fwd(L, bm, **{name: 0x1008})) == L.FA_ERR_SHAPE, name
        assert b"16-byte aligned" in lib.fa_last_error_message()
    assert F(_fwd(L, bm, lse=0x1002)) == L.FA_ERR_SHAPE
    # a decode step's split-KV workspace must be 16-byte aligned
    bmd = _bm(L, q_len=1, kv_len=4096, q_offset=4095)
    for name in ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx"):
        setattr(bmd, name, 0x1000)
    dec = _fwd(L, bmd, q_len=1, kv_len=4096)
    n = C.c_size_t(0)
    assert lib.fa_forward_workspace_size(C.byref(dec), C.byref(n)) == L.FA_OK and n.value > 0
    dec.workspace, dec.ws_bytes = 0x1008, n.value
    assert F(dec) == L.FA_ERR_WORKSPACE
    assert b"16-byte aligned" in lib.fa_last_error_message()
    bm2 = _bm(L, B=3)
    for name in ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx"):
        setattr(bm2, name, 0x1000)
    assert F(_fwd(L, bm2)) == L.FA_ERR_MASK_MISMATCH
    bm3 = _bm(L, H=2)
    for name in ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx"):
        setattr(bm3, name, 0x1000)
    assert F(_fwd(L, bm3)) == L.FA_ERR_MASK_MISMATCH
    # the no-allocation forward validates exactly like fa_forward, before any GPU work
    N = lambda a: lib.fa_forward_noalloc(C.byref(a), None)
    assert lib.fa_forward_noalloc(None, None) == L.FA_ERR_NULL
    assert N(_fwd(L, bm, q=None)) == L.FA_ERR_NULL
    assert N(_fwd(L, bm, d=96)) == L.FA_ERR_UNSUPPORTED
    assert N(_fwd(L, bm, q_len=128)) == L.FA_ERR_MASK_MISMATCH
    assert N(_fwd(L, bm2)) == L.FA_ERR_MASK_MISMATCH
    # paged caches: argument checks, and the paged cache is only read by the short-query path
    P = lambda a, kv: lib.fa_forward_paged(C.byref(a), C.byref(kv), None)
    kv = L.fa_paged_kv(page_table=0x1000, pt_stride=16, page_size=16, num_pages=4)
    assert lib.fa_forward_paged(None, C.byref(kv), None) == L.FA_ERR_NULL
    assert P(_fwd(L, bm), L.fa_paged_kv(page_table=None, pt_stride=16, page_size=16, num_pages=4)) == L.FA_ERR_NULL
    for ps in (8, 24, 1 << 17):
        assert P(_fwd(L, bm), L.fa_paged_kv(page_table=0x1000, pt_stride=64, page_size=ps,
                                            num_pages=4)) == L.FA_ERR_UNSUPPORTED
    assert P(_fwd(L, bm), L.fa_paged_kv(page_table=0x1000, pt_stride=15, page_size=16,
                                        num_pages=4)) == L.FA_ERR_SHAPE      # 256 keys need 16
    assert P(_fwd(L, bm), L.fa_paged_kv(page_table=0x1000, pt_stride=16, page_size=16,
                                        num_pages=0)) == L.FA_ERR_SHAPE
    assert P(_fwd(L, bm), kv) == L.FA_ERR_UNSUPPORTED                          # prefill shape
    assert b"short-query" in lib.fa_last_error_message()
    # backward: needs dout, the gradient buffers and the q-side tables; workspace rules
    fwd = _fwd(L, bm)
    Bk = lambda **kw: L.fa_bwd_args(fwd=C.pointer(fwd), **kw)
    assert lib.fa_backward(None, None) == L.FA_ERR_NULL
    assert lib.fa_backward(C.byref(Bk(dout=0x1000, dq=0x1000, dk=0x1000)), None) == L.FA_ERR_NULL
    for name in ("q_num", "full_q_idx"):
        saved = getattr(bm, name)
        setattr(bm, name, None)
        assert lib.fa_backward(C.byref(Bk(dout=0x1000, dq=0x1000, dk=0x1000, dv=0x1000)), None) == L.FA_ERR_NULL
        setattr(bm, name, saved)
    for name in ("q_num", "q_ptr", "q_idx", "full_q_num", "full_q_ptr", "full_q_idx"):
        setattr(bm, name, 0x1000)
    ok = Bk(dout=0x1000, dq=0x1000, dk=0x1000, dv=0x1000)
    n = C.c_size_t(0)
    assert lib.fa_backward_workspace_min_size(C.byref(ok), C.byref(n)) == L.FA_OK
    assert n.value == 2 * 1 * 4 * 256 * 4                             # two fp32 values per row
    full = C.c_size_t(0)
    assert lib.fa_backward_workspace_size(C.byref(ok), C.byref(full)) == L.FA_OK
    # plus the stored per-pair gradients: B * Hq * NQB * NKB tiles of 128 x 128 bf16
    assert full.value == n.value + 1 * 4 * 2 * 2 * 128 * 128 * 2
    assert lib.fa_backward(C.byref(ok), None) == L.FA_ERR_WORKSPACE
    ok.workspace, ok.ws_bytes = 0x1010, n.value
    assert lib.fa_backward(C.byref(ok), None) == L.FA_ERR_WORKSPACE    # misaligned
    for name in ("dout", "dq", "dk", "dv"):
        kw = dict(dout=0x1000, dq=0x1000, dk=0x1000, dv=0x1000)
        kw[name] = 0x1004
        assert lib.fa_backward(C.byref(Bk(**kw)), None) == L.FA_ERR_SHAPE, name
    # parameter gradients: only for their own score kind, table radius <= 1024
    assert lib.fa_backward(C.byref(Bk(dout=0x1000, dq=0x1000, dk=0x1000, dv=0x1000, dslopes=0x2000)),
                           None) == L.FA_ERR_UNSUPPORTED                 # identity score
    rp = _fwd(L, bm, score_kind=L.FA_S_RELPOS, score_relpos=0x3000, score_relpos_radius=2000)
    assert lib.fa_backward(C.byref(L.fa_bwd_args(fwd=C.pointer(rp), dout=0x1000, dq=0x1000, dk=0x1000,
                                                 dv=0x1000, dtable=0x2000)), None) == L.FA_ERR_UNSUPPORTED
    assert b"radius" in lib.fa_last_error_message()
    bad = _fwd(L, bm, d=96)                                           # forward checks apply
    assert lib.fa_backward(C.byref(L.fa_bwd_args(fwd=C.pointer(bad), dout=0x1000, dq=0x1000, dk=0x1000,
                                                 dv=0x1000)), None) == L.FA_ERR_UNSUPPORTED
    bm.kv_idx = None
    assert F(_fwd(L, bm)) == L.FA_ERR_NULL
    for s in range(8):
        assert lib.fa_status_string(s)


def test_compile_mask_postfix():
    from block_sparse_programmable_amd import _lib as L
    from block_sparse_programmable_amd.api import compile_mask
    prog = compile_mask(("and", ("doc",), ("or", ("swa", 7), ("prefix", 3))))
    assert prog == [(L.FA_M_DOC, 0), (L.FA_M_SWA, 7), (L.FA_M_PREFIX, 3), (L.FA_M_OR, 0), (L.FA_M_AND, 0)]


def test_slice_validation(lib):
    from block_sparse_programmable_amd import _lib as L
    names = ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx",
             "q_num", "q_ptr", "q_idx", "full_q_num", "full_q_ptr", "full_q_idx")

    def tabs(d, which=names, base=0x1000):
        for i, n in enumerate(which):
            setattr(d, n, base + 0x100 * i)       # never dereferenced: every case is rejected first
        return d
    src = tabs(_bm(L, q_len=4096, kv_len=4096, block_q=128, block_kv=128))
    ok_dst = dict(q_len=1, kv_len=1000, q_offset=999, block_q=128, block_kv=128)
    assert lib.fa_block_mask_slice(None, None, None, 0, None) == L.FA_ERR_NULL
    # past the prebuilt length: rows and keys
    d = tabs(_bm(L, **dict(ok_dst, q_offset=4096, kv_len=4097)), base=0x9000)
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), None, 0, None) == L.FA_ERR_SHAPE
    assert b"prebuilt" in lib.fa_last_error_message()
    d = tabs(_bm(L, **dict(ok_dst, kv_len=5000)), base=0x9000)
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), None, 0, None) == L.FA_ERR_SHAPE
    # rows straddling two prebuilt query blocks, and an unaligned multi-block slice
    d = tabs(_bm(L, **dict(ok_dst, q_len=2, q_offset=127)), base=0x9000)
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), None, 0, None) == L.FA_ERR_SHAPE
    d = tabs(_bm(L, **dict(ok_dst, q_len=300, q_offset=64)), base=0x9000)
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), None, 0, None) == L.FA_ERR_SHAPE
    # another rule, other block sizes, other extents
    d = tabs(_bm(L, **dict(ok_dst, mask=("swa", 64))), base=0x9000)
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), None, 0, None) == L.FA_ERR_MASK_MISMATCH
    d = tabs(_bm(L, **dict(ok_dst, block_q=64)), base=0x9000)
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), None, 0, None) == L.FA_ERR_MASK_MISMATCH
    d = tabs(_bm(L, **dict(ok_dst, H=2)), base=0x9000)
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), None, 0, None) == L.FA_ERR_MASK_MISMATCH
    sw = tabs(_bm(L, mask=("swa", 64), q_len=4096, kv_len=4096))
    d = tabs(_bm(L, **dict(ok_dst, mask=("swa", 65))), base=0x9000)
    assert lib.fa_block_mask_slice(C.byref(sw), C.byref(d), None, 0, None) == L.FA_ERR_MASK_MISMATCH
    # missing tables: dst kv side, a partial q side, src q side for a q-side slice
    d = _bm(L, **ok_dst)
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), None, 0, None) == L.FA_ERR_NULL
    d = tabs(_bm(L, **ok_dst), which=names[:7], base=0x9000)
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), None, 0, None) == L.FA_ERR_NULL
    assert b"all set or all NULL" in lib.fa_last_error_message()
    # workspace missing, short or misaligned
    d = tabs(_bm(L, **ok_dst), base=0x9000)
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), None, 0, None) == L.FA_ERR_WORKSPACE
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), C.c_void_p(0x20000), 1, None) == L.FA_ERR_WORKSPACE
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), C.c_void_p(0x20008), 1 << 20, None) == L.FA_ERR_WORKSPACE
    # malformed geometry on either side
    d = tabs(_bm(L, **dict(ok_dst, block_kv=96)), base=0x9000)
    assert lib.fa_block_mask_slice(C.byref(src), C.byref(d), None, 0, None) == L.FA_ERR_UNSUPPORTED


def test_from_indices_and_order_validation(lib):
    from block_sparse_programmable_amd import _lib as L
    names = ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx",
             "q_num", "q_ptr", "q_idx", "full_q_num", "full_q_ptr", "full_q_idx")

    def tabs(d, which=names):
        for i, n in enumerate(which):
            setattr(d, n, 0x1000 + 0x100 * i)      # never dereferenced: every case is rejected first
        return d
    sel = C.c_void_p(0x80000)
    assert lib.fa_block_mask_from_indices(None, sel, 4, None, 0, None) == L.FA_ERR_NULL
    d = _bm(L)
    assert lib.fa_block_mask_from_indices(C.byref(d), sel, 4, None, 0, None) == L.FA_ERR_NULL   # no tables
    d = tabs(_bm(L), which=names[:8])
    assert lib.fa_block_mask_from_indices(C.byref(d), sel, 4, None, 0, None) == L.FA_ERR_NULL   # half a q side
    d = tabs(_bm(L))
    assert lib.fa_block_mask_from_indices(C.byref(d), sel, -1, None, 0, None) == L.FA_ERR_SHAPE
    assert lib.fa_block_mask_from_indices(C.byref(d), None, 4, None, 0, None) == L.FA_ERR_NULL
    assert lib.fa_block_mask_from_indices(C.byref(d), sel, 4, None, 0, None) == L.FA_ERR_WORKSPACE
    assert lib.fa_block_mask_from_indices(C.byref(d), sel, 4, C.c_void_p(0x20004), 1 << 20, None) == \
        L.FA_ERR_WORKSPACE
    d = tabs(_bm(L, mask=("swa", 0)))
    assert lib.fa_block_mask_from_indices(C.byref(d), sel, 4, None, 0, None) == L.FA_ERR_MASK_SPEC
    # a work order is limited to 4096 query blocks, for every writer and the forward
    d = tabs(_bm(L, q_len=4097 * 64, kv_len=64, block_q=64, block_kv=64))
    d.order = 0x7000
    assert lib.fa_block_mask_from_indices(C.byref(d), sel, 4, C.c_void_p(0x20000), 1 << 30, None) == \
        L.FA_ERR_UNSUPPORTED
    assert lib.fa_create_block_mask(C.byref(d), C.c_void_p(0x20000), 1 << 30, None) == L.FA_ERR_UNSUPPORTED
    a = _fwd(L, d)
    a.q_len, a.kv_len = d.q_len, d.kv_len
    assert lib.fa_forward(C.byref(a), None) == L.FA_ERR_UNSUPPORTED
    assert b"work order" in lib.fa_last_error_message()


def test_paged_per_head_tables_short_queries_only(lib):
    from block_sparse_programmable_amd import _lib as L
    # per-head tables (H = Hq = 4) under GQA (Hkv = 2): each query head walks its own row,
    # so up to 16 query rows fit the split-KV path, the only paged one; 17 do not
    bm = _bm(L, H=4, q_len=17, kv_len=1000, q_offset=983)
    for i, n in enumerate(("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx")):
        setattr(bm, n, 0x1000 + 0x100 * i)
    a = _fwd(L, bm)
    a.q_len, a.kv_len = 17, 1000
    kv = L.fa_paged_kv()
    kv.page_table, kv.pt_stride, kv.page_size, kv.num_pages = 0x5000, 63, 16, 1000
    assert lib.fa_forward_paged(C.byref(a), C.byref(kv), None) == L.FA_ERR_UNSUPPORTED
    assert b"short-query path" in lib.fa_last_error_message()
