"""Python binding of the C ABI: same operations, torch tensors for device memory.

``create_block_mask`` and ``forward`` only marshal arguments (tensor pointers, the
current HIP stream, the mask rule as a postfix program) and call the library.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import torch

from . import _lib as L

SCORE_KINDS = {"identity": L.FA_S_IDENTITY, "alibi": L.FA_S_ALIBI,
               "softcap": L.FA_S_SOFTCAP, "relpos": L.FA_S_RELPOS}
TABLE_NAMES = ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr", "full_kv_idx",
               "q_num", "q_ptr", "q_idx", "full_q_num", "full_q_ptr", "full_q_idx")


def compile_mask(spec):
    """Nested-tuple mask rule -> postfix list of (op, arg)."""
    out = []

    def walk(s):
        op = s[0]
        if op == "causal":
            out.append((L.FA_M_CAUSAL, 0))
        elif op == "swa":
            out.append((L.FA_M_SWA, int(s[1])))
        elif op == "doc":
            out.append((L.FA_M_DOC, 0))
        elif op == "prefix":
            out.append((L.FA_M_PREFIX, int(s[1])))
        elif op in ("and", "or"):
            walk(s[1])
            walk(s[2])
            out.append((L.FA_M_AND if op == "and" else L.FA_M_OR, 0))
        else:
            raise ValueError(f"unknown mask node {op!r}")

    walk(spec)
    return out


def _stream(stream):
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


class BlockMask:
    """Caller-owned block tables (twelve int32 device tensors) plus their descriptor."""

    def __init__(self, desc, tensors, keep):
        self.desc = desc
        self.tensors = tensors
        self._keep = keep        # doc-ID tensor and workspace stay alive with the tables

    def __getattr__(self, name):
        t = self.__dict__.get("tensors")
        if t is not None and name in t:
            return t[name]
        raise AttributeError(name)

    @property
    def q_len(self):
        return self.desc.q_len

    @property
    def kv_len(self):
        return self.desc.kv_len

    def compact(self):
        """Host copies of the tables trimmed to their used length (numpy int32)."""
        out = {}
        for side in ("kv", "full_kv", "q", "full_q"):
            if f"{side}_num" not in self.tensors:
                continue
            ptr = self.tensors[f"{side}_ptr"].cpu().numpy()
            num = self.tensors[f"{side}_num"][: len(ptr) - 1].cpu().numpy()   # allocated >= 1
            idx = self.tensors[f"{side}_idx"][: int(ptr[-1])].cpu().numpy()
            out[f"{side}_num"], out[f"{side}_ptr"], out[f"{side}_idx"] = num, ptr, idx
        if "order" in self.tensors:
            out["order"] = self.tensors["order"][: len(out["kv_ptr"]) - 1].cpu().numpy()
        return out


def block_mask_desc(mask, B, H, q_len, kv_len, block_q=128, block_kv=128, q_offset=0,
                    doc_ids: Optional[torch.Tensor] = None):
    prog = compile_mask(mask)
    d = L.fa_block_mask()
    d.mask.n = len(prog)
    for i, (op, arg) in enumerate(prog[: L.FA_MASK_MAX_NODES]):
        d.mask.node[i].op = op
        d.mask.node[i].arg = arg
    if len(prog) > L.FA_MASK_MAX_NODES:
        d.mask.n = len(prog)   # the library rejects it
    if doc_ids is not None:
        if doc_ids.dim() == 1:
            doc_ids = doc_ids[None]
        d.mask.doc_ids = doc_ids.data_ptr()
        d.mask.doc_batch = doc_ids.shape[0]
        d.mask.doc_len = doc_ids.shape[1]
    else:
        d.mask.doc_batch = 1
    d.B, d.H = int(B), int(H)
    d.q_len, d.kv_len, d.q_offset = int(q_len), int(kv_len), int(q_offset)
    d.block_q, d.block_kv = int(block_q), int(block_kv)
    return d, doc_ids


def block_mask_sizes(desc):
    lib = L.load()
    rows, cols, cap = C.c_int64(), C.c_int64(), C.c_int64()
    ws = C.c_size_t()
    L.check(lib.fa_block_mask_sizes(C.byref(desc), C.byref(rows), C.byref(cols),
                                    C.byref(cap), C.byref(ws)))
    return rows.value, cols.value, cap.value, ws.value


def _alloc_tables(rows, cols, cap, device, q_side=True, order=False):
    tables = {}
    sides = (("kv", rows), ("full_kv", rows)) + ((("q", cols), ("full_q", cols)) if q_side else ())
    for side, n in sides:
        tables[f"{side}_num"] = torch.empty(max(n, 1), dtype=torch.int32, device=device)
        tables[f"{side}_ptr"] = torch.empty(n + 1, dtype=torch.int32, device=device)
        tables[f"{side}_idx"] = torch.empty(max(cap, 1), dtype=torch.int32, device=device)
    if order:
        tables["order"] = torch.empty(max(rows, 1), dtype=torch.int32, device=device)
    return tables


def _set_tables(d, tables):
    for name in TABLE_NAMES + ("order",):
        setattr(d, name, tables[name].data_ptr() if name in tables else None)


def create_block_mask(mask, B, H, q_len, kv_len, block_q=128, block_kv=128, q_offset=0,
                      doc_ids: Optional[torch.Tensor] = None, device="cuda", stream=None,
                      tables=None, workspace=None, order=False, q_side=True):
    """Build the block tables on the GPU.  ``mask`` is a nested tuple rule
    (see workloads); ``doc_ids`` an int32 device tensor [doc_batch, doc_len];
    ``order`` also writes the longest-row-first work order; ``q_side=False`` writes only
    the kv side (all a forward reads; the backward needs both)."""
    lib = L.load()
    d, doc_ids = block_mask_desc(mask, B, H, q_len, kv_len, block_q, block_kv, q_offset, doc_ids)
    rows, cols, cap, ws = block_mask_sizes(d)
    if tables is None:
        tables = _alloc_tables(rows, cols, cap, device, q_side=q_side, order=order)
    _set_tables(d, tables)
    if workspace is None:
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
    L.check(lib.fa_create_block_mask(C.byref(d), C.c_void_p(workspace.data_ptr()),
                                     workspace.numel(), _stream(stream)))
    return BlockMask(d, tables, (doc_ids, workspace))


def slice_block_mask(src: BlockMask, q_len, kv_len, q_offset, q_side=True, stream=None, tables=None,
                     workspace=None, order=False):
    """Tables for rows [q_offset, q_offset + q_len) and keys [0, kv_len) cut out of the
    prebuilt ``src`` (fa_block_mask_slice); ``q_side=False`` writes only the kv side."""
    lib = L.load()
    d = L.fa_block_mask.from_buffer_copy(src.desc)
    d.q_len, d.kv_len, d.q_offset = int(q_len), int(kv_len), int(q_offset)
    rows, cols, cap, ws = block_mask_sizes(d)
    device = src.tensors["kv_num"].device
    if tables is None:
        tables = _alloc_tables(rows, cols, cap, device, q_side=q_side, order=order)
    _set_tables(d, tables)
    if workspace is None:
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=device)
    L.check(lib.fa_block_mask_slice(C.byref(src.desc), C.byref(d), C.c_void_p(workspace.data_ptr()),
                                    workspace.numel(), _stream(stream)))
    return BlockMask(d, tables, (src._keep[0], workspace))


def block_mask_from_indices(sel: torch.Tensor, mask, B, H, q_len, kv_len, block_q=128, block_kv=128, q_offset=0,
                            doc_ids: Optional[torch.Tensor] = None, stream=None, tables=None, workspace=None,
                            order=False, q_side=True):
    """Block tables from selector output (fa_block_mask_from_indices): ``sel`` is an int32
    device tensor [B, H, NQB, k] of KV block indices per query block (values outside
    [0, NKB) are dropped, repeats count once); ``mask`` is the rule applied inside the
    chosen blocks; ``q_side=False`` writes only the kv side (enough for the forward)."""
    lib = L.load()
    d, doc_ids = block_mask_desc(mask, B, H, q_len, kv_len, block_q, block_kv, q_offset, doc_ids)
    rows, cols, cap, ws = block_mask_sizes(d)
    if sel.dtype != torch.int32 or not sel.is_contiguous() or sel.dim() != 4 or \
            tuple(sel.shape[:3]) != (int(B), int(H), -(-int(q_len) // int(block_q))):
        raise ValueError("sel must be a contiguous int32 tensor [B, H, NQB, k]")
    if tables is None:
        tables = _alloc_tables(rows, cols, cap, sel.device, q_side=q_side, order=order)
    _set_tables(d, tables)
    if workspace is None:
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=sel.device)
    L.check(lib.fa_block_mask_from_indices(C.byref(d), C.c_void_p(sel.data_ptr()), int(sel.shape[3]),
                                           C.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(stream)))
    return BlockMask(d, tables, (doc_ids, workspace, sel))


def forward_args(q, k, v, block_mask: BlockMask, score="identity", softcap=0.0,
                 alibi_slopes=None, relpos=None, relpos_radius=0, scale=None, out=None,
                 lse=None, kv_len=None):
    B, Hq, q_len, d = q.shape
    Hkv = k.shape[1]
    kv_len = k.shape[2] if kv_len is None else int(kv_len)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor")
    if out is None:
        out = torch.empty(B, Hq, q_len, d, dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty(B, Hq, q_len, dtype=torch.float32, device=q.device)
    a = L.fa_fwd_args()
    a.q, a.k, a.v, a.o, a.lse = q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr()
    a.B, a.Hq, a.Hkv, a.d = B, Hq, Hkv, d
    a.q_len, a.kv_len = q_len, kv_len
    a.scale = 0.0 if scale is None else float(scale)
    a.score.kind = SCORE_KINDS[score]
    a.score.softcap = float(softcap or 0.0)
    a.score.alibi_slopes = None if alibi_slopes is None else alibi_slopes.data_ptr()
    a.score.relpos = None if relpos is None else relpos.data_ptr()
    a.score.relpos_radius = int(relpos_radius)
    a.bm = C.pointer(block_mask.desc)
    return a, out, lse


def forward_workspace_size(args) -> int:
    lib = L.load()
    n = C.c_size_t()
    L.check(lib.fa_forward_workspace_size(C.byref(args), C.byref(n)))
    return n.value


def backward(q, k, v, out, lse, dout, block_mask: BlockMask, score="identity", softcap=0.0,
             alibi_slopes=None, relpos=None, relpos_radius=0, scale=None, dq=None, dk=None, dv=None,
             workspace=None, stream=None, param_grad=False, store_grads=True):
    """dQ [B,Hq,q_len,d], dK and dV [B,Hkv,kv_len,d] (fp32) of the forward that produced
    out and lse, for the output gradient dout (bf16, same shape as out).  With
    ``param_grad`` a fourth result is the gradient of the ALiBi slopes [Hq] or of the
    relative-position table [Hq, 2R+1] (fp32).  ``store_grads`` gives the call the
    workspace in which the dK/dV pass stores the per-pair gradients for the dQ pass
    (where the library offers it); without it the dQ pass recomputes them."""
    lib = L.load()
    if dout.dtype != torch.bfloat16 or not dout.is_contiguous() or dout.shape != out.shape:
        raise ValueError("dout must be a contiguous bfloat16 tensor shaped like out")
    a, _, _ = forward_args(q, k, v, block_mask, score, softcap, alibi_slopes, relpos, relpos_radius,
                           scale, out, lse)
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.shape != ref.shape:
            raise ValueError(f"{name} must be a contiguous float32 tensor shaped like its input")
    ba = L.fa_bwd_args()
    ba.fwd = C.pointer(a)
    ba.dout = dout.data_ptr()
    ba.dq, ba.dk, ba.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    gpar = None
    if param_grad:
        if score == "alibi":
            gpar = torch.empty(q.shape[1], dtype=torch.float32, device=q.device)
            ba.dslopes = gpar.data_ptr()
        elif score == "relpos":
            gpar = torch.empty((q.shape[1], 2 * int(relpos_radius) + 1), dtype=torch.float32, device=q.device)
            ba.dtable = gpar.data_ptr()
        else:
            raise ValueError("param_grad needs the alibi or relpos score")
    n = C.c_size_t()
    size_fn = lib.fa_backward_workspace_size if store_grads else lib.fa_backward_workspace_min_size
    L.check(size_fn(C.byref(ba), C.byref(n)))
    if n.value > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < n.value:
            workspace = torch.empty(n.value, dtype=torch.uint8, device=q.device)
        ba.workspace = workspace.data_ptr()
        ba.ws_bytes = n.value   # exactly the size asked for: a larger buffer may not pick the path
    L.check(lib.fa_backward(C.byref(ba), _stream(stream)))
    return (dq, dk, dv, gpar) if param_grad else (dq, dk, dv)


def forward_paged(q, k_cache, v_cache, page_table, kv_len, block_mask: BlockMask, score="identity",
                  softcap=0.0, alibi_slopes=None, relpos=None, relpos_radius=0, scale=None, out=None,
                  lse=None, workspace=None, stream=None):
    """Short-query forward over paged caches k_cache/v_cache bf16 [num_pages, Hkv, page_size, d]
    with page_table int32 [B, pt_stride] (logical page -> physical page) and logical length
    kv_len.  Returns O [B,Hq,q_len,d] bf16 and LSE [B,Hq,q_len] fp32."""
    lib = L.load()
    num_pages, _, page_size, _ = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    if page_table.dtype != torch.int32 or page_table.dim() != 2 or not page_table.is_contiguous():
        raise ValueError("page_table must be a contiguous int32 [B, pt_stride] tensor")
    a, out, lse = forward_args(q, k_cache, v_cache, block_mask, score, softcap, alibi_slopes, relpos,
                               relpos_radius, scale, out, lse, kv_len=kv_len)
    kv = L.fa_paged_kv()
    kv.page_table = page_table.data_ptr()
    kv.pt_stride = page_table.shape[1]
    kv.page_size = page_size
    kv.num_pages = num_pages
    need = forward_workspace_size(a)
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        a.workspace = workspace.data_ptr()
        a.ws_bytes = workspace.numel() * workspace.element_size()
    L.check(lib.fa_forward_paged(C.byref(a), C.byref(kv), _stream(stream)))
    return out, lse


def forward(q, k, v, block_mask: BlockMask, score="identity", softcap=0.0, alibi_slopes=None,
            relpos=None, relpos_radius=0, scale=None, out=None, lse=None, workspace=None,
            stream=None):
    """O [B,Hq,q_len,d] bf16 and LSE [B,Hq,q_len] fp32."""
    lib = L.load()
    a, out, lse = forward_args(q, k, v, block_mask, score, softcap, alibi_slopes, relpos,
                               relpos_radius, scale, out, lse)
    need = forward_workspace_size(a)
    if need > 0:
        if workspace is None or workspace.numel() * workspace.element_size() < need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        a.workspace = workspace.data_ptr()
        a.ws_bytes = workspace.numel() * workspace.element_size()
    L.check(lib.fa_forward(C.byref(a), _stream(stream)))
    return out, lse


def forward_noalloc(q, k, v, block_mask: BlockMask, out, lse, score="identity", softcap=0.0,
                    alibi_slopes=None, relpos=None, relpos_radius=0, scale=None, stream=None):
    """fa_forward_noalloc: the forward into the caller's ``out`` [B,Hq,q_len,d] bf16 and
    ``lse`` [B,Hq,q_len] fp32, with the split-KV partial states in the library's static
    scratch (no workspace; the call allocates nothing)."""
    lib = L.load()
    a, out, lse = forward_args(q, k, v, block_mask, score, softcap, alibi_slopes, relpos,
                               relpos_radius, scale, out, lse)
    L.check(lib.fa_forward_noalloc(C.byref(a), _stream(stream)))
    return out, lse
