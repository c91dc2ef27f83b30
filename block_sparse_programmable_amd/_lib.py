"""ctypes mirror of include/fa.h and the loader of libfa.so.

Argument marshalling only: every computation happens in the HIP library.  Importing
this module raises if the library has not been built; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfa.so")

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED = 0, 1, 2, 3
FA_ERR_MASK_SPEC, FA_ERR_MASK_MISMATCH, FA_ERR_WORKSPACE, FA_ERR_HIP = 4, 5, 6, 7

FA_M_CAUSAL, FA_M_SWA, FA_M_DOC, FA_M_PREFIX, FA_M_AND, FA_M_OR = 1, 2, 3, 4, 5, 6
FA_MASK_MAX_NODES = 16
FA_S_IDENTITY, FA_S_ALIBI, FA_S_SOFTCAP, FA_S_RELPOS = 0, 1, 2, 3
FA_NOALLOC_SCRATCH_BYTES = 16 << 20

# names declared in include/fa.h (checked against the header by the tests)
EXPORTS = ("fa_block_mask_sizes", "fa_create_block_mask", "fa_block_mask_slice", "fa_block_mask_from_indices",
           "fa_forward_workspace_size",
           "fa_forward", "fa_forward_noalloc", "fa_forward_paged", "fa_backward_workspace_size",
           "fa_backward_workspace_min_size", "fa_backward",
           "fa_status_string", "fa_last_error_message")


class fa_mask_node(C.Structure):
    _fields_ = [("op", C.c_int32), ("arg", C.c_int32)]


class fa_mask_desc(C.Structure):
    _fields_ = [("n", C.c_int32),
                ("node", fa_mask_node * FA_MASK_MAX_NODES),
                ("doc_ids", C.c_void_p),
                ("doc_batch", C.c_int32),
                ("doc_len", C.c_int64)]


class fa_block_mask(C.Structure):
    _fields_ = [("mask", fa_mask_desc),
                ("B", C.c_int32), ("H", C.c_int32),
                ("q_len", C.c_int64), ("kv_len", C.c_int64), ("q_offset", C.c_int64),
                ("block_q", C.c_int32), ("block_kv", C.c_int32)] + [
        (n, C.c_void_p) for n in ("kv_num", "kv_ptr", "kv_idx", "full_kv_num", "full_kv_ptr",
                                  "full_kv_idx", "q_num", "q_ptr", "q_idx", "full_q_num",
                                  "full_q_ptr", "full_q_idx", "order")]


class fa_score_desc(C.Structure):
    _fields_ = [("kind", C.c_int32), ("softcap", C.c_float),
                ("alibi_slopes", C.c_void_p), ("relpos", C.c_void_p),
                ("relpos_radius", C.c_int32)]


class fa_fwd_args(C.Structure):
    _fields_ = [("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p), ("o", C.c_void_p),
                ("lse", C.c_void_p),
                ("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("d", C.c_int32),
                ("q_len", C.c_int64), ("kv_len", C.c_int64),
                ("scale", C.c_float),
                ("score", fa_score_desc),
                ("bm", C.POINTER(fa_block_mask)),
                ("workspace", C.c_void_p), ("ws_bytes", C.c_size_t)]


class fa_bwd_args(C.Structure):
    _fields_ = [("fwd", C.POINTER(fa_fwd_args)), ("dout", C.c_void_p), ("dq", C.c_void_p),
                ("dk", C.c_void_p), ("dv", C.c_void_p), ("workspace", C.c_void_p),
                ("ws_bytes", C.c_size_t), ("dslopes", C.c_void_p), ("dtable", C.c_void_p)]


class fa_paged_kv(C.Structure):
    _fields_ = [("page_table", C.c_void_p), ("pt_stride", C.c_int64), ("page_size", C.c_int32),
                ("num_pages", C.c_int64)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libfa.so (once).  Raises if it is missing: build it with
    ``python -m block_sparse_programmable_amd.build``."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: the HIP library is not built "
                          "(python -m block_sparse_programmable_amd.build)")
    lib = C.CDLL(path)
    lib.fa_block_mask_sizes.argtypes = [C.POINTER(fa_block_mask), C.POINTER(C.c_int64),
                                        C.POINTER(C.c_int64), C.POINTER(C.c_int64),
                                        C.POINTER(C.c_size_t)]
    lib.fa_block_mask_sizes.restype = C.c_int
    lib.fa_create_block_mask.argtypes = [C.POINTER(fa_block_mask), C.c_void_p, C.c_size_t, C.c_void_p]
    lib.fa_create_block_mask.restype = C.c_int
    lib.fa_block_mask_slice.argtypes = [C.POINTER(fa_block_mask), C.POINTER(fa_block_mask), C.c_void_p,
                                        C.c_size_t, C.c_void_p]
    lib.fa_block_mask_slice.restype = C.c_int
    lib.fa_block_mask_from_indices.argtypes = [C.POINTER(fa_block_mask), C.c_void_p, C.c_int32, C.c_void_p,
                                               C.c_size_t, C.c_void_p]
    lib.fa_block_mask_from_indices.restype = C.c_int
    lib.fa_forward_workspace_size.argtypes = [C.POINTER(fa_fwd_args), C.POINTER(C.c_size_t)]
    lib.fa_forward_workspace_size.restype = C.c_int
    lib.fa_forward.argtypes = [C.POINTER(fa_fwd_args), C.c_void_p]
    lib.fa_forward.restype = C.c_int
    lib.fa_forward_paged.argtypes = [C.POINTER(fa_fwd_args), C.POINTER(fa_paged_kv), C.c_void_p]
    lib.fa_forward_paged.restype = C.c_int
    lib.fa_forward_noalloc.argtypes = [C.POINTER(fa_fwd_args), C.c_void_p]
    lib.fa_forward_noalloc.restype = C.c_int
    lib.fa_backward_workspace_size.argtypes = [C.POINTER(fa_bwd_args), C.POINTER(C.c_size_t)]
    lib.fa_backward_workspace_size.restype = C.c_int
    lib.fa_backward_workspace_min_size.argtypes = [C.POINTER(fa_bwd_args), C.POINTER(C.c_size_t)]
    lib.fa_backward_workspace_min_size.restype = C.c_int
    lib.fa_backward.argtypes = [C.POINTER(fa_bwd_args), C.c_void_p]
    lib.fa_backward.restype = C.c_int
    lib.fa_status_string.argtypes = [C.c_int]
    lib.fa_status_string.restype = C.c_char_p
    lib.fa_last_error_message.argtypes = []
    lib.fa_last_error_message.restype = C.c_char_p
    _lib = lib
    return lib


class FAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status
        self.message = message


def check(status: int):
    if status != FA_OK:
        lib = load()
        raise FAError(status, lib.fa_last_error_message().decode(errors="replace"))
