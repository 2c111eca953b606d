"""ctypes binding of libspa.so (include/spa.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  Loading fails loudly when the library has not been
built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspa.so")

SPA_OK = 0
STATUS_NAMES = {
    0: "SPA_OK", -1: "SPA_ERR_NULL", -2: "SPA_ERR_SHAPE", -3: "SPA_ERR_DTYPE",
    -4: "SPA_ERR_UNSUPPORTED", -5: "SPA_ERR_ALIGN", -6: "SPA_ERR_WORKSPACE",
    -7: "SPA_ERR_SPLITS", -8: "SPA_ERR_LAUNCH", -9: "SPA_ERR_MODE",
}
SPA_BF16 = 0
SPA_FP8_E4M3_OCP = 1
SPA_FP8_E4M3_FNUZ = 2
SPA_MAX_SPLITS = 64

# exported symbols, in include/spa.h order
SYMBOLS = ("attn_workspace_size", "attn_fwd_decode", "attn_fwd_decode_noalloc", "attn_noalloc_scratch_bytes",
           "attn_fwd_prefill", "attn_merge_lse",
           "attn_build_gather", "attn_topk_select", "attn_topk_select_ids", "attn_bwd_workspace_size", "attn_bwd",
           "attn_last_error", "attn_abi_version")
SPA_MAX_TOPK = 2048


class SpaFwdArgs(ctypes.Structure):
    """Mirror of struct spa_fwd_args."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_queries", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("ratio", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("raw_dtype", ctypes.c_int32),
        ("cmp_dtype", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("heads_per_block", ctypes.c_int32),
        ("queries_per_block", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("k_raw", ctypes.c_void_p),
        ("v_raw", ctypes.c_void_p),
        ("k_cmp", ctypes.c_void_p),
        ("v_cmp", ctypes.c_void_p),
        ("k_cmp_scale", ctypes.c_void_p),
        ("v_cmp_scale", ctypes.c_void_p),
        ("raw_pages", ctypes.c_int64),
        ("cmp_pages", ctypes.c_int64),
        ("raw_pt", ctypes.c_void_p),
        ("cmp_pt", ctypes.c_void_p),
        ("raw_pt_stride", ctypes.c_int32),
        ("cmp_pt_stride", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p),
        ("query_seq", ctypes.c_void_p),
        ("query_pos", ctypes.c_void_p),
        ("cmp_idx", ctypes.c_void_p),
        ("cmp_cnt", ctypes.c_void_p),
        ("sink", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("err_flag", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class SpaBwdGrads(ctypes.Structure):
    """Mirror of struct spa_bwd_grads."""
    _fields_ = [
        ("d_o", ctypes.c_void_p),
        ("dq", ctypes.c_void_p),
        ("dk_raw", ctypes.c_void_p),
        ("dv_raw", ctypes.c_void_p),
        ("dk_cmp", ctypes.c_void_p),
        ("dv_cmp", ctypes.c_void_p),
        ("d_sink", ctypes.c_void_p),
    ]


class SpaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspa.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run sparse_paged_attention_amd.build.build()")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(SpaFwdArgs)
    lib.attn_workspace_size.argtypes = [P]
    lib.attn_workspace_size.restype = ctypes.c_size_t
    for fn in (lib.attn_fwd_decode, lib.attn_fwd_prefill, lib.attn_fwd_decode_noalloc):
        fn.argtypes = [P, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.attn_noalloc_scratch_bytes.argtypes = []
    lib.attn_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.attn_merge_lse.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                   ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_merge_lse.restype = ctypes.c_int
    lib.attn_build_gather.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_build_gather.restype = ctypes.c_int
    for fn in (lib.attn_topk_select, lib.attn_topk_select_ids):
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    lib.attn_bwd_workspace_size.argtypes = [P]
    lib.attn_bwd_workspace_size.restype = ctypes.c_size_t
    lib.attn_bwd.argtypes = [P, ctypes.POINTER(SpaBwdGrads), ctypes.c_void_p]
    lib.attn_bwd.restype = ctypes.c_int
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = ctypes.c_int32
    if lib.attn_abi_version() != 1:
        raise RuntimeError("libspa ABI version mismatch")
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != SPA_OK:
        msg = load().attn_last_error().decode(errors="replace")
        raise SpaError(status, msg)
