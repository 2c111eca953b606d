"""Torch-facing wrappers over the C ABI (include/spa.h).

PyTorch supplies device memory and the current HIP stream, nothing else:
these functions fill the argument block with ``data_ptr()`` values and call
the library.  They never compute any part of the attention themselves.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional, Tuple

import numpy as np
import torch

from . import _lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclasses.dataclass
class DeviceProblem:
    """Device-resident inputs of one attention call (torch tensors)."""
    mode: str
    num_seqs: int
    num_queries: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    window: int
    ratio: int
    topk: int
    scale: float
    cmp_fp8: bool
    num_splits: int
    q: torch.Tensor
    k_raw: torch.Tensor
    v_raw: torch.Tensor
    k_cmp: Optional[torch.Tensor]
    v_cmp: Optional[torch.Tensor]
    k_cmp_scale: Optional[torch.Tensor]
    v_cmp_scale: Optional[torch.Tensor]
    raw_pt: torch.Tensor
    cmp_pt: Optional[torch.Tensor]
    seq_lens: torch.Tensor
    query_seq: Optional[torch.Tensor]
    query_pos: Optional[torch.Tensor]
    cmp_idx: Optional[torch.Tensor]
    cmp_cnt: Optional[torch.Tensor]
    sink: Optional[torch.Tensor]
    cmp_fp8_fnuz: bool = False           # e4m3 pages in the FNUZ variant

    @classmethod
    def from_problem(cls, p, device="cuda") -> "DeviceProblem":
        """Copy a host problem (sparse_paged_attention_amd.synth.Problem) to the device."""
        def dev(a, dtype=None):
            if a is None:
                return None
            t = torch.from_numpy(np.ascontiguousarray(a))
            if dtype is not None:
                t = t.view(dtype)
            return t.to(device)

        def bits16(a):
            return dev(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)

        has_cmp = p.ratio > 0
        # a shared latent cache (value arrays that are the key arrays) stays
        # one device buffer, so the library sees K == V
        k_raw = bits16(p.k_raw)
        k_cmp = (dev(p.k_cmp) if p.cmp_fp8 else bits16(p.k_cmp)) if has_cmp else None
        k_scale = dev(p.k_cmp_scale) if (has_cmp and p.cmp_fp8) else None
        return cls(
            mode=p.mode, num_seqs=p.num_seqs, num_queries=p.num_queries,
            num_q_heads=p.num_q_heads, num_kv_heads=p.num_kv_heads, head_dim=p.head_dim,
            page_size=p.page_size, window=p.window, ratio=p.ratio, topk=p.topk,
            scale=float(np.float32(p.scale)), cmp_fp8=bool(p.cmp_fp8), num_splits=p.num_splits,
            q=bits16(p.q), k_raw=k_raw, v_raw=k_raw if p.v_raw is p.k_raw else bits16(p.v_raw),
            k_cmp=k_cmp,
            v_cmp=(k_cmp if p.v_cmp is p.k_cmp else (dev(p.v_cmp) if p.cmp_fp8 else bits16(p.v_cmp))) if has_cmp
            else None,
            k_cmp_scale=k_scale,
            v_cmp_scale=(k_scale if p.v_cmp_scale is p.k_cmp_scale else dev(p.v_cmp_scale))
            if (has_cmp and p.cmp_fp8) else None,
            raw_pt=dev(p.raw_pt), cmp_pt=dev(p.cmp_pt) if has_cmp else None,
            seq_lens=dev(p.seq_lens),
            query_seq=dev(p.query_seq) if p.mode == "prefill" else None,
            query_pos=dev(p.query_pos) if p.mode == "prefill" else None,
            cmp_idx=dev(p.cmp_idx) if (has_cmp and p.topk > 0) else None,
            cmp_cnt=dev(p.cmp_cnt) if (has_cmp and p.topk > 0) else None,
            sink=dev(p.sink) if p.sink is not None else None,
            cmp_fp8_fnuz=bool(getattr(p, "cmp_fp8_fnuz", False)),
        )

    def args(self, num_splits: Optional[int] = None, heads_per_block: int = 0,
             queries_per_block: int = 0) -> _lib.SpaFwdArgs:
        a = _lib.SpaFwdArgs()
        a.num_seqs = self.num_seqs
        a.num_queries = self.num_queries
        a.num_q_heads = self.num_q_heads
        a.num_kv_heads = self.num_kv_heads
        a.head_dim = self.head_dim
        a.page_size = self.page_size
        a.window = self.window
        a.ratio = self.ratio
        a.topk = self.topk
        a.scale = self.scale
        a.raw_dtype = _lib.SPA_BF16
        a.cmp_dtype = ((_lib.SPA_FP8_E4M3_FNUZ if self.cmp_fp8_fnuz else _lib.SPA_FP8_E4M3_OCP) if self.cmp_fp8
                       else _lib.SPA_BF16)
        a.num_splits = self.num_splits if num_splits is None else num_splits
        a.heads_per_block = heads_per_block
        a.queries_per_block = queries_per_block
        a.q = _ptr(self.q)
        a.k_raw = _ptr(self.k_raw)
        a.v_raw = _ptr(self.v_raw)
        a.k_cmp = _ptr(self.k_cmp)
        a.v_cmp = _ptr(self.v_cmp)
        a.k_cmp_scale = _ptr(self.k_cmp_scale)
        a.v_cmp_scale = _ptr(self.v_cmp_scale)
        a.raw_pages = self.k_raw.shape[0]
        a.cmp_pages = self.k_cmp.shape[0] if self.k_cmp is not None else 0
        a.raw_pt = _ptr(self.raw_pt)
        a.cmp_pt = _ptr(self.cmp_pt)
        a.raw_pt_stride = self.raw_pt.shape[1]
        a.cmp_pt_stride = self.cmp_pt.shape[1] if self.cmp_pt is not None else 0
        a.seq_lens = _ptr(self.seq_lens)
        a.query_seq = _ptr(self.query_seq)
        a.query_pos = _ptr(self.query_pos)
        a.cmp_idx = _ptr(self.cmp_idx)
        a.cmp_cnt = _ptr(self.cmp_cnt)
        a.sink = _ptr(self.sink)
        return a


def workspace_size(args: _lib.SpaFwdArgs) -> int:
    return int(_lib.load().attn_workspace_size(ctypes.byref(args)))


def forward_args(dp: DeviceProblem, args: _lib.SpaFwdArgs, o: torch.Tensor, lse: Optional[torch.Tensor],
                 workspace: Optional[torch.Tensor], err_flag: Optional[torch.Tensor],
                 stream: Optional[int] = None) -> None:
    """Fill the output/workspace fields of ``args`` and launch (decode or prefill)."""
    lib = _lib.load()
    args.o = _ptr(o)
    args.lse = _ptr(lse)
    args.err_flag = _ptr(err_flag)
    args.workspace = _ptr(workspace)
    args.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = lib.attn_fwd_decode if dp.mode == "decode" else lib.attn_fwd_prefill
    _lib.check(fn(ctypes.byref(args), _stream() if stream is None else stream))


def forward(dp: DeviceProblem, num_splits: Optional[int] = None, *, err_flag: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None,
            heads_per_block: int = 0, queries_per_block: int = 0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Run attn_fwd_decode / attn_fwd_prefill; returns (O bf16 [Nq,Hq,D], LSE f32 [Nq,Hq])."""
    args = dp.args(num_splits, heads_per_block, queries_per_block)
    dev = dp.q.device
    if out is None:
        out = torch.empty((dp.num_queries, dp.num_q_heads, dp.head_dim), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((dp.num_queries, dp.num_q_heads), dtype=torch.float32, device=dev)
    need = workspace_size(args)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    forward_args(dp, args, out, lse, workspace, err_flag)
    return out, lse


def merge_lse(o_parts: torch.Tensor, lse_parts: torch.Tensor, num_q_heads: int,
              sink: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              lse_out: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """attn_merge_lse: o_parts f32 [S, rows, D], lse_parts f32 [S, rows]."""
    S, rows, D = o_parts.shape
    if out is None:
        out = torch.empty((rows, D), dtype=torch.bfloat16, device=o_parts.device)
    if lse_out is None:
        lse_out = torch.empty((rows,), dtype=torch.float32, device=o_parts.device)
    lib = _lib.load()
    _lib.check(lib.attn_merge_lse(_ptr(o_parts), _ptr(lse_parts), S, rows, D, num_q_heads, _ptr(sink),
                                  _ptr(out), _ptr(lse_out), _stream()))
    return out, lse_out


def build_gather(dp: DeviceProblem, cap: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """attn_build_gather: (rows int64 [Nq, cap], counts int32 [Nq, 4])."""
    args = dp.args()
    dev = dp.q.device
    rows = torch.empty((dp.num_queries, cap), dtype=torch.int64, device=dev)
    counts = torch.empty((dp.num_queries, 4), dtype=torch.int32, device=dev)
    lib = _lib.load()
    _lib.check(lib.attn_build_gather(ctypes.byref(args), 1 if dp.mode == "decode" else 0, cap,
                                     _ptr(rows), _ptr(counts), _stream()))
    return rows, counts


def topk_select(scores: torch.Tensor, n_valid: torch.Tensor, k: int,
                by_id: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """attn_topk_select (by score) or attn_topk_select_ids (by_id: the same
    selection in ascending id order): scores f32 [rows, ld] (row stride ld),
    n_valid i32 [rows] -> (ids i32 [rows, k], -1 past the count; counts i32
    [rows])."""
    lib = _lib.load()
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be a float32 [rows, ld] tensor with unit column stride")
    rows = scores.shape[0]
    ids = torch.empty((rows, k), dtype=torch.int32, device=scores.device)
    cnt = torch.empty(rows, dtype=torch.int32, device=scores.device)
    nv = n_valid.to(device=scores.device, dtype=torch.int32).contiguous()
    fn = lib.attn_topk_select_ids if by_id else lib.attn_topk_select
    _lib.check(fn(_ptr(scores), scores.stride(0) if rows else max(scores.shape[1], 1), _ptr(nv), rows, k, _ptr(ids),
                  _ptr(cnt), _stream()))
    return ids, cnt


def backward(dp: DeviceProblem, o: torch.Tensor, lse: torch.Tensor, d_o: torch.Tensor, *,
             err_flag: Optional[torch.Tensor] = None, want_dsink: bool = True,
             grads: Optional[dict] = None, stream: Optional[int] = None, queries_per_block: int = 0,
             fused: bool = False) -> dict:
    """attn_bwd: gradients of the forward call described by ``dp`` from its
    outputs (o bf16, lse f32) and the upstream gradient d_o (bf16 [Nq,Hq,D]).
    Returns dict dq, dk_raw, dv_raw, dk_cmp, dv_cmp, d_sink (f32; the cache
    gradients have the caches' shapes).  ``grads`` reuses buffers, which the
    call accumulates into (dq is overwritten).  The workspace is sized by
    attn_bwd_workspace_size, which lets the library take the KV-block path;
    ``fused`` passes only the sink partials' share, which keeps the fused
    kernel."""
    lib = _lib.load()
    dev = dp.q.device
    if grads is None:
        grads = {
            "dq": torch.empty(dp.q.shape, dtype=torch.float32, device=dev),
            "dk_raw": torch.zeros(dp.k_raw.shape, dtype=torch.float32, device=dev),
            "dv_raw": torch.zeros(dp.v_raw.shape, dtype=torch.float32, device=dev),
            "dk_cmp": None if dp.k_cmp is None else torch.zeros(dp.k_cmp.shape, dtype=torch.float32, device=dev),
            "dv_cmp": None if dp.v_cmp is None else torch.zeros(dp.v_cmp.shape, dtype=torch.float32, device=dev),
            "d_sink": (torch.zeros(dp.num_q_heads, dtype=torch.float32, device=dev)
                       if (want_dsink and dp.sink is not None) else None),
        }
    args = dp.args(1, 0, queries_per_block)
    args.o = _ptr(o)
    args.lse = _ptr(lse)
    args.err_flag = _ptr(err_flag)
    ws = None
    need = int(lib.attn_bwd_workspace_size(ctypes.byref(args)))
    if fused:
        need = dp.num_queries * dp.num_q_heads * 4 if grads["d_sink"] is not None else 0
    if need > 0:
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        args.workspace = _ptr(ws)
        args.workspace_bytes = ws.numel()
    g = _lib.SpaBwdGrads()
    g.d_o = _ptr(d_o)
    for name in ("dq", "dk_raw", "dv_raw", "dk_cmp", "dv_cmp", "d_sink"):
        setattr(g, name, _ptr(grads[name]))
    _lib.check(lib.attn_bwd(ctypes.byref(args), ctypes.byref(g), _stream() if stream is None else stream))
    grads["_workspace"] = ws        # kept alive until the caller synchronises
    return grads
