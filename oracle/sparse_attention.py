"""Sparse paged attention with a sink, in float64, by its definition.

Test infrastructure only (see the package docstring).

Sources (the pages this follows; no code from them):
* RL-Kernel PR "Roadmap item 24: joint compressed/window attention with sink",
  section "Reuse and arithmetic": the selected compressed KV, the full recent
  window of raw KV and a per-head sink logit share one softmax denominator;
  the sink has no value row; P and O are bf16 and the log-sum-exp is fp32 in
  natural log.  Section "Contracts and lifetime": complete windows, C4/C128
  group boundaries, a canonical KV ordering.
* ATOM PR "test: add block-level DeepSeek-V4 attention test", sections
  "What the reference proves" and "Validation": layer types by compress
  ratio (0 dense window only, 4 CSA top-k, 128 HCA all groups), the window of
  at most 128 raw tokens, and top-k truncation only once the number of
  complete groups exceeds index_topk.
* RL-Kernel "Fixed paged CK attention on ROCm": page-table translation with
  64-bit cache addressing.
* RL-Kernel PR "[WS2] CP-aware Attention contract" (Summary, Behavior) and the
  tessera "Block AttnRes" PR (attn-with-stats + softmax_merge pair): the
  exact merge of partial (out, lse) pairs.

Readings taken where the pages are silent:
* group c of ratio r is complete at token position t when r*(c+1) <= t+1, so
  n_c = floor((t+1)/r);
* the window is the min(W, t+1) raw positions ending at t (the token itself
  included);
* window rows and compressed rows are distinct KV entries (no de-duplication);
* the sink enters the denominator unscaled, and LSE includes it;
* an empty KV set with no sink gives O = 0 and LSE = -inf.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .formats import bf16_to_f64, e4m3_to_f64, e4m3fnuz_to_f64


@dataclasses.dataclass
class KVSet:
    """One query's KV set in canonical order: [compressed in list order || window ascending]."""
    seq: int
    pos: int
    win_lo: int
    win_len: int
    n_c: int
    n_sel: int
    cmp_ids: np.ndarray     # int64 logical compressed ids, list order
    win_pos: np.ndarray     # int64 raw positions, ascending

    @property
    def size(self) -> int:
        return self.n_sel + self.win_len


def _query_seq_pos(p, i: int) -> Tuple[int, int]:
    if p.mode == "decode":
        return i, int(p.seq_lens[i]) - 1
    return int(p.query_seq[i]), int(p.query_pos[i])


def kv_set(p, i: int) -> KVSet:
    """The KV set of query i (ATOM DeepSeek-V4 block test, "What the reference
    proves"; RL-Kernel joint attention PR, "Contracts and lifetime").

    Window: raw positions max(0, t-W+1) .. t.  Compressed: the listed ids for a
    top-k (CSA) layer, every complete group for an all-groups (HCA) layer,
    nothing when the ratio is 0 (dense layer).  Complete groups at t:
    floor((t+1)/r).
    """
    b, t = _query_seq_pos(p, i)
    if not (0 <= b < p.num_seqs):
        raise ValueError(f"query {i}: sequence {b} out of range")
    if not (0 <= t < int(p.seq_lens[b])):
        raise ValueError(f"query {i}: position {t} outside sequence of length {p.seq_lens[b]}")
    W = int(p.window)
    win_lo = max(0, t - W + 1) if W > 0 else t + 1
    win_len = t - win_lo + 1
    r = int(p.ratio)
    n_c = (t + 1) // r if r > 0 else 0
    if r > 0 and p.topk > 0:
        cnt = int(p.cmp_cnt[i])
        if not (0 <= cnt <= p.topk):
            raise ValueError(f"query {i}: list count {cnt} outside [0, {p.topk}]")
        ids = np.asarray(p.cmp_idx[i, :cnt], dtype=np.int64)
        if cnt and (ids.min() < 0 or ids.max() >= n_c):
            raise ValueError(f"query {i}: compressed id outside the {n_c} complete groups")
        if len(np.unique(ids)) != cnt:
            raise ValueError(f"query {i}: repeated compressed id")
    elif r > 0:
        ids = np.arange(n_c, dtype=np.int64)
    else:
        ids = np.zeros(0, dtype=np.int64)
    return KVSet(seq=b, pos=t, win_lo=win_lo, win_len=win_len, n_c=n_c, n_sel=len(ids),
                 cmp_ids=ids, win_pos=np.arange(win_lo, t + 1, dtype=np.int64))


def kv_sets(p) -> List[KVSet]:
    return [kv_set(p, i) for i in range(p.num_queries)]


def _physical_rows(pt_row: np.ndarray, logical: np.ndarray, page_size: int, n_pages: int) -> np.ndarray:
    """Page-table translation, 64-bit (RL-Kernel "Fixed paged CK attention on
    ROCm"): row = page_table[p // P] * P + p % P."""
    pages = pt_row[logical // page_size].astype(np.int64)
    if len(pages) and (pages.min() < 0 or pages.max() >= n_pages):
        raise ValueError("page id outside the cache pool")
    return pages * page_size + logical % page_size


def physical_rows(p, s: KVSet) -> Tuple[np.ndarray, np.ndarray]:
    """(compressed rows, window rows) as int64 row indices into each pool."""
    P = p.page_size
    crow = _physical_rows(p.cmp_pt[s.seq], s.cmp_ids, P, p.k_cmp.shape[0])
    wrow = _physical_rows(p.raw_pt[s.seq], s.win_pos, P, p.k_raw.shape[0])
    return crow, wrow


def gather_rows(p, s: KVSet) -> Tuple[np.ndarray, np.ndarray]:
    """K and V of one KV set, [N, Hkv, D] float64, canonical order."""
    crow, wrow = physical_rows(p, s)
    P = p.page_size
    Hkv, D = p.num_kv_heads, p.head_dim
    kr = bf16_to_f64(p.k_raw[wrow // P, wrow % P])
    vr = bf16_to_f64(p.v_raw[wrow // P, wrow % P])
    if p.cmp_fp8:
        dec = e4m3fnuz_to_f64 if getattr(p, "cmp_fp8_fnuz", False) else e4m3_to_f64
        kc = dec(p.k_cmp[crow // P, crow % P])
        vc = dec(p.v_cmp[crow // P, crow % P])
        kc = kc * p.k_cmp_scale[crow // P, crow % P].astype(np.float64)[..., None]
        vc = vc * p.v_cmp_scale[crow // P, crow % P].astype(np.float64)[..., None]
    else:
        kc = bf16_to_f64(p.k_cmp[crow // P, crow % P])
        vc = bf16_to_f64(p.v_cmp[crow // P, crow % P])
    K = np.concatenate([kc.reshape(-1, Hkv, D), kr.reshape(-1, Hkv, D)], axis=0)
    V = np.concatenate([vc.reshape(-1, Hkv, D), vr.reshape(-1, Hkv, D)], axis=0)
    return K, V


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           sink: Optional[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of one query over one KV set, sink in the denominator
    (RL-Kernel joint attention PR, "Reuse and arithmetic").

    q [Hq, D]; K, V [N, Hkv, D]; query head h reads KV head h // (Hq/Hkv).
    s_j = scale * <q_h, k_j>;  m = max(max_j s_j, sink_h);
    Z = sum_j exp(s_j - m) + exp(sink_h - m);  O = sum_j exp(s_j - m) v_j / Z;
    LSE = m + ln Z.  sink None means -inf (no sink).
    """
    Hq, D = q.shape
    N, Hkv, _ = K.shape
    group = Hq // Hkv
    O = np.zeros((Hq, D), dtype=np.float64)
    LSE = np.full(Hq, -np.inf, dtype=np.float64)
    for g in range(Hkv):
        hs = slice(g * group, (g + 1) * group)
        s = float(scale) * (q[hs] @ K[:, g, :].T)                   # [group, N]
        sig = (np.full(group, -np.inf) if sink is None
               else np.asarray(sink[hs], dtype=np.float64))
        m = np.maximum(s.max(axis=1) if N else np.full(group, -np.inf), sig)
        finite = np.isfinite(m)
        m_safe = np.where(finite, m, 0.0)
        e = np.exp(s - m_safe[:, None]) if N else np.zeros((group, 0))
        z = e.sum(axis=1) + np.exp(sig - m_safe)
        with np.errstate(invalid="ignore", divide="ignore"):
            o = (e @ V[:, g, :]) / z[:, None]
            lse = m_safe + np.log(z)
        O[hs] = np.where(finite[:, None], o, 0.0)
        LSE[hs] = np.where(finite, lse, -np.inf)
    return O, LSE


def attend_partial(q, K, V, scale) -> Tuple[np.ndarray, np.ndarray]:
    """Sink-free partial (O_p, LSE_p) over a subset of a KV set; an empty
    subset gives O_p = 0, LSE_p = -inf (the "attn_with_stats" half of the
    tessera Block AttnRes primitive pair)."""
    return attend(q, K, V, scale, None)


def merge(parts: Sequence[Tuple[np.ndarray, np.ndarray]],
          sink: Optional[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Exact merge of sink-free partials plus the sink (RL-Kernel WS2 PR,
    "Behavior": deterministic (out, lse) reduction; tessera Block AttnRes PR:
    softmax_merge).

    LSE = ln(sum_p exp(LSE_p) + exp(sink));  O = sum_p exp(LSE_p - LSE) O_p.
    The sink acts as one more part with LSE = sink and O = 0.
    """
    O0, L0 = parts[0]
    Hq = L0.shape[0]
    lses = [np.asarray(l, dtype=np.float64) for _, l in parts]
    if sink is not None:
        lses.append(np.asarray(sink, dtype=np.float64))
    M = np.max(np.stack(lses), axis=0)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    Z = np.zeros(Hq)
    O = np.zeros_like(O0, dtype=np.float64)
    for (o, l) in parts:
        w = np.exp(np.asarray(l, dtype=np.float64) - Ms)
        Z += w
        O += w[:, None] * o
    if sink is not None:
        Z += np.exp(np.asarray(sink, dtype=np.float64) - Ms)
    with np.errstate(invalid="ignore", divide="ignore"):
        O = np.where(finite[:, None], O / Z[:, None], 0.0)
        L = np.where(finite, Ms + np.log(Z), -np.inf)
    return O, L


def query_f64(p, i: int) -> np.ndarray:
    return bf16_to_f64(p.q[i])


def attention(p, queries: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """O [n, Hq, D] and LSE [n, Hq] (float64) for the given queries (all by default)."""
    idx = range(p.num_queries) if queries is None else list(queries)
    sink = None if p.sink is None else p.sink.astype(np.float64)
    scale = float(np.float32(p.scale))
    Os, Ls = [], []
    for i in idx:
        s = kv_set(p, i)
        K, V = gather_rows(p, s)
        o, l = attend(query_f64(p, i), K, V, scale, sink)
        Os.append(o)
        Ls.append(l)
    return np.stack(Os), np.stack(Ls)


def partial_split(n: int, parts: int) -> List[Tuple[int, int]]:
    """Contiguous slices of ceil(n/parts) entries (the last ones may be empty)."""
    step = -(-n // parts) if parts > 0 else n
    return [(min(n, j * step), min(n, (j + 1) * step)) for j in range(parts)]


def gather_plan(p, cap: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-query gather metadata: rows [Nq, cap] int64 (compressed rows in list
    order, then window rows ascending; -1 padded) and counts [Nq, 4] int32 =
    (win_lo, win_len, n_c, n_sel)."""
    Nq = p.num_queries
    rows = np.full((Nq, cap), -1, dtype=np.int64)
    counts = np.zeros((Nq, 4), dtype=np.int32)
    for i in range(Nq):
        s = kv_set(p, i)
        crow, wrow = physical_rows(p, s)
        allr = np.concatenate([crow, wrow])
        if len(allr) > cap:
            raise ValueError(f"query {i}: KV set of {len(allr)} exceeds cap {cap}")
        rows[i, :len(allr)] = allr
        counts[i] = (s.win_lo, s.win_len, s.n_c, s.n_sel)
    return rows, counts


def lse_merge_arrays(o_parts: np.ndarray, lse_parts: np.ndarray,
                     sink: Optional[np.ndarray], num_q_heads: int) -> Tuple[np.ndarray, np.ndarray]:
    """merge() over flat arrays: o_parts [S, rows, D], lse_parts [S, rows];
    row r takes sink[r % num_q_heads]."""
    S, R, D = o_parts.shape
    sk = None
    if sink is not None:
        sk = np.asarray(sink, dtype=np.float64)[np.arange(R) % num_q_heads]
    parts = [(o_parts[s].astype(np.float64), lse_parts[s].astype(np.float64)) for s in range(S)]
    return merge(parts, sk)

