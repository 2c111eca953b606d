"""Gradients of sparse paged attention with a sink, in float64.

Test infrastructure only (see the package docstring).

The RL-Kernel PR "Roadmap item 24: joint compressed/window attention with
sink" keeps the log-sum-exp as the forward state for a backward pass that
follows it (section "Reuse and arithmetic", and the summary naming the
backward as the next item).  The pages give no formulas for it, so this is
the derivative of the forward definition (``sparse_attention.attend``),
worked out here.  For one query head h with KV set j = 1..N, sink logit
sigma, scores s_j = scale * <q, k_j>, LSE = ln(sum_j e^{s_j} + e^{sigma}),
p_j = e^{s_j - LSE}, O = sum_j p_j v_j and an upstream gradient dO:

    dv_j     += p_j dO
    dp_j      = <dO, v_j>
    Delta     = <dO, O>              (= sum_j p_j dp_j, since the sink has no value)
    ds_j      = p_j (dp_j - Delta)
    dq        = scale * sum_j ds_j k_j
    dk_j     += scale * ds_j q
    dsigma   += -e^{sigma - LSE} Delta

Readings taken:
* O and LSE are the exact forward values (recomputed here in float64);
* gradients of the caches are accumulated in the caches' own paged layout,
  so a row read by several queries (a shared window row, a group listed by
  several queries) sums their contributions;
* a query with an empty KV set and no sink (LSE = -inf) contributes nothing;
* bf16 caches only: the e4m3 pages are a storage format of the forward.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .formats import bf16_to_f64
from .sparse_attention import attend, kv_set, physical_rows


@dataclasses.dataclass
class Grads:
    dq: np.ndarray          # [Nq, Hq, D]
    dk_raw: np.ndarray      # the raw cache's shape [raw_pages, P, Hkv, D]
    dv_raw: np.ndarray
    dk_cmp: Optional[np.ndarray]   # the compressed cache's shape (None without one)
    dv_cmp: Optional[np.ndarray]
    dsink: Optional[np.ndarray]    # [Hq] (None without a sink)


def backward_values(p, q, k_raw, v_raw, k_cmp, v_cmp, sink, dO) -> Grads:
    """The gradients above for float64 inputs laid out like the problem's
    arrays (q [Nq, Hq, D]; caches [pages, P, Hkv, D]; sink [Hq] or None;
    dO [Nq, Hq, D]); the KV sets and page tables are the problem's."""
    Hq, D = p.num_q_heads, p.head_dim
    Hkv = p.num_kv_heads
    group = Hq // Hkv
    P = p.page_size
    scale = float(np.float32(p.scale))
    dq = np.zeros_like(q)
    dk_raw = np.zeros_like(k_raw)
    dv_raw = np.zeros_like(v_raw)
    dk_cmp = None if k_cmp is None else np.zeros_like(k_cmp)
    dv_cmp = None if v_cmp is None else np.zeros_like(v_cmp)
    dsink = None if sink is None else np.zeros(Hq)
    for i in range(q.shape[0]):
        s = kv_set(p, i)
        crow, wrow = physical_rows(p, s)
        nc = len(crow)
        if nc:
            Kc, Vc = k_cmp[crow // P, crow % P], v_cmp[crow // P, crow % P]
        else:
            Kc = Vc = np.zeros((0, Hkv, D))
        K = np.concatenate([Kc, k_raw[wrow // P, wrow % P]], axis=0)    # [N, Hkv, D]
        V = np.concatenate([Vc, v_raw[wrow // P, wrow % P]], axis=0)
        O, LSE = attend(q[i], K, V, scale, sink)
        for g in range(Hkv):
            hs = slice(g * group, (g + 1) * group)
            lse = LSE[hs]
            live = np.isfinite(lse)                     # heads with a softmax at all
            lse_safe = np.where(live, lse, 0.0)
            sc = scale * (q[i, hs] @ K[:, g, :].T)     # [group, N]
            pr = np.where(live[:, None], np.exp(sc - lse_safe[:, None]), 0.0)
            dp = dO[i, hs] @ V[:, g, :].T               # [group, N]
            delta = np.where(live, np.sum(dO[i, hs] * O[hs], axis=1), 0.0)
            ds = pr * (dp - delta[:, None])
            dq[i, hs] = scale * (ds @ K[:, g, :])
            dk_rows = scale * (ds.T @ q[i, hs])         # [N, D]
            dv_rows = pr.T @ dO[i, hs]
            for j in range(nc):
                r = crow[j]
                dk_cmp[r // P, r % P, g] += dk_rows[j]
                dv_cmp[r // P, r % P, g] += dv_rows[j]
            for j, r in enumerate(wrow):
                dk_raw[r // P, r % P, g] += dk_rows[nc + j]
                dv_raw[r // P, r % P, g] += dv_rows[nc + j]
            if sink is not None:
                psink = np.where(live, np.exp(sink[hs] - lse_safe), 0.0)
                dsink[hs] += -psink * delta
    return Grads(dq, dk_raw, dv_raw, dk_cmp, dv_cmp, dsink)


def attention_backward(p, dO_bits: np.ndarray) -> Grads:
    """Gradients of the problem's attention (bf16 inputs, decoded exactly)
    for the upstream gradient dO given as bf16 bits [Nq, Hq, D]."""
    if p.cmp_fp8:
        raise NotImplementedError("the backward takes bf16 caches")
    has_cmp = p.ratio > 0
    return backward_values(
        p, bf16_to_f64(p.q), bf16_to_f64(p.k_raw), bf16_to_f64(p.v_raw),
        bf16_to_f64(p.k_cmp) if has_cmp else None, bf16_to_f64(p.v_cmp) if has_cmp else None,
        None if p.sink is None else p.sink.astype(np.float64), bf16_to_f64(dO_bits))
