"""Seeded synthetic inputs for sparse paged attention with a sink.

This module builds the host-side arrays that both the HIP path and the CPU
oracle consume: queries, paged raw and compressed KV caches, page tables,
per-token compressed-index lists and sink logits.  It computes no attention:
no gathering, no scores, no softmax.  The one rule it has to know is which
inputs are *valid*: a compressed index may name only a complete group
(group c of ratio r is complete at position t when r*(c+1) <= t+1), and a
window never reaches past the token itself.  Both the oracle and the kernels
recompute these bounds on their own.

Workloads (shapes, distributions and structure follow the joint
compressed/window attention PR "Roadmap item 24" of RL-Kernel and the
block-level DeepSeek-V4 attention test PR of ATOM, section "Validation"):

* ``tiny``     1 sequence of 64 tokens, 4 query heads / 1 KV head, D 64,
               page 16, window 16, ratio 4, top-k 8, 16 prefill queries at
               positions 48..63, scale 1/8, seed 0.
* ``decode_csa``  batch 32 x 1 query at position 4095, 128/1 heads, D 128,
               page 64, window 128, ratio 4, top-k 512 of 1024 groups.
* ``prefill_csa`` 1 sequence of 2560 tokens all queried, 64/1 heads, D 128,
               page 16, window 128, ratio 4, top-k 512 chosen by a seeded
               random score among the complete groups.
* ``decode_hca``  batch 4 x 1 query at position 32767, 128/1 heads, D 128,
               page 128, window 128, ratio 128, all 256 groups (no list),
               4 split-KV partitions.
* ``mixed_fp8``   batch 16, context lengths uniform in [1024, 16384],
               128/1 heads, D 128, page 64, window 128 (bf16), ratio-4
               compressed KV stored as OCP e4m3 with one fp32 scale per
               token row, top-k 512.

Data: every floating value is drawn fp32 N(0, 1) and rounded to bf16 by
round-to-nearest-even; sinks stay fp32 N(0, 1).  One
``numpy.random.Generator(PCG64(seed))`` per workload; the draws happen in a
fixed order.  Page pools are random permutations of the pages every sequence
needs plus a few spare pages; every cache row that no sequence owns (spare
pages and the tail of a sequence's last page) holds NaN so that a gather of a
row outside the KV set shows up as NaN in the output.  Page-table columns
past a sequence's last page hold 0x7FFFFFFF.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
E4M3_NAN = np.uint8(0x7F)
E4M3FNUZ_NAN = np.uint8(0x80)
PT_PAD = np.int32(0x7FFFFFFF)
E4M3_MAX = 448.0
E4M3FNUZ_MAX = 240.0


@dataclasses.dataclass
class Problem:
    name: str
    mode: str                      # "decode" or "prefill"
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    window: int
    ratio: int                     # 0 = no compressed KV
    topk: int                      # list capacity; 0 = every complete group
    scale: np.float32
    cmp_fp8: bool
    num_splits: int
    q: np.ndarray                  # uint16 bf16 bits [Nq, Hq, D]
    k_raw: np.ndarray              # uint16 [raw_pages, P, Hkv, D]
    v_raw: np.ndarray
    k_cmp: np.ndarray              # uint16 (bf16) or uint8 (e4m3) [cmp_pages, P, Hkv, D]
    v_cmp: np.ndarray
    k_cmp_scale: Optional[np.ndarray]   # float32 [cmp_pages, P, Hkv] (fp8 only)
    v_cmp_scale: Optional[np.ndarray]
    raw_pt: np.ndarray             # int32 [B, raw_stride]
    cmp_pt: np.ndarray             # int32 [B, cmp_stride]
    seq_lens: np.ndarray           # int32 [B]
    query_seq: np.ndarray          # int32 [Nq]
    query_pos: np.ndarray          # int32 [Nq]
    cmp_idx: np.ndarray            # int32 [Nq, max(topk, 1)], -1 padded
    cmp_cnt: np.ndarray            # int32 [Nq]
    sink: Optional[np.ndarray]     # float32 [Hq] or None (= -inf)
    cmp_fp8_fnuz: bool = False     # e4m3 pages in the FNUZ variant (else OCP)
    # logical (unpaged) copies, used only by tests that bypass page tables
    k_raw_logical: Optional[list] = None   # per seq: [len, Hkv, D]
    v_raw_logical: Optional[list] = None
    k_cmp_logical: Optional[list] = None   # per seq: [n_groups, Hkv, D]
    v_cmp_logical: Optional[list] = None
    k_cmp_scale_logical: Optional[list] = None
    v_cmp_scale_logical: Optional[list] = None

    @property
    def num_queries(self) -> int:
        return int(self.q.shape[0])


# ---------------------------------------------------------------- rounding

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = BF16_NAN
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_e4m3(y: np.ndarray) -> np.ndarray:
    """Encode float values as OCP e4m3 (bias 7, no infinities, max 448).

    Round to nearest, ties to even, saturating to +-448.  Written from the OCP
    8-bit floating point format definition; returns uint8 codes.
    """
    y = np.asarray(y, dtype=np.float64)
    sign = (np.signbit(y)).astype(np.uint8) << 7
    a = np.minimum(np.abs(y), E4M3_MAX)
    codes = np.zeros(a.shape, dtype=np.uint8)
    # exponent of the value's binade, clamped at the subnormal binade (-6)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, 8).astype(np.int64)
    step = np.ldexp(1.0, e - 3)                 # spacing of codes in this binade
    q = a / step
    qi = np.floor(q)
    frac = q - qi
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(qi, 2) == 1))
    qi = qi + up
    # qi in [0, 16]; 16 means the next binade
    norm = e > -6
    mant_units = qi.astype(np.int64)              # multiples of step
    # normal: value = mant_units * 2^(e-3), mant_units in [8, 16]
    # subnormal (e == -6): value = mant_units * 2^-9, mant_units in [0, 8]
    ee = np.where(mant_units >= 16, e + 1, e)
    mu = np.where(mant_units >= 16, 8, mant_units)
    is_norm = norm | (mu >= 8)
    exp_field = np.where(is_norm, ee + 7, 0)
    mant_field = np.where(is_norm, mu - 8, mu)
    codes = ((exp_field.astype(np.uint8) << 3) | mant_field.astype(np.uint8)).astype(np.uint8)
    codes = np.where(a == 0, 0, codes).astype(np.uint8)
    return (codes | sign).astype(np.uint8)


def _fnuz_grid() -> np.ndarray:
    """The 128 non-negative finite FNUZ e4m3 values, by code 0x00 .. 0x7F
    (bias 8: subnormals m/8 * 2^-7, normals (1 + m/8) * 2^(e-8))."""
    v = []
    for c in range(128):
        e, m = c >> 3, c & 7
        v.append((m / 8.0) * 2.0 ** -7 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 8))
    return np.array(v, dtype=np.float64)


_FNUZ_GRID = _fnuz_grid()


def quantize_e4m3_fnuz(y: np.ndarray) -> np.ndarray:
    """Encode float values as FNUZ e4m3 (bias 8, max 240, no negative zero).

    Round to nearest, ties to the even code, saturating to +-240; zero and
    values that round to zero get code 0x00 (0x80 is NaN).  Returns uint8.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3FNUZ_MAX)
    hi = np.clip(np.searchsorted(_FNUZ_GRID, a, side="left"), 0, 127)
    lo = np.clip(hi - 1, 0, 127)
    dlo, dhi = a - _FNUZ_GRID[lo], _FNUZ_GRID[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    sign = (np.signbit(y) & (code != 0)).astype(np.uint8) << 7
    return (code | sign).astype(np.uint8)


# ---------------------------------------------------------------- builders

def _spawn(seed: int, n: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(n)]


def _normal_bf16(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _page_pool(rng, lens_rows, page_size, spare_pages=3):
    """Scatter per-sequence logical rows into a shuffled page pool.

    ``lens_rows``: list of per-sequence row counts.  Returns (page table
    [B, stride] int32 padded with 0x7FFFFFFF, pool page count, list of per
    sequence page-id arrays).
    """
    need = [(n + page_size - 1) // page_size for n in lens_rows]
    total = int(sum(need)) + spare_pages
    perm = rng.permutation(total).astype(np.int32)
    stride = max(1, max(need) if need else 1)
    pt = np.full((len(lens_rows), stride), PT_PAD, dtype=np.int32)
    pos = 0
    pages = []
    for b, n in enumerate(need):
        ids = perm[pos:pos + n]
        pt[b, :n] = ids
        pages.append(ids)
        pos += n
    return pt, total, pages


def _scatter(pool, pages, logical, page_size):
    """Write logical rows [n, ...] of one sequence into its pages of pool."""
    n = logical.shape[0]
    for j, pid in enumerate(pages):
        lo = j * page_size
        hi = min(n, lo + page_size)
        if hi > lo:
            pool[pid, :hi - lo] = logical[lo:hi]


def make_problem(name: str, mode: str, seq_lens, num_q_heads, num_kv_heads, head_dim,
                 page_size, window, ratio, topk, *, seed, cmp_fp8=False, num_splits=1,
                 query_positions=None, selection="random", with_sink=True,
                 scale=None, spare_pages=3, keep_logical=True, shared_kv=False, fp8_format="ocp"):
    """Generic builder used by every named workload and by parametrised tests.

    ``query_positions``: prefill only, a list of (seq, pos) pairs.  Decode
    queries sit at position seq_len-1 of each sequence.
    ``selection``: "random" (distinct random groups, random order), "score"
    (top-k of a seeded random score, ties to the lower index), or "all"
    (list of every complete group in ascending order).
    ``shared_kv``: one latent cache per pool serves as K and V (the value
    arrays are the key arrays, the same objects); with e4m3 compressed
    pages the row scales are shared too (one scale per latent row).
    ``fp8_format``: "ocp" (max 448) or "fnuz" (max 240) for e4m3 pages.
    """
    fnuz = cmp_fp8 and fp8_format == "fnuz"
    qmax = np.float32(E4M3FNUZ_MAX if fnuz else E4M3_MAX)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    B = len(seq_lens)
    Hq, Hkv, D, P = num_q_heads, num_kv_heads, head_dim, page_size
    (r_q, r_raw, r_cmp, r_scale, r_pages, r_sel, r_sink) = _spawn(seed, 7)

    if mode == "decode":
        qs = np.arange(B, dtype=np.int32)
        qp = (seq_lens - 1).astype(np.int32)
    else:
        qs = np.asarray([s for s, _ in query_positions], dtype=np.int32)
        qp = np.asarray([p for _, p in query_positions], dtype=np.int32)
    Nq = len(qs)

    q = _normal_bf16(r_q, (Nq, Hq, D))

    # raw cache
    raw_pt, raw_pages_n, raw_pages = _page_pool(r_pages, [int(n) for n in seq_lens], P, spare_pages)
    k_raw = np.full((raw_pages_n, P, Hkv, D), BF16_NAN, dtype=np.uint16)
    v_raw = np.full_like(k_raw, BF16_NAN)
    k_log, v_log = [], []
    for b in range(B):
        kl = _normal_bf16(r_raw, (int(seq_lens[b]), Hkv, D))
        vl = _normal_bf16(r_raw, (int(seq_lens[b]), Hkv, D))
        _scatter(k_raw, raw_pages[b], kl, P)
        _scatter(v_raw, raw_pages[b], vl, P)
        k_log.append(kl)
        v_log.append(vl)

    # compressed cache: one entry per complete group of the whole sequence
    n_groups = [int(n) // ratio if ratio > 0 else 0 for n in seq_lens]
    cmp_pt, cmp_pages_n, cmp_pages = _page_pool(r_pages, n_groups, P, spare_pages)
    kc_log, vc_log, ks_log, vs_log = [], [], [], []
    if cmp_fp8:
        poison = E4M3FNUZ_NAN if fnuz else E4M3_NAN
        k_cmp = np.full((cmp_pages_n, P, Hkv, D), poison, dtype=np.uint8)
        v_cmp = np.full_like(k_cmp, poison)
        k_sc = np.full((cmp_pages_n, P, Hkv), np.nan, dtype=np.float32)
        v_sc = np.full_like(k_sc, np.nan)
    else:
        k_cmp = np.full((cmp_pages_n, P, Hkv, D), BF16_NAN, dtype=np.uint16)
        v_cmp = np.full_like(k_cmp, BF16_NAN)
        k_sc = v_sc = None
    for b in range(B):
        g = n_groups[b]
        if cmp_fp8:
            pair = []
            for _ in range(2):
                x = r_cmp.standard_normal((g, Hkv, D), dtype=np.float32)
                amax = np.max(np.abs(x), axis=-1)
                sc = (amax / qmax).astype(np.float32)
                sc = np.where(sc > 0, sc, np.float32(1.0)).astype(np.float32)
                quant = quantize_e4m3_fnuz if fnuz else quantize_e4m3
                codes = quant(x.astype(np.float64) / sc[..., None].astype(np.float64))
                pair.append((codes, sc))
            (kc, ks), (vc, vs) = pair
            _scatter(k_sc, cmp_pages[b], ks, P)
            _scatter(v_sc, cmp_pages[b], vs, P)
            ks_log.append(ks)
            vs_log.append(vs)
        else:
            kc = _normal_bf16(r_cmp, (g, Hkv, D))
            vc = _normal_bf16(r_cmp, (g, Hkv, D))
        _scatter(k_cmp, cmp_pages[b], kc, P)
        _scatter(v_cmp, cmp_pages[b], vc, P)
        kc_log.append(kc)
        vc_log.append(vc)

    if shared_kv:
        v_raw, v_log, v_cmp, vc_log = k_raw, k_log, k_cmp, kc_log
        if cmp_fp8:
            v_sc, vs_log = k_sc, ks_log

    # per-query compressed index lists
    cap = max(topk, 1)
    cmp_idx = np.full((Nq, cap), -1, dtype=np.int32)
    cmp_cnt = np.zeros(Nq, dtype=np.int32)
    if ratio > 0 and topk > 0:
        if selection == "score":
            max_g = max(n_groups) if n_groups else 0
            scores = r_sel.standard_normal((Nq, max(max_g, 1)), dtype=np.float32)
        for i in range(Nq):
            t = int(qp[i])
            nc = (t + 1) // ratio          # groups complete at position t
            k = min(topk, nc)
            if selection == "random":
                sel = r_sel.permutation(nc)[:k]
            elif selection == "score":
                order = np.argsort(-scores[i, :nc], kind="stable")
                sel = order[:k]
            elif selection == "all":
                sel = np.arange(nc)
            else:
                raise ValueError(selection)
            cmp_idx[i, :k] = sel
            cmp_cnt[i] = k

    sink = r_sink.standard_normal(Hq, dtype=np.float32) if with_sink else None
    if scale is None:
        scale = np.float32(1.0) / np.sqrt(np.float32(D))
    p = Problem(
        name=name, mode=mode, num_seqs=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
        page_size=P, window=window, ratio=ratio, topk=topk, scale=np.float32(scale),
        cmp_fp8=cmp_fp8, num_splits=num_splits, q=q, k_raw=k_raw, v_raw=v_raw,
        k_cmp=k_cmp, v_cmp=v_cmp, k_cmp_scale=k_sc, v_cmp_scale=v_sc, raw_pt=raw_pt,
        cmp_pt=cmp_pt, seq_lens=seq_lens, query_seq=qs, query_pos=qp, cmp_idx=cmp_idx,
        cmp_cnt=cmp_cnt, sink=sink, cmp_fp8_fnuz=fnuz)
    if keep_logical:
        p.k_raw_logical, p.v_raw_logical = k_log, v_log
        p.k_cmp_logical, p.v_cmp_logical = kc_log, vc_log
        if cmp_fp8:
            p.k_cmp_scale_logical, p.v_cmp_scale_logical = ks_log, vs_log
    return p


WORKLOADS = ("tiny", "decode_csa", "prefill_csa", "decode_hca", "mixed_fp8", "decode_latent")


def make_workload(name: str, *, batch: Optional[int] = None, keep_logical: bool = False,
                  context: Optional[int] = None) -> Problem:
    """The named workloads (the five measured configurations and the 512-wide
    shared-latent decode).  ``batch`` overrides the decode batch size
    (one GPU's share of a larger batch, or a bounded CPU sample); ``context``
    gives every decode sequence that length (for sweeps of the KV-set size)."""
    if context is not None and name in ("tiny", "prefill_csa"):
        raise ValueError("context applies to the decode workloads")
    if name == "tiny":
        return make_problem("tiny", "prefill", [64], 4, 1, 64, 16, 16, 4, 8, seed=0,
                            query_positions=[(0, p) for p in range(48, 64)],
                            selection="random", keep_logical=True)
    if name == "decode_csa":
        b = batch or 32
        return make_problem("decode_csa", "decode", [context or 4096] * b, 128, 1, 128, 64, 128, 4, 512,
                            seed=1, selection="random", keep_logical=keep_logical)
    if name == "prefill_csa":
        return make_problem("prefill_csa", "prefill", [2560], 64, 1, 128, 16, 128, 4, 512,
                            seed=2, query_positions=[(0, p) for p in range(2560)],
                            selection="score", keep_logical=keep_logical)
    if name == "decode_hca":
        b = batch or 4
        return make_problem("decode_hca", "decode", [context or 32768] * b, 128, 1, 128, 128, 128, 128, 0,
                            seed=3, num_splits=4, keep_logical=keep_logical)
    if name == "mixed_fp8":
        b = batch or 16
        rng = np.random.Generator(np.random.PCG64(4))
        lens = rng.integers(1024, 16384, size=b, endpoint=True).astype(np.int32)
        if context is not None:
            lens[:] = context
        return make_problem("mixed_fp8", "decode", lens, 128, 1, 128, 64, 128, 4, 512,
                            seed=4, cmp_fp8=True, selection="random", keep_logical=keep_logical)
    if name == "decode_latent":
        # the 512-wide shared latent cache (K = V) in 256-token pages, with
        # the CSA layer's window and top-k of decode_csa and 64 query heads
        b = batch or 32
        return make_problem("decode_latent", "decode", [context or 4096] * b, 64, 1, 512, 256, 128, 4, 512,
                            seed=5, selection="random", num_splits=8, shared_kv=True, keep_logical=keep_logical)
    raise ValueError(f"unknown workload {name!r}")
