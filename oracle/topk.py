"""Top-k selection of compressed groups from per-token scores, exactly.

Test infrastructure only (see the package docstring).

On the pages, the step right before the attention core scores every
complete compressed group of a token, selects index_topk of them and turns
the selected ids into paged offsets. The ATOM PR "test: add block-level
DeepSeek-V4 attention test" shows this in two sections:
* "What this test actually drives": the indexer scoring, a radix top-k
  select and a top-k -> paged-offset pack, as separate kernels;
* "Validation": the top-k truncates only once the complete groups
  outnumber index_topk.

The pages do not define the scoring itself (the same PR leaves it out of
scope), so this selects from given scores.  The offsets are the canonical
row list of ``sparse_attention.gather_plan``.

The order is a reading, since the pages fix none:
* descending score;
* ties by ascending id;
* -0.0 below +0.0;
* a NaN score below every number, -inf included.

It is a total order, so the selected list is unique and parity with it is
bit-exact.  With ``by_id`` the same selection is listed in ascending id
order (the attention core takes a list as a set).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def order_key(scores: np.ndarray) -> np.ndarray:
    """uint32 keys whose unsigned order is the order above, for float32
    scores: a non-negative float sets the top bit, a negative one is
    bit-inverted (so larger magnitudes rank lower), and NaN maps to 0."""
    bits = np.ascontiguousarray(scores, dtype=np.float32).view(np.uint32)
    key = np.where(bits >> 31, ~bits, bits | np.uint32(0x80000000)).astype(np.uint32)
    return np.where(np.isnan(scores), np.uint32(0), key).astype(np.uint32)


def topk_select(scores: np.ndarray, n_valid: np.ndarray, k: int,
                by_id: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """For each row i, the min(k, n_i) highest of scores[i, :n_i] (n_i is
    n_valid[i] clamped to [0, row length]), in the order above, or by
    ascending id with ``by_id``.

    Returns (ids int32 [rows, k], -1 past the count; counts int32 [rows])."""
    scores = np.asarray(scores, dtype=np.float32)
    rows, ld = scores.shape
    ids = np.full((rows, k), -1, dtype=np.int32)
    cnt = np.zeros(rows, dtype=np.int32)
    for i in range(rows):
        n = int(min(max(int(n_valid[i]), 0), ld))
        keys = order_key(scores[i, :n]).astype(np.int64)
        order = np.lexsort((np.arange(n), -keys))     # primary: key descending; then id ascending
        take = min(k, n)
        ids[i, :take] = np.sort(order[:take]) if by_id else order[:take]
        cnt[i] = take
    return ids, cnt
