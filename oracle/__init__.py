"""FP64 CPU oracle for sparse paged attention with a sink.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The HIP library never does, and this package imports nothing from
the HIP library or its Python binding: the two share no code.

The oracle is the plain definition of the method, written for a reader to
check against the pages by eye: gather each query's KV set through the page
tables, score it, and take one softmax whose denominator also holds the
per-head sink logit (which has no value row).  Everything runs in float64.

Modules:
  formats    bf16, OCP e4m3 and FNUZ e4m3 decoding (exact, to float64)
  sparse_attention  KV-set metadata, gather, attention with sink, (O, LSE) merge
  topk       top-k selection of compressed groups from per-token scores
  backward   gradients of q, the caches and the sink (float64)
  compare    the acceptance comparator

Every function cites the passage it follows.  Pins live in
``tests/test_oracle_*.py``.
"""
from .formats import bf16_to_f64, e4m3_table, e4m3_to_f64, e4m3fnuz_table, e4m3fnuz_to_f64  # noqa: F401
from .sparse_attention import (  # noqa: F401
    KVSet, kv_set, kv_sets, gather_rows, attend, attend_partial, merge, attention,
    gather_plan, partial_split, physical_rows, query_f64, lse_merge_arrays,
)
from .compare import accept, AcceptReport  # noqa: F401
from .topk import order_key, topk_select  # noqa: F401
from .backward import Grads, attention_backward, backward_values  # noqa: F401
