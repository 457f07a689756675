"""CPU oracle for anchor-masked block-sparse cross-attention (test infrastructure).

This package is test infrastructure only.  It is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``;
the product path (the HIP library and its Python binding) never imports, links
or calls it, and it shares no code with that path.

Everything here is plain numpy in float64, written from the Split-KV
description of what is computed:

* ``attention``  - the masked softmax forward (partial output + log-sum-exp)
  and its backward, per "Split-KV speeds diffusion drafter training..." section
  "Why short queries change the problem" (the mask) and section "Exchange the
  smaller side" (keys/values stay local; partials carry normalisation
  statistics);
* ``combine``    - the exact merge of partials from their log-sum-exp
  statistics (same page, section "Exchange the smaller side");
* ``cost``       - the per-chunk realised attention cost, by brute force over
  (query, key) pairs (same page, section "Balance actual attention work");
* ``lpt``        - longest-processing-time-first assignment with equal chunk
  counts (same section);
* ``dense``      - a textbook dense masked softmax used only to pin the above.
"""

from .attention import allowed_local_rows, sparse_xattn_fwd, sparse_xattn_bwd
from .combine import lse_combine
from .cost import chunk_cost, chunk_cost_one, total_pairs
from .lpt import lpt_assign, imbalance
from .dense import dense_mask, dense_fwd

__all__ = [
    "allowed_local_rows", "sparse_xattn_fwd", "sparse_xattn_bwd", "lse_combine",
    "chunk_cost", "chunk_cost_one", "total_pairs", "lpt_assign", "imbalance",
    "dense_mask", "dense_fwd",
]
