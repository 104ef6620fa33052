"""CPU oracle for head-aware SegPaged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import anything from here. The product path (the HIP library and its Python binding) never
imports, links or calls this package, and this package never imports the product.

What it computes, and from which passage of the RedKnot pages:

* ``attention``: dense attention in float64 with an explicit per-head visibility mask. The
  pages state that SegPagedAttention changes only the storage layout and must reproduce the
  dense-plus-mask result (page "RedKnot SegPagedAttention runtime design", section 4:
  the cosine check against a dense-plus-mask baseline must exceed 0.99998). GLOBAL heads read
  the whole prefix and LOCAL heads read the first S sink tokens plus a recent window of W
  tokens (same page, sections 1-3; page "RedKnot head classification", the four head types,
  defaults window 512 and sink 4). So the oracle is that definition written out. An adaptive
  LOCAL head has window max(1, L // d) for a request of context length L (page "RedKnot head
  classification", windows that scale with the request's context). A RETRIEVAL head sees the
  top fraction of its prefix tokens by an importance input, its sink and its query chunk
  (same page, the four head types; page "RedKnot SegPagedAttention runtime design", closing
  summary: retrieval heads take pages on demand).
* ``plan``: the per-(request, KV head) segment list, true KV length, virtual page ids and the
  virtual-to-physical map (page "RedKnot SegPagedAttention runtime design", section 3: one
  page table per (layer, head, segment) over contiguous virtual pages, a shared physical
  pool, LOCAL heads allocate only sink + recent pages).
* ``append``: the growable page layout (each segment owns pages for a reserve of decode
  tokens) and the decode-time append, where a LOCAL head's recent segment is a ring of whole
  pages whose oldest page is recycled once it falls out of the window (page "RedKnot
  SegPagedAttention runtime design", section 3: LOCAL storage does not grow with the context;
  the product overview page, section 3.2: idle pages are reclaimed).
* ``brute``: pure-Python float loops on tiny inputs, used to pin ``attention``.

Parity status: every function here is pinned by tests under ``tests/test_oracle_*.py``
(brute force, closed forms, library special cases, invariants and a hand-derived worked
example). Nothing here is "parity unpinned".
"""

from .attention import (GLOBAL, LOCAL, attention, attention_group_rows,  # noqa: F401
                        attention_rows, to_f64, visible)
from .plan import (LOCAL_ADAPTIVE, RETRIEVAL, gather_positions, head_policy,  # noqa: F401
                   plan_tables, plan_tables_layers, retrieval_counts, retrieval_keep, segments)
from .append import append_step, grow_tables, owned_pages  # noqa: F401
