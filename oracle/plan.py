"""Page-plan oracle: segments, true KV lengths, virtual pages and the physical map.

Test infrastructure: see the package docstring. Pure Python integer code.

Source: page "RedKnot SegPagedAttention runtime design", section 3 -- each (layer, head,
segment) maps to contiguous virtual pages; the page table records, per head, the page numbers
of its segments, its policy and its segment list; a shared physical pool where LOCAL heads
allocate only sink + recent pages and GLOBAL heads the full context; a virtual-to-physical map
keeps pages apart; the builder keeps only the tokens a LOCAL head can see. Section 4: the
attention call reads each head's true KV length from its page table.

Readings taken where the pages are silent (one layer per call):

* A LOCAL head must store every token some query of the chunk can see. The chunk's queries
  sit at positions L-q .. L-1, so the recent part starts at R0 = max(0, L - q - W + 1).
* Segments, in position order: GLOBAL -> (0, L). LOCAL -> (0, L) when R0 <= S (sink and
  window touch or overlap); else (R0, L - R0) when S = 0; else (0, S) and (R0, L - R0).
  A sink longer than the context is clipped to L. L = 0 stores nothing.
* Every segment starts on a fresh page; slot i of the segment's k-th page holds position
  pos_start + k*P + i. n_pages = ceil(n_tok / P).
* Virtual page ids are handed out in the order (request, head, segment); a segment's
  vpage_start is the running total of the pages before it.
* An unused segment slot reads (pos_start 0, n_tok 0, vpage_start = running total, n_pages 0).
* v2p[v] = free_pages[v]: physical pages are taken from the caller's free list in order.
* kv_len[b, h] = total stored tokens of the head.
* Several layers in one pool (same page, section 3: the page table is keyed by (layer, head,
  segment)): each layer's heads follow the rules above with that layer's policies, and virtual
  pages are handed out in (request, layer, head, segment) order; tables are stored per layer.
* An adaptive LOCAL head (page "RedKnot head classification", the passage on windows that
  scale with each request's context length, whose example is half the context) is a LOCAL
  head whose window for a request of context length L is max(1, L // d), d being its
  configured divisor; L is the request's whole context at this call, query chunk included.
* A RETRIEVAL head (page "RedKnot head classification", the four head types: full KV of which
  only the top-p important tokens are kept; page "RedKnot SegPagedAttention runtime design",
  closing summary: retrieval heads take only the pages they need) with sink S and keep fraction
  p = window / 1000 keeps, of the prefix before the query chunk (positions < L - q): its first
  min(S, L - q) tokens, and of the others the ceil(p * n) with the highest importance (n =
  their count; importance is an input, one float per (token, KV head); ties go to the lower
  position). It also keeps the whole chunk, which its own queries see causally. Segments: the
  kept prefix tokens compacted in position order (slot i of the segment holds the i-th kept
  position; pos_start reads 0), then the chunk (L - q, q); a head with an empty prefix has the
  chunk alone. The count of kept tokens depends only on (L, q, S, p), so the tables do too;
  which tokens fill the first segment depends on the importance.
"""

from __future__ import annotations

import numpy as np

GLOBAL = 0
LOCAL = 1
LOCAL_ADAPTIVE = 2
RETRIEVAL = 3


def head_policy(kind: int, sink: int, window: int, L: int):
    """(kind, sink, window) of one head for a request of context length L: an adaptive LOCAL
    head (``window`` = divisor d) becomes LOCAL with window max(1, L // d)."""
    if kind == LOCAL_ADAPTIVE:
        return LOCAL, sink, max(1, L // window)
    return kind, sink, window


def retrieval_counts(sink: int, permille: int, L: int, q: int):
    """(sink tokens kept, other prefix tokens kept) of a RETRIEVAL head."""
    prefix = max(0, L - q)
    s = min(sink, prefix)
    n = prefix - s
    return s, -(-permille * n // 1000)


def retrieval_keep(importance, sink: int, permille: int, L: int, q: int):
    """Kept prefix positions of a RETRIEVAL head, ascending. importance[j] for j < L - q."""
    s, k = retrieval_counts(sink, permille, L, q)
    prefix = max(0, L - q)
    others = sorted(range(s, prefix), key=lambda j: (-float(importance[j]), j))
    return sorted(list(range(s)) + others[:k])


def segments(kind: int, sink: int, window: int, L: int, q: int):
    """List of (pos_start, n_tok) for one (request, KV head)."""
    if L <= 0:
        return []
    if kind == GLOBAL:
        return [(0, L)]
    if kind == RETRIEVAL:
        s, k = retrieval_counts(sink, window, L, q)
        segs = [(0, s + k)] if s + k > 0 else []
        return segs + ([(L - q, q)] if q > 0 else [])
    if kind != LOCAL:
        raise ValueError(kind)
    s = min(sink, L)
    r0 = max(0, L - q - window + 1)
    if r0 <= s:
        return [(0, L)]
    if s == 0:
        return [(r0, L - r0)]
    return [(0, s), (r0, L - r0)]


def plan_tables(ctx_len, q_len, policy, P: int):
    """Returns (seg_table int32 [B, Hkv, 2, 4], kv_len int32 [B, Hkv], n_virt)."""
    B = len(ctx_len)
    Hkv = len(policy)
    seg_table = np.zeros((B, Hkv, 2, 4), dtype=np.int32)
    kv_len = np.zeros((B, Hkv), dtype=np.int32)
    v = 0
    for b in range(B):
        L = int(ctx_len[b])
        q = int(q_len[b])
        for h in range(Hkv):
            kind, sink, window = head_policy(*(int(x) for x in policy[h]), L)
            segs = segments(kind, sink, window, L, q)
            total = 0
            for s in range(2):
                if s < len(segs):
                    pos, n = segs[s]
                    npg = -(-n // P)
                    seg_table[b, h, s] = (pos, n, v, npg)
                    v += npg
                    total += n
                else:
                    seg_table[b, h, s] = (0, 0, v, 0)
            kv_len[b, h] = total
    return seg_table, kv_len, v


def plan_tables_layers(ctx_len, q_len, policies, P: int):
    """Several layers in one pool: policies [n_layers][Hkv][3]. Returns (seg_table int32
    [n_layers, B, Hkv, 2, 4], kv_len int32 [n_layers, B, Hkv], n_virt)."""
    policies = np.asarray(policies, dtype=np.int64)
    n_layers, Hkv = policies.shape[0], policies.shape[1]
    B = len(ctx_len)
    seg_table = np.zeros((n_layers, B, Hkv, 2, 4), dtype=np.int32)
    kv_len = np.zeros((n_layers, B, Hkv), dtype=np.int32)
    v = 0
    for b in range(B):  # virtual pages: request, then layer, then head, then segment
        L, q = int(ctx_len[b]), int(q_len[b])
        for layer in range(n_layers):
            for h in range(Hkv):
                kind, sink, window = head_policy(*(int(x) for x in policies[layer, h]), L)
                segs = segments(kind, sink, window, L, q)
                for s in range(2):
                    if s < len(segs):
                        pos, n = segs[s]
                        npg = -(-n // P)
                        seg_table[layer, b, h, s] = (pos, n, v, npg)
                        v += npg
                        kv_len[layer, b, h] += n
                    else:
                        seg_table[layer, b, h, s] = (0, 0, v, 0)
    return seg_table, kv_len, v


def gather_positions(seg_table, v2p, P: int, b: int, h: int, kept=None):
    """(position, physical page, slot) of every token stored for (b, h), in position order.
    ``kept``: the kept prefix positions of a RETRIEVAL head, whose first segment holds them."""
    out = []
    for s in range(2):
        pos, n, vstart, npg = (int(x) for x in seg_table[b, h, s])
        for i in range(n):
            vpage = vstart + i // P
            p = int(kept[i]) if (s == 0 and kept is not None and len(kept)) else pos + i
            out.append((p, int(v2p[vpage]), i % P))
    return out
