"""Growable page layout and decode-time append -- TEST INFRASTRUCTURE ONLY (see the package
docstring). Pure Python integer code.

What the pages fix:

* Page "RedKnot SegPagedAttention runtime design", section 3: each (layer, head, segment) owns
  contiguous virtual pages of one shared physical pool, reached through a virtual-to-physical
  map; LOCAL heads hold only sink and recent pages, so what a LOCAL head occupies does not
  grow with the total context; GLOBAL heads hold the whole context.
* Same page, section 5: layout work belongs to KV-write time and is then reused.
* Page "RedKnot：小红书开源的长上下文LLM推理优化工具…" (the product overview), section 3.2,
  items (1) and (3): LOCAL heads cache a bounded length of KV, and idle pages are reclaimed
  dynamically.

The pages give no decode-time algorithm; the readings taken here:

1. A decode step appends one token per request at position L (the old context length); the
   context becomes L + 1 and the step's query sits at position L. Its K/V rows are stored
   before that query attends (a query sees itself).
2. Growable layout: the segments, positions and page order of ``plan.plan_tables`` for the
   build's (ctx_len, q_len), but each segment owns enough contiguous virtual pages for
   ``reserve[b]`` more tokens; all owned pages are mapped at build (v2p[v] = free_pages[v]).
   Field 3 of a segment row is the number of pages it owns; with reserve 0 it equals the
   pages it uses, so the table is exactly ``plan.plan_tables``'s.
3. Ring: the recent segment of a LOCAL head is a ring of whole pages. After each append its
   oldest pages whose tokens all lie before the next query's window (positions < L + 1 - W)
   are dropped: pos_start advances P per page and the dropped physical pages move to the end
   of the segment's page list (its v2p entries rotate), where later tokens reuse them. A ring
   therefore keeps at most W + P - 1 tokens, the stale ones (fewer than P) being older than
   the window; attention masks them by position.
4. A LOCAL head with S > 0 whose sink and window touch is one segment (0, L). It grows as one
   segment until the window start reaches S_pg = ceil(S / P) * P, the first page boundary past
   the sink; then it splits into the sink (0, S) on its first ceil(S / P) pages and a ring
   starting at S_pg on the remaining owned pages. With S = 0 the only segment is the ring.
5. Owned pages = the most the segment can use while the context grows to Lmax = L + reserve:
   GLOBAL ceil(Lmax / P); a ring whose build pos_start is o: max(ceil((L - o) / P),
   ceil(min(Lmax - o, W + P - 1) / P)); a one-segment LOCAL head with S > 0: the largest of
   ceil(L / P), ceil(min(Lmax, S_pg + W - 1) / P) (before the split) and, if Lmax >= S_pg + W,
   ceil(S / P) + ceil(min(Lmax - S_pg, W + P - 1) / P) (after it); a sink segment its pages.
   Appending into a full segment is an error.
6. Context-adaptive LOCAL windows change W as the context grows; they are not growable here.
7. A RETRIEVAL head grows like a GLOBAL one: appended tokens join its last segment, the query
   chunk, which owns ceil((q + reserve) / P) pages; its kept prefix segment never changes. A
   growable request needs a non-empty chunk (q >= 1) for its retrieval heads.
"""

from __future__ import annotations

import numpy as np

from .plan import GLOBAL, LOCAL, RETRIEVAL, segments


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def owned_pages(kind: int, sink: int, window: int, L: int, q: int, reserve: int, P: int):
    """(segments, pages owned by each) of one (request, KV head) in the growable layout."""
    segs = segments(kind, sink, window, L, q)
    if not segs:
        return segs, []
    lmax = L + reserve
    if kind == GLOBAL:
        return segs, [_cdiv(lmax, P)]
    if kind == RETRIEVAL:  # the chunk (the last segment) grows; the kept prefix does not
        own = [_cdiv(n, P) for _, n in segs]
        own[-1] = _cdiv(segs[-1][1] + reserve, P)
        return segs, own
    if sink > 0 and len(segs) == 1:  # sink and window in one segment (0, L)
        s_pg = _cdiv(sink, P) * P
        own = max(_cdiv(L, P), _cdiv(min(lmax, s_pg + window - 1), P))
        if lmax >= s_pg + window:
            own = max(own, _cdiv(sink, P) + _cdiv(min(lmax - s_pg, window + P - 1), P))
        return segs, [own]
    own = [_cdiv(n, P) for _, n in segs]
    o, n = segs[-1]  # the ring: the only segment (S = 0) or the one after the sink
    own[-1] = max(_cdiv(n, P), _cdiv(min(lmax - o, window + P - 1), P))
    return segs, own


def grow_tables(ctx_len, q_len, reserve, policy, P: int):
    """Growable layout: (seg_table int32 [B, Hkv, 2, 4], kv_len int32 [B, Hkv], n_virt)."""
    B, Hkv = len(ctx_len), len(policy)
    seg_table = np.zeros((B, Hkv, 2, 4), dtype=np.int32)
    kv_len = np.zeros((B, Hkv), dtype=np.int32)
    v = 0
    for b in range(B):
        L, q, R = int(ctx_len[b]), int(q_len[b]), int(reserve[b])
        if R < 0 or (R > 0 and L < 1):
            raise ValueError("a request that grows needs a non-empty context")
        for h in range(Hkv):
            kind, sink, window = (int(x) for x in policy[h])
            if kind not in (GLOBAL, LOCAL, RETRIEVAL):
                raise ValueError("growable layouts take GLOBAL, LOCAL and RETRIEVAL heads")
            if kind == RETRIEVAL and R > 0 and q < 1:
                raise ValueError("a growing retrieval head needs a non-empty query chunk")
            segs, own = owned_pages(kind, sink, window, L, q, R, P)
            for s in range(2):
                if s < len(segs):
                    pos, n = segs[s]
                    seg_table[b, h, s] = (pos, n, v, own[s])
                    v += own[s]
                    kv_len[b, h] += n
                else:
                    seg_table[b, h, s] = (0, 0, v, 0)
    return seg_table, kv_len, v


def append_step(seg_table, kv_len, v2p, policy, P: int, n_new=None):
    """One decode append (readings 1, 3, 4). n_new[b] in {0, 1} (None: every request).

    Returns new (seg_table, kv_len, v2p) and the writes [(b, h, position, phys, slot)]: the new
    token of request b, KV head h, goes to slot ``slot`` of physical page ``phys``.
    """
    st = np.array(seg_table, dtype=np.int64)
    kl = np.array(kv_len, dtype=np.int64)
    vp = [int(x) for x in v2p]
    B, Hkv = st.shape[0], st.shape[1]
    writes = []
    for b in range(B):
        if n_new is not None and int(n_new[b]) == 0:
            continue
        for h in range(Hkv):
            kind, sink, window = (int(x) for x in policy[h])
            rows = [[int(x) for x in st[b, h, s]] for s in range(2)]
            ends = [r[0] + r[1] for r in rows if r[1] > 0]
            if not ends:
                raise ValueError("nothing stored for (%d, %d)" % (b, h))
            L = max(ends)  # the newest stored token is the last one of the context
            r0 = max(0, L + 1 - window)  # window start of the query at position L
            target = 0
            if kind == RETRIEVAL:
                target = 1 if rows[1][3] > 0 else 0  # the query chunk
            if kind == LOCAL:
                ring = 0 if sink == 0 else None
                if sink > 0 and rows[1][3] > 0:
                    ring = 1
                elif sink > 0:  # still one segment (0, L)
                    s_pg = _cdiv(sink, P) * P
                    if r0 >= s_pg:  # split into sink and ring
                        pos0, n0, vs0, own0 = rows[0]
                        k_sink = _cdiv(sink, P)
                        rows[1] = [s_pg, n0 - s_pg, vs0 + k_sink, own0 - k_sink]
                        rows[0] = [0, sink, vs0, k_sink]
                        ring = 1
                if ring is not None:
                    pos, n, vs, own = rows[ring]
                    k = max(0, (r0 - pos) // P)  # whole pages older than the window
                    if k > 0:
                        pages = vp[vs:vs + own]
                        vp[vs:vs + own] = pages[k:] + pages[:k]
                        rows[ring] = [pos + k * P, n - k * P, vs, own]
                    target = ring
            pos, n, vs, own = rows[target]
            if n // P >= own:
                raise ValueError("segment full at (%d, %d)" % (b, h))
            writes.append((b, h, L, vp[vs + n // P], n % P))
            rows[target][1] = n + 1
            st[b, h] = rows
            kl[b, h] = rows[0][1] + rows[1][1]
    return st.astype(np.int32), kl.astype(np.int32), np.asarray(vp, dtype=np.int32), writes
