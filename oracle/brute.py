"""Pure-Python brute force for tiny inputs (float loops, ``math.exp``).

Test infrastructure: used only to pin ``oracle.attention``. The visible set is built here
constructively, as a union of index ranges, rather than as the predicate the numpy oracle
evaluates, so a slip in either form shows up as a mismatch.
"""

from __future__ import annotations

import math


def visible_set(kind: int, sink: int, window: int, p: int):
    """Sorted key positions a query at position p may read (kind 0 GLOBAL, 1 LOCAL)."""
    if kind == 0:
        return list(range(0, p + 1))
    recent = set(range(max(0, p - window + 1), p + 1))
    first = set(range(0, min(sink, p + 1)))
    return sorted(recent | first)


def attention_row(q_row, k_rows, v_rows, p: int, kind: int, sink: int, window: int,
                  scale: float):
    """One output row: plain lists of floats in, list of floats out."""
    vis = visible_set(kind, sink, window, p)
    logits = []
    for j in vis:
        acc = 0.0
        for a, c in zip(q_row, k_rows[j]):
            acc += a * c
        logits.append(scale * acc)
    mx = max(logits)
    w = [math.exp(x - mx) for x in logits]
    tot = sum(w)
    d = len(v_rows[0])
    out = [0.0] * d
    for wi, j in zip(w, vis):
        for c in range(d):
            out[c] += (wi / tot) * v_rows[j][c]
    return out


def retrieval_kept(importance, sink: int, permille: int, prefix: int):
    """Kept prefix positions of a RETRIEVAL head, found by repeatedly taking the most important
    token not yet taken (scanning positions upward, so a tie goes to the lower position)."""
    first = list(range(min(sink, prefix)))
    rest = list(range(len(first), prefix))
    k = (permille * len(rest) + 999) // 1000
    chosen = []
    for _ in range(k):
        best = None
        for j in rest:
            if j in chosen:
                continue
            if best is None or importance[j] > importance[best]:
                best = j
        chosen.append(best)
    return sorted(first + chosen)


def attention_row_over(q_row, k_rows, v_rows, vis, scale: float):
    """One output row over an explicit list of visible key positions."""
    logits = [scale * sum(a * c for a, c in zip(q_row, k_rows[j])) for j in vis]
    mx = max(logits)
    w = [math.exp(x - mx) for x in logits]
    tot = sum(w)
    out = [0.0] * len(v_rows[0])
    for wi, j in zip(w, vis):
        for c in range(len(out)):
            out[c] += (wi / tot) * v_rows[j][c]
    return out
