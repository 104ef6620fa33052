"""Dense attention with an explicit per-head visibility mask (float64, numpy).

Test infrastructure: see the package docstring. Nothing here touches pages.

Definition (page "RedKnot SegPagedAttention runtime design", sections 1 and 4; page "RedKnot
head classification", head types): for request b with context length L and query chunk of
q tokens, query token t sits at absolute position p = L - q + t. Query head hq reads KV head
h = hq // G (G = Hq / Hkv, contiguous groups). The keys it may see are

* GLOBAL head: every position j with j <= p;
* LOCAL head (sink S, window W): j <= p and (j < S or j > p - W), i.e. the first S tokens
  plus the W most recent tokens up to and including p;
* adaptive LOCAL head: a LOCAL head with W = max(1, L // d) for the request's context length
  L (``plan.head_policy``);
* RETRIEVAL head: j <= p and (j is one of the head's kept prefix tokens or j >= L - q, the
  query chunk), the kept tokens chosen from an importance input (``plan.retrieval_keep``).

O[b, t, hq] = sum_j softmax_j(scale * <Q, K_j>) V_j over the visible j, with the softmax
taken over the visible set only (masked logits are -inf).
"""

from __future__ import annotations

import numpy as np

from .plan import GLOBAL, LOCAL, RETRIEVAL, head_policy, retrieval_keep

# Rows of one (request, head) are processed a slice at a time so that the dense logits stay
# within a bounded amount of memory. Each output row is independent of the others, so this
# only chooses which outputs are computed together.
_MAX_LOGITS = 1 << 24


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (uint16) or of float32 values."""
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def visible(kind: int, sink: int, window: int, p, j, kept=None, chunk0: int = 0):
    """Boolean visibility of key position ``j`` to a query at position ``p`` (broadcasts).
    RETRIEVAL heads also take their kept prefix positions and the chunk's first position."""
    causal = j <= p
    if kind == GLOBAL:
        return causal
    if kind == LOCAL:
        return causal & ((j < sink) | (j > p - window))
    if kind == RETRIEVAL:
        return causal & (np.isin(j, np.asarray(kept, dtype=np.int64)) | (j >= chunk0))
    raise ValueError(kind)


def _head_rows(q_rows, positions, k_head, v_head, kind, sink, window, scale, kept=None,
               chunk0=0):
    """O rows for one (request, query head): q_rows [R, D], positions [R], K/V [L, D]."""
    L = k_head.shape[0]
    out = np.empty((q_rows.shape[0], v_head.shape[1]), dtype=np.float64)
    if q_rows.shape[0] == 0:
        return out
    j = np.arange(L)
    step = max(1, _MAX_LOGITS // max(1, L))
    for r0 in range(0, q_rows.shape[0], step):
        r1 = min(q_rows.shape[0], r0 + step)
        logits = scale * (q_rows[r0:r1] @ k_head.T)
        mask = visible(kind, sink, window, positions[r0:r1, None], j[None, :], kept, chunk0)
        logits = np.where(mask, logits, -np.inf)
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        prob = e / e.sum(axis=1, keepdims=True)
        out[r0:r1] = prob @ v_head
    return out


def attention_rows(q, k, v, ctx_len, q_len, policy, Hq: int, Hkv: int, scale: float,
                   dtype: str, b: int, hq: int, tokens=None, importance=None) -> np.ndarray:
    """O[b, tokens, hq] in float64, shape [len(tokens), D].

    ``q`` is [sum(q_len), Hq, D] and ``k``/``v`` are [sum(ctx_len), Hkv, D] (token-major,
    requests concatenated); bf16 inputs are uint16 bit patterns. ``policy`` is [Hkv, 3] =
    (kind, sink, window), kinds GLOBAL, LOCAL, LOCAL_ADAPTIVE or RETRIEVAL. ``tokens`` indexes
    the request's query chunk (default: all). ``importance`` [sum(ctx_len), Hkv] (float32) is
    needed when the head is a RETRIEVAL head.
    """
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    q_len = np.asarray(q_len, dtype=np.int64)
    G = Hq // Hkv
    h = hq // G
    L = int(ctx_len[b])
    nq = int(q_len[b])
    kv0 = int(ctx_len[:b].sum())
    q0 = int(q_len[:b].sum())
    if tokens is None:
        tokens = np.arange(nq)
    tokens = np.asarray(tokens, dtype=np.int64)
    kind, sink, window = head_policy(*(int(x) for x in policy[h]), L)
    q_rows = to_f64(q[q0 + tokens, hq, :], dtype)
    k_head = to_f64(k[kv0:kv0 + L, h, :], dtype)
    v_head = to_f64(v[kv0:kv0 + L, h, :], dtype)
    positions = L - nq + tokens
    kept = None
    if kind == RETRIEVAL:
        kept = retrieval_keep(importance[kv0:kv0 + L, h], sink, window, L, nq)
    return _head_rows(q_rows, positions, k_head, v_head, kind, sink, window, scale, kept,
                      L - nq)


def attention_group_rows(q, k, v, ctx_len, q_len, policy, Hq: int, Hkv: int, scale: float,
                         dtype: str, b: int, h: int, tokens=None,
                         importance=None) -> np.ndarray:
    """O[b, tokens, hq] for every query head hq of KV head h's group, float64, shape
    [G, len(tokens), D]. The same rows as ``attention_rows`` called once per query head
    hq = h*G .. h*G+G-1; the group's K/V (and kept set) are converted once for all of them."""
    ctx_len = np.asarray(ctx_len, dtype=np.int64)
    q_len = np.asarray(q_len, dtype=np.int64)
    G = Hq // Hkv
    L = int(ctx_len[b])
    nq = int(q_len[b])
    kv0 = int(ctx_len[:b].sum())
    q0 = int(q_len[:b].sum())
    if tokens is None:
        tokens = np.arange(nq)
    tokens = np.asarray(tokens, dtype=np.int64)
    kind, sink, window = head_policy(*(int(x) for x in policy[h]), L)
    k_head = to_f64(k[kv0:kv0 + L, h, :], dtype)
    v_head = to_f64(v[kv0:kv0 + L, h, :], dtype)
    positions = L - nq + tokens
    kept = None
    if kind == RETRIEVAL:
        kept = retrieval_keep(importance[kv0:kv0 + L, h], sink, window, L, nq)
    out = np.empty((G, len(tokens), v.shape[-1]), dtype=np.float64)
    for g in range(G):
        q_rows = to_f64(q[q0 + tokens, h * G + g, :], dtype)
        out[g] = _head_rows(q_rows, positions, k_head, v_head, kind, sink, window, scale, kept,
                            L - nq)
    return out


def attention(q, k, v, ctx_len, q_len, policy, Hq: int, Hkv: int, scale: float,
              dtype: str, importance=None) -> np.ndarray:
    """Full O [sum(q_len), Hq, D] in float64."""
    ctx_len = np.asarray(ctx_len)
    q_len = np.asarray(q_len)
    D = q.shape[-1]
    out = np.zeros((int(q_len.sum()), Hq, D), dtype=np.float64)
    q0 = 0
    for b in range(len(ctx_len)):
        nq = int(q_len[b])
        for hq in range(Hq):
            out[q0:q0 + nq, hq, :] = attention_rows(q, k, v, ctx_len, q_len, policy, Hq, Hkv,
                                                    scale, dtype, b, hq, importance=importance)
        q0 += nq
    return out
