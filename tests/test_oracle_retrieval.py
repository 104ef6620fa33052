"""Pins of the RETRIEVAL head in the oracle (CPU): ``plan.retrieval_keep`` / ``segments`` and
``attention`` with an importance input.

Checked against: pure-Python brute force whose kept set comes from repeated arg-max selection
(not a sort) and whose visible set is built as a union; the full-keep case equal to GLOBAL; tied
importance keeping the earliest tokens; the zero-query closed form (mean of V over the visible
set); hand-derived counts and tables; the stored set equal to the union of the chunk's visible
sets.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import GLOBAL, LOCAL, RETRIEVAL, attention, brute
from workloads import custom_case, importance_scores


def _case(seed, dtype, Hkv, G, D, ctx, ql, pol, scale=None):
    return custom_case(seed, dtype=dtype, Hq=Hkv * G, Hkv=Hkv, D=D, P=16, ctx_len=ctx,
                       q_len=ql, policy=pol, scale=scale)


@pytest.mark.parametrize("trial", range(12))
def test_against_brute_force(trial):
    rng = np.random.default_rng(300 + trial)
    Hkv, G, D = int(rng.integers(1, 4)), int(rng.choice([1, 2])), int(rng.integers(2, 7))
    B = int(rng.integers(1, 4))
    ctx = [int(rng.integers(1, 49)) for _ in range(B)]
    ql = [int(rng.integers(1, c + 1)) for c in ctx]
    pol = [(RETRIEVAL, int(rng.integers(0, 6)), int(rng.integers(1, 1001))) if h % 2 == 0 else
           (LOCAL, int(rng.integers(0, 4)), int(rng.integers(1, 20))) for h in range(Hkv)]
    dtype = "f32" if trial % 2 else "bf16"
    c = _case(40 + trial, dtype, Hkv, G, D, ctx, ql, pol, scale=float(rng.choice([0.4, 1.0])))
    imp = importance_scores(c, levels=3 if trial % 3 == 0 else 0)
    got = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv, c.scale, dtype,
                    importance=imp)
    k64, v64, q64 = (oracle.to_f64(x, dtype) for x in (c.k, c.v, c.q))
    kv0 = q0 = 0
    for b in range(B):
        L, nq = ctx[b], ql[b]
        for hq in range(c.Hq):
            h = hq // G
            kind, sink, window = pol[h]
            for t in range(nq):
                p = L - nq + t
                if kind == RETRIEVAL:
                    kept = brute.retrieval_kept(imp[kv0:kv0 + L, h].tolist(), sink, window, L - nq)
                    vis = sorted(set(kept) | set(range(L - nq, p + 1)))
                else:
                    vis = brute.visible_set(kind, sink, window, p)
                ref = brute.attention_row_over(q64[q0 + t, hq].tolist(),
                                               k64[kv0:kv0 + L, h].tolist(),
                                               v64[kv0:kv0 + L, h].tolist(), vis, c.scale)
                np.testing.assert_allclose(got[q0 + t, hq], ref, rtol=1e-12, atol=1e-12)
        kv0 += L
        q0 += nq


def test_full_keep_equals_global():
    pol_r = [(RETRIEVAL, 3, 1000), (RETRIEVAL, 0, 1000)]
    pol_g = [(GLOBAL, 0, 1), (GLOBAL, 0, 1)]
    c = _case(60, "bf16", 2, 2, 16, [90, 37], [20, 1], pol_r)
    imp = importance_scores(c)  # all positive: the full fraction keeps every prefix token
    a = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, pol_r, c.Hq, c.Hkv, c.scale, "bf16",
                  importance=imp)
    b = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, pol_g, c.Hq, c.Hkv, c.scale, "bf16")
    np.testing.assert_array_equal(a, b)


def test_tied_importance_keeps_the_earliest_tokens():
    imp = np.zeros(100, dtype=np.float32)
    kept = oracle.retrieval_keep(imp, 4, 250, 100, 10)
    assert kept == list(range(4 + 22))  # 4 sink + ceil(0.25 * 86) = 22
    imp[50] = 1.0
    imp[70] = 1.0
    kept = oracle.retrieval_keep(imp, 4, 30, 100, 10)  # ceil(0.03 * 86) = 3
    assert kept == [0, 1, 2, 3, 4, 50, 70]


def test_zero_query_closed_form():
    # With Q = 0 every visible key has the same logit, so O is the mean of V over the visible
    # set: the sink, the kept prefix tokens and the chunk up to the query.
    c = _case(61, "f32", 1, 1, 8, [60], [9], [(RETRIEVAL, 2, 400)])
    c.q[:] = 0
    imp = importance_scores(c)
    got = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, 1, 1, 1.0, "f32",
                    importance=imp)
    kept = oracle.retrieval_keep(imp[:, 0], 2, 400, 60, 9)
    assert len(kept) == 2 + math.ceil(0.4 * 49)
    for t in range(9):
        vis = kept + list(range(51, 51 + t + 1))
        np.testing.assert_allclose(got[t, 0], c.v[vis, 0].astype(np.float64).mean(axis=0),
                                   rtol=1e-12, atol=1e-12)


def test_segments_and_tables_worked_example():
    # L = 100, q = 10, S = 4, p = 250: prefix 90 tokens, 4 sink + ceil(0.25 * 86) = 22 kept,
    # then the 10-token chunk. Page size 16: 2 + 1 pages.
    assert oracle.segments(RETRIEVAL, 4, 250, 100, 10) == [(0, 26), (90, 10)]
    assert oracle.segments(RETRIEVAL, 4, 250, 10, 10) == [(0, 10)]  # no prefix: chunk only
    assert oracle.segments(RETRIEVAL, 4, 1, 6, 1) == [(0, 5), (5, 1)]  # 4 sink + ceil(0.001)
    st, kl, nv = oracle.plan_tables([100, 10], [10, 10], [(RETRIEVAL, 4, 250)], 16)
    assert st[0, 0].tolist() == [[0, 26, 0, 2], [90, 10, 2, 1]]
    assert st[1, 0].tolist() == [[0, 10, 3, 1], [0, 0, 4, 0]]
    assert kl.tolist() == [[36], [10]] and nv == 4


def test_stored_set_is_union_of_visible_sets_and_gather():
    rng = np.random.default_rng(62)
    for _ in range(40):
        L = int(rng.integers(1, 200))
        q = int(rng.integers(1, L + 1))
        S, pm = int(rng.integers(0, 8)), int(rng.integers(1, 1001))
        c = _case(63, "f32", 1, 1, 4, [L], [q], [(RETRIEVAL, S, pm)])
        imp = importance_scores(c, levels=int(rng.integers(0, 4)))
        kept = oracle.retrieval_keep(imp[:, 0], S, pm, L, q)
        j = np.arange(L)
        union = set()
        for p in range(L - q, L):
            vis = oracle.visible(RETRIEVAL, S, pm, p, j, kept, L - q)
            union |= set(np.nonzero(vis)[0].tolist())
        st, kl, nv = oracle.plan_tables([L], [q], [(RETRIEVAL, S, pm)], 16)
        got = oracle.gather_positions(st, np.arange(nv), 16, 0, 0, kept)
        stored = [g[0] for g in got]
        assert stored == sorted(union) and len(stored) == kl[0, 0]
