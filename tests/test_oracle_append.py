"""Pins of the growable layout and the decode append in oracle/append.py (CPU).

Checked against things other than the oracle itself: a hand-derived worked example, the
already-pinned build layout (reserve 0), and brute-force invariants of every state along
random append trajectories (each head stores every key the next decode query may see, stale
keys are few and older than the window, no segment outgrows its pages, no page changes owner,
no stored token is overwritten, LOCAL storage stays bounded).
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle.append import append_step, grow_tables, owned_pages
from oracle.attention import visible

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "append_example.json")


def test_worked_example():
    d = json.load(open(GOLDEN))
    P = d["page_size"]
    st, kl, nv = grow_tables(d["ctx_len"], d["q_len"], d["reserve"], d["policy"], P)
    np.testing.assert_array_equal(st, d["initial"]["seg_table"])
    np.testing.assert_array_equal(kl, d["initial"]["kv_len"])
    assert nv == d["initial"]["n_virt"]
    v2p = np.asarray(d["free_pages"][:nv], dtype=np.int32)
    for step in d["steps"]:
        st, kl, v2p, writes = append_step(st, kl, v2p, d["policy"], P)
        np.testing.assert_array_equal(st, step["seg_table"])
        np.testing.assert_array_equal(kl, step["kv_len"])
        assert v2p.tolist() == step["v2p"]
        assert [list(w) for w in writes] == step["writes"]


def _random_policy(rng, Hkv, P, retrieval=False):
    pol = []
    for h in range(Hkv):
        if h == 0 or rng.random() < 0.25:
            pol.append((oracle.GLOBAL, 0, 1))
        elif retrieval and rng.random() < 0.4:
            pol.append((oracle.RETRIEVAL, int(rng.integers(0, P)), int(rng.integers(1, 1001))))
        else:
            pol.append((oracle.LOCAL, int(rng.integers(0, 2 * P)), int(rng.integers(1, 5 * P))))
    return pol


@pytest.mark.parametrize("retrieval", [False, True])
def test_reserve_zero_is_the_build_layout(retrieval):
    rng = np.random.default_rng(11 + retrieval)
    for _ in range(200):
        P = int(rng.choice([4, 8, 16]))
        B, Hkv = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        ctx = rng.integers(0, 12 * P, size=B)
        q = np.array([int(rng.integers(0, c + 1)) if c else 0 for c in ctx])
        pol = _random_policy(rng, Hkv, P, retrieval)
        a = grow_tables(ctx, q, np.zeros(B, dtype=np.int64), pol, P)
        b = oracle.plan_tables(ctx, q, pol, P)
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])
        assert a[2] == b[2]


def _stored(st, v2p, P, b, h, kept=None):
    return oracle.gather_positions(st, v2p, P, b, h, kept)


def _head_pages(st, v2p, b, h):
    """Physical pages owned by (b, h): the v2p entries of its owned virtual ranges."""
    out = []
    for s in range(2):
        _, _, vs, own = (int(x) for x in st[b, h, s])
        out += [int(v2p[v]) for v in range(vs, vs + own)]
    return sorted(out)


def _trajectory(rng, P, B, Hkv, steps, pol=None, q_one=False, retrieval=False):
    ctx = rng.integers(1, 10 * P, size=B)
    q = np.ones(B, dtype=np.int64) if q_one else np.array([int(rng.integers(1, c + 1)) for c in ctx])
    reserve = np.full(B, steps, dtype=np.int64)
    pol = pol or _random_policy(rng, Hkv, P, retrieval)
    st, kl, nv = grow_tables(ctx, q, reserve, pol, P)
    v2p = rng.permutation(nv + 5)[:nv].astype(np.int32)  # a free list with spare pages
    return ctx, q, pol, st, kl, v2p


@pytest.mark.parametrize("retrieval", [False, True])
def test_append_trajectory_invariants(retrieval):
    # With RETRIEVAL heads, a stand-in keep list (every other prefix token, as many as the
    # head keeps) names the positions of the kept segment; growth never touches it.
    rng = np.random.default_rng(12 + retrieval)
    for case in range(60):
        P = int(rng.choice([4, 8, 16]))
        B, Hkv = int(rng.integers(1, 3)), int(rng.integers(2, 5))
        steps = int(rng.integers(1, 8 * P))
        ctx, q, pol, st, kl, v2p = _trajectory(rng, P, B, Hkv, steps, retrieval=retrieval)
        kept = {}
        for b in range(B):
            for h in range(Hkv):
                if pol[h][0] == oracle.RETRIEVAL and ctx[b] - q[b] > 0:
                    s_, k_ = oracle.retrieval_counts(pol[h][1], pol[h][2], ctx[b], q[b])
                    cand = list(range(s_, ctx[b] - q[b]))
                    kept[(b, h)] = list(range(s_)) + sorted(cand[::2] + cand[1::2])[:k_]
        owned0 = {(b, h): _head_pages(st, v2p, b, h) for b in range(B) for h in range(Hkv)}
        pool = {}
        for b in range(B):
            for h in range(Hkv):
                for pos, ph, sl in _stored(st, v2p, P, b, h, kept.get((b, h))):
                    assert (ph, sl) not in pool
                    pool[(ph, sl)] = (b, h, pos)
        L = ctx.copy()
        for t in range(steps):
            n_new = (rng.random(B) < 0.85).astype(np.int32)
            st, kl, v2p, writes = append_step(st, kl, v2p, pol, P, n_new)
            assert len(writes) == int(n_new.sum()) * Hkv
            for b, h, pos, ph, sl in writes:
                assert pos == L[b]
                pool[(ph, sl)] = (b, h, pos)
            L = L + n_new
            for b in range(B):
                for h in range(Hkv):
                    kind, sink, window = pol[h]
                    got = _stored(st, v2p, P, b, h, kept.get((b, h)))
                    pos = np.array(sorted(p for p, _, _ in got))
                    assert len(pos) == kl[b, h] and len(set(pos.tolist())) == len(pos)
                    for p_, ph, sl in got:  # every stored token still holds its own row
                        assert pool[(ph, sl)] == (b, h, p_)
                    p_q = L[b] - 1  # the next decode query
                    vis = np.nonzero(visible(kind, sink, window, p_q, np.arange(L[b]),
                                             kept.get((b, h), []), ctx[b] - q[b]))[0]
                    assert set(vis.tolist()) <= set(pos.tolist()), (case, t, b, h)
                    stale = sorted(set(pos.tolist()) - set(vis.tolist()))
                    if kind == oracle.GLOBAL:
                        assert not stale
                    elif L[b] > ctx[b]:
                        assert len(stale) <= P - 1
                        assert all(sink <= j <= p_q - window for j in stale)
                    for s in range(2):
                        p0, n, vs, own = (int(x) for x in st[b, h, s])
                        assert -(-n // P) <= own
                    assert _head_pages(st, v2p, b, h) == owned0[(b, h)]
                    if kind == oracle.LOCAL and L[b] > ctx[b]:
                        assert len(pos) <= sink + window + P - 1


def test_owned_pages_are_reached():
    # With a long enough growth every segment uses all the pages it owns at some point, so the
    # owned counts are no larger than needed.
    rng = np.random.default_rng(13)
    for _ in range(40):
        P = int(rng.choice([4, 8]))
        B, Hkv = 1, int(rng.integers(2, 5))
        pol = _random_policy(rng, Hkv, P)
        steps = max(w for _, _, w in pol) + 3 * P + 2 * P
        ctx, q, pol, st, kl, v2p = _trajectory(rng, P, B, Hkv, steps, pol=pol)
        owned = [int(st[0, h, 0, 3] + st[0, h, 1, 3]) for h in range(Hkv)]
        peak = [0] * Hkv

        def used(st):
            return [sum(-(-int(st[0, h, s, 1]) // P) for s in range(2)) for h in range(Hkv)]

        peak = used(st)
        for _ in range(steps):
            st, kl, v2p, _ = append_step(st, kl, v2p, pol, P)
            peak = [max(a, b) for a, b in zip(peak, used(st))]
        assert peak == owned, (pol, ctx, q)


def test_full_segment_raises():
    P = 4
    pol = [(oracle.GLOBAL, 0, 1), (oracle.LOCAL, 0, 3)]
    st, kl, nv = grow_tables([5], [1], [3], pol, P)
    assert st[0, 0, 0, 3] == 2  # ceil(8 / 4)
    v2p = np.arange(nv, dtype=np.int32)
    for _ in range(3):
        st, kl, v2p, _ = append_step(st, kl, v2p, pol, P)
    with pytest.raises(ValueError):
        append_step(st, kl, v2p, pol, P)


def test_owned_pages_closed_forms():
    P = 16
    # GLOBAL: ceil((L + R) / P)
    assert owned_pages(oracle.GLOBAL, 0, 1, 100, 1, 60, P)[1] == [10]
    # ring with S = 0, built for one query: W = 64 stored, owns ceil((64 + 15) / 16) = 5
    segs, own = owned_pages(oracle.LOCAL, 0, 64, 1000, 1, 500, P)
    assert segs == [(936, 64)] and own == [5]
    # the same ring with a growth too short to reach a fifth page: 64 + 3 tokens -> 5 pages,
    # 64 + 0 -> 4 pages
    assert owned_pages(oracle.LOCAL, 0, 64, 1000, 1, 3, P)[1] == [5]
    assert owned_pages(oracle.LOCAL, 0, 64, 1000, 1, 0, P)[1] == [4]
    # split head after a 300-token prefill chunk: the ring keeps its build pages
    segs, own = owned_pages(oracle.LOCAL, 4, 64, 1000, 300, 500, P)
    assert segs == [(0, 4), (637, 363)] and own == [1, 23]


def test_retrieval_growth_closed_form():
    # L = 100, q = 10, S = 4, p = 250, reserve 30, P = 16: the kept prefix (26 tokens) keeps its
    # 2 pages, the chunk owns ceil((10 + 30) / 16) = 3; each append lands in the chunk.
    pol = [(oracle.RETRIEVAL, 4, 250)]
    st, kl, nv = grow_tables([100], [10], [30], pol, 16)
    assert st[0, 0].tolist() == [[0, 26, 0, 2], [90, 10, 2, 3]] and nv == 5
    st2, kl2, v2p, w = append_step(st, kl, np.arange(nv), pol, 16)
    assert st2[0, 0].tolist() == [[0, 26, 0, 2], [90, 11, 2, 3]] and kl2[0, 0] == 37
    assert w == [(0, 0, 100, 2, 10)]
    with pytest.raises(ValueError):  # a growing retrieval head needs a query chunk
        grow_tables([100], [0], [30], pol, 16)


def test_adaptive_and_empty_context_rejected():
    with pytest.raises(ValueError):
        grow_tables([100], [1], [10], [(oracle.LOCAL_ADAPTIVE, 4, 2)], 16)
    with pytest.raises(ValueError):
        grow_tables([0], [0], [10], [(oracle.GLOBAL, 0, 1)], 16)
