"""Pins for the page-plan oracle (CPU only).

The plan's rules come from page "RedKnot SegPagedAttention runtime design", section 3. The
pins: a hand-derived worked example (tests/golden/tiny_tables.json), closed-form page counts,
page totals derived by hand for the 8K and 128K workloads, and -- tying storage to the
visibility definition -- the stored positions of each head must be exactly the union of the
positions its chunk's queries can see (built by brute force).
"""

import json
import os

import numpy as np
import pytest

from oracle import GLOBAL, LOCAL, gather_positions, plan_tables, segments
from oracle import brute
from workloads import config_case, free_list

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_tables.json")


def test_tiny_worked_example():
    g = json.load(open(GOLDEN))
    seg, kv_len, n_virt = plan_tables(g["ctx_len"], g["q_len"], g["policy"], g["page_size"])
    np.testing.assert_array_equal(seg, np.array(g["seg_table"], dtype=np.int32))
    np.testing.assert_array_equal(kv_len, np.array(g["kv_len"], dtype=np.int32))
    assert n_virt == g["n_virt"]


@pytest.mark.parametrize("index,expected", [(0, 59), (1, 358), (4, 20136)])
def test_page_totals_of_fixed_workloads(index, expected):
    # 8K workload: 2 GLOBAL heads x 128 pages + 6 LOCAL heads x (1 + ceil(1023/64)) = 358.
    # 128K workload: 8 x 2048 + 56 x (1 + ceil(4223/64)) = 20136.
    c = config_case(index, with_tensors=False)
    _, _, n_virt = plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    assert n_virt == expected


def _closed_form_pages(kind, S, W, L, q, P):
    if L == 0:
        return 0
    if kind == GLOBAL:
        return -(-L // P)
    s = min(S, L)
    r0 = max(0, L - q - W + 1)
    if r0 <= s:
        return -(-L // P)
    return -(-s // P) + -(-(L - r0) // P)


def test_page_counts_closed_form():
    rng = np.random.default_rng(0)
    for _ in range(400):
        P = int(rng.choice([16, 32, 64]))
        L = int(rng.integers(0, 300))
        q = int(rng.integers(0, L + 1))
        kind = int(rng.integers(0, 2))
        S = int(rng.integers(0, 10))
        W = int(rng.integers(1, 200))
        seg, kv, n_virt = plan_tables([L], [q], [(kind, S, W)], P)
        assert n_virt == _closed_form_pages(kind, S, W, L, q, P)
        assert seg[0, 0, :, 3].sum() == n_virt
        assert kv[0, 0] == seg[0, 0, :, 1].sum()


def test_stored_set_is_union_of_visible_sets():
    rng = np.random.default_rng(1)
    for _ in range(300):
        L = int(rng.integers(1, 120))
        q = int(rng.integers(0, L + 1))
        kind = int(rng.integers(0, 2))
        S = int(rng.integers(0, 8))
        W = int(rng.integers(1, 130))
        stored = []
        for pos, n in segments(kind, S, W, L, q):
            stored.extend(range(pos, pos + n))
        assert stored == sorted(set(stored)), "segments overlap or are out of order"
        union = set()
        for p in range(L - q, L):
            union |= set(brute.visible_set(kind, S, W, p))
        if q > 0:
            assert set(stored) == union, (kind, S, W, L, q)


def test_layout_invariants_and_gather():
    c = config_case(0, with_tensors=False)
    seg, kv_len, n_virt = plan_tables(c.ctx_len, c.q_len, c.policy, c.P)
    fl = free_list(c.seed, n_virt + 5)
    v2p = fl[:n_virt]
    assert len(set(v2p.tolist())) == n_virt
    # virtual pages are contiguous per segment and handed out in (b, h, seg) order
    nxt = 0
    for b in range(c.B):
        for h in range(c.Hkv):
            for s in range(2):
                pos, n, vstart, npg = seg[b, h, s]
                assert vstart == nxt
                assert npg == -(-n // c.P)
                nxt += npg
    assert nxt == n_virt
    # every stored position appears once, in a distinct (page, slot)
    slots = set()
    for b in range(c.B):
        for h in range(c.Hkv):
            rows = gather_positions(seg, v2p, c.P, b, h)
            assert len(rows) == kv_len[b, h]
            for pos, page, slot in rows:
                assert (page, slot) not in slots
                slots.add((page, slot))
                assert 0 <= slot < c.P


def test_empty_and_degenerate_heads():
    assert segments(LOCAL, 4, 8, 0, 0) == []
    assert segments(GLOBAL, 0, 1, 0, 0) == []
    # sink longer than the context is clipped; window covering everything merges
    assert segments(LOCAL, 50, 3, 10, 10) == [(0, 10)]
    assert segments(LOCAL, 2, 100, 10, 1) == [(0, 10)]
    assert segments(LOCAL, 0, 3, 10, 1) == [(7, 3)]
    seg, kv, n = plan_tables([0, 5], [0, 2], [(LOCAL, 4, 2)], 16)
    assert kv.tolist() == [[0], [5]]
    assert seg[0, 0].tolist() == [[0, 0, 0, 0], [0, 0, 0, 0]]
    assert seg[1, 0].tolist() == [[0, 5, 0, 1], [0, 0, 1, 0]]


def test_adaptive_window_tables_worked_example():
    # Page "RedKnot head classification": a LOCAL window may follow the request's context
    # length, its example being half of it. Two requests, sink 4, divisor 2, pages of 16:
    #   L = 1000, q = 100 -> W = 500, R0 = 1000 - 100 - 500 + 1 = 401:
    #     segments (0, 4) -> 1 page, (401, 599) -> ceil(599 / 16) = 38 pages.
    #   L = 300, q = 1 -> W = 150, R0 = 300 - 1 - 150 + 1 = 150:
    #     segments (0, 4) -> 1 page, (150, 150) -> ceil(150 / 16) = 10 pages.
    # Virtual pages in (request, head, segment) order: 0, 1 | 39, 40; 50 in total.
    from oracle import LOCAL_ADAPTIVE
    seg, kv_len, n_virt = plan_tables([1000, 300], [100, 1], [(LOCAL_ADAPTIVE, 4, 2)], 16)
    np.testing.assert_array_equal(seg[0, 0], [[0, 4, 0, 1], [401, 599, 1, 38]])
    np.testing.assert_array_equal(seg[1, 0], [[0, 4, 39, 1], [150, 150, 40, 10]])
    np.testing.assert_array_equal(kv_len, [[603], [154]])
    assert n_virt == 50


def test_adaptive_window_divisor_one_stores_like_global():
    # Divisor 1 gives W = L, so every query of the chunk sees the whole prefix: the head's
    # storage must be a GLOBAL head's, for any sink and chunk length.
    from oracle import LOCAL_ADAPTIVE
    rng = np.random.default_rng(3)
    for _ in range(50):
        B = int(rng.integers(1, 4))
        L = rng.integers(1, 500, B)
        q = np.array([int(rng.integers(1, x + 1)) for x in L])
        S = int(rng.integers(0, 9))
        a = plan_tables(L, q, [(LOCAL_ADAPTIVE, S, 1)], 32)
        g = plan_tables(L, q, [(GLOBAL, 0, 1)], 32)
        np.testing.assert_array_equal(a[0], g[0])
        np.testing.assert_array_equal(a[1], g[1])


def test_layers_worked_example():
    # Two layers, two requests, one KV head, pages of 16 (virtual pages in request, layer,
    # head, segment order). Layer 0: GLOBAL. Layer 1: LOCAL sink 2, window 20.
    #   request 0, L = 50, q = 10: layer 0 (0, 50) -> 4 pages [0, 4);
    #     layer 1: R0 = 50 - 10 - 20 + 1 = 21 -> (0, 2) 1 page [4], (21, 29) 2 pages [5, 7).
    #   request 1, L = 16, q = 16: layer 0 (0, 16) -> 1 page [7];
    #     layer 1: R0 = max(0, 16 - 16 - 20 + 1) = 0 <= 2 -> one segment (0, 16), 1 page [8].
    from oracle import plan_tables_layers
    pol = [[(GLOBAL, 0, 1)], [(LOCAL, 2, 20)]]
    seg, kv_len, n_virt = plan_tables_layers([50, 16], [10, 16], pol, 16)
    np.testing.assert_array_equal(seg[0, 0, 0], [[0, 50, 0, 4], [0, 0, 4, 0]])
    np.testing.assert_array_equal(seg[1, 0, 0], [[0, 2, 4, 1], [21, 29, 5, 2]])
    np.testing.assert_array_equal(seg[0, 1, 0], [[0, 16, 7, 1], [0, 0, 8, 0]])
    np.testing.assert_array_equal(seg[1, 1, 0], [[0, 16, 8, 1], [0, 0, 9, 0]])
    np.testing.assert_array_equal(kv_len, [[[50], [16]], [[31], [16]]])
    assert n_virt == 9


def test_layers_match_single_layer_tables_up_to_page_numbering():
    # Each layer stores what a one-layer layout with its policies stores; only the virtual
    # page numbers move, and the totals add up.
    from oracle import plan_tables_layers
    rng = np.random.default_rng(11)
    for _ in range(30):
        B, Hkv, n_layers = int(rng.integers(1, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 5))
        ctx = rng.integers(0, 400, B)
        q = np.array([int(rng.integers(0, x + 1)) for x in ctx])
        pol = [[(int(rng.integers(0, 3)), int(rng.integers(0, 9)), int(rng.integers(1, 6)) * 17)
                for _ in range(Hkv)] for _ in range(n_layers)]
        seg, kvl, n_virt = plan_tables_layers(ctx, q, pol, 32)
        total = 0
        for layer in range(n_layers):
            s1, k1, n1 = plan_tables(ctx, q, pol[layer], 32)
            np.testing.assert_array_equal(seg[layer][..., [0, 1, 3]], s1[..., [0, 1, 3]])
            np.testing.assert_array_equal(kvl[layer], k1)
            total += n1
        assert n_virt == total
        if n_layers == 1:
            np.testing.assert_array_equal(seg[0], plan_tables(ctx, q, pol[0], 32)[0])
