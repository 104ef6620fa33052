"""Host logic of the work list (no GPU): the plan the library would upload, decoded and checked
against sets derived from the oracle's page plan and visibility rule.

For every (request, KV head) the work items' query blocks must partition the request's query
rows; for every query block the items' KV steps must cover exactly the stored slots that some
query of the block can see, each once (a slot covered twice would be counted twice in the
softmax); split items must form one combine group per block with distinct partial slots.
"""

import numpy as np
import pytest

import oracle
from head_aware_paged_segpaged_amd import segpaged_attention_plan_host
from workloads import GLOBAL, LOCAL, LOCAL_ADAPTIVE, RETRIEVAL, config_case, custom_case

STEP = 64          # stored slots per KV step
TILE_ROWS = 128    # rows of a prefill item
DECODE_ROWS = 16   # rows of a decode item


def decode_plan(buf):
    """Header counts, queue bounds, prefill/decode items [n][16] and combine items [n][8]."""
    i32 = buf[:1024].view(np.int32)
    i64 = buf[:1024].view(np.int64)
    n_pre, n_dec, n_comb = int(i32[6]), int(i32[7]), int(i32[8])
    pre_q, dec_q = i32[10:19].copy(), i32[19:28].copy()
    off_pre, off_dec, off_comb = int(i64[14]), int(i64[15]), int(i64[16])
    pre = buf[off_pre:off_pre + 64 * n_pre].view(np.int32).reshape(n_pre, 16)
    dec = buf[off_dec:off_dec + 64 * n_dec].view(np.int32).reshape(n_dec, 16)
    comb = buf[off_comb:off_comb + 32 * n_comb].view(np.int32).reshape(n_comb, 8)
    return pre_q, dec_q, pre, dec, comb


def item_slots(it):
    """(segment, slot) pairs covered by the KV steps [c_begin, c_end) of one item."""
    (ra_seg, ra_b, ra_e, rb_seg, rb_b, rb_e, c0, c1) = (int(x) for x in it[4:12])
    n_ra = (-(-ra_e // STEP) - ra_b // STEP) if ra_e > ra_b else 0
    out = []
    for c in range(c0, c1):
        if c < n_ra:
            seg, lo, hi, base = ra_seg, ra_b, ra_e, ra_b // STEP + c
        else:
            seg, lo, hi, base = rb_seg, rb_b, rb_e, rb_b // STEP + (c - n_ra)
        for slot in range(max(lo, base * STEP), min(hi, base * STEP + STEP)):
            out.append((seg, slot))
    return out


def visible_slots(case, b, h, t0, nq):
    """(segment, slot) of every stored token some query t0 .. t0+nq-1 of request b sees."""
    L, q = int(case.ctx_len[b]), int(case.q_len[b])
    kind, sink, window = oracle.head_policy(*(int(x) for x in case.policy[h]), L)
    segs = oracle.segments(kind, sink, window, L, q)
    p = np.arange(L - q + t0, L - q + t0 + nq)
    out = set()
    if kind == RETRIEVAL:
        # the kept prefix tokens (the first segment unless the prefix is empty) are all
        # visible; the chunk is read causally
        for s, (pos0, n) in enumerate(segs):
            if pos0 == L - q and s == len(segs) - 1 and q > 0:
                out.update((s, i) for i in range(int(p.max()) + 1 - pos0))
            else:
                out.update((s, i) for i in range(n))
        return out
    for s, (pos0, n) in enumerate(segs):
        j = np.arange(pos0, pos0 + n)
        seen = oracle.visible(kind, sink, window, p[:, None], j[None, :]).any(axis=0)
        out.update((s, int(x)) for x in (j[seen] - pos0))
    return out


def check_plan(case, slots=512):
    buf, _ = segpaged_attention_plan_host(case.dtype, case.Hq, case.Hkv, case.D, case.P,
                                          case.ctx_len, case.q_len, case.policy, slots, slots)
    pre_q, dec_q, pre, dec, comb = decode_plan(buf)
    G = case.Hq // case.Hkv
    for q, items in ((pre_q, pre), (dec_q, dec)):
        assert q[0] == 0 and q[-1] == len(items) and np.all(np.diff(q) >= 0)
    assert np.all(pre[:, 3] * G <= TILE_ROWS) and np.all(dec[:, 3] * G <= DECODE_ROWS)
    q_row0 = np.concatenate([[0], np.cumsum(case.q_len)[:-1]])
    kv_row0 = np.concatenate([[0], np.cumsum(case.ctx_len)[:-1]])
    blocks = {}
    for it in np.concatenate([pre, dec]):
        b, h, t0, nq = (int(x) for x in it[:4])
        assert 0 <= b < case.B and 0 <= h < case.Hkv and nq > 0
        assert it[10] < it[11], "empty item"
        assert it[13] == q_row0[b] and it[15] == kv_row0[b]
        assert it[14] == case.ctx_len[b] - case.q_len[b]
        blocks.setdefault((b, h, t0, nq), []).append(it)
    # query blocks partition every (request, head)'s rows
    for b in range(case.B):
        for h in range(case.Hkv):
            tq = sorted((k[2], k[3]) for k in blocks if k[0] == b and k[1] == h)
            want = int(case.q_len[b]) if visible_slots(case, b, h, 0, int(case.q_len[b])) else 0
            got = 0
            for t0, nq in tq:
                assert t0 == got
                got += nq
            assert got == want, (b, h)
    # KV coverage: exactly the visible stored slots, each once
    parts = {}
    for (b, h, t0, nq), its in blocks.items():
        covered = [s for it in its for s in item_slots(it)]
        assert len(covered) == len(set(covered)), "a slot is covered twice"
        assert set(covered) == visible_slots(case, b, h, t0, nq)
        split = [int(it[12]) for it in its]
        if len(its) == 1:
            assert split == [-1]
        else:
            assert all(s >= 0 for s in split) and len(set(split)) == len(split)
            parts[(b, h, t0, nq)] = sorted(split)
    # one combine group per split block, listing exactly its partial slots
    assert len(comb) == len(parts)
    for c in comb:
        key = tuple(int(x) for x in c[:4])
        assert parts[key] == list(range(int(c[4]), int(c[4]) + int(c[5])))
        assert c[6] == q_row0[key[0]]
    return len(pre), len(dec), len(comb)


@pytest.mark.parametrize("index", [0, 1, 3])
def test_plan_covers_each_visible_slot_once(index):
    check_plan(config_case(index, with_tensors=False))


def test_plan_random_shapes():
    rng = np.random.default_rng(7)
    for trial in range(12):
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.choice([1, 2, 4, 8, 16]))
        B = int(rng.integers(1, 4))
        P = int(rng.choice([16, 32, 64, 128, 256]))
        ctx = rng.integers(0, 3000, B)
        q = np.minimum(ctx, rng.choice([1, 2, 7, 64, 300], B))
        pol = []
        for _ in range(Hkv):
            r = rng.random()
            if r < 0.3:
                pol.append((GLOBAL, 0, 1))
            elif r < 0.42:  # top fraction of the prefix by importance, sink, chunk
                pol.append((RETRIEVAL, int(rng.choice([0, 4])), int(rng.choice([1, 100, 999, 1000]))))
            elif r < 0.5:  # window = context length // divisor, per request
                pol.append((LOCAL_ADAPTIVE, int(rng.choice([0, 4])), int(rng.choice([1, 2, 5, 40]))))
            else:
                pol.append((LOCAL, int(rng.choice([0, 1, 4, 70])), int(rng.choice([1, 33, 64, 500]))))
        c = custom_case(100 + trial, dtype="bf16", Hq=Hkv * G, Hkv=Hkv, D=64, P=P,
                        ctx_len=list(ctx), q_len=list(q), policy=pol)
        check_plan(c, slots=int(rng.choice([1, 7, 512])))
