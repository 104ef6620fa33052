"""Pins for the attention oracle (CPU only).

Each test checks ``oracle.attention`` against something it does not compute itself:
pure-Python brute force, closed forms, library routines on textbook special cases and
invariants of the definition (page "RedKnot SegPagedAttention runtime design", sections 1-4;
page "RedKnot head classification", head types).
"""

import math

import numpy as np
import pytest
import torch

from oracle import GLOBAL, LOCAL, attention, attention_rows, visible
from oracle import brute
from workloads import custom_case


def _rand_policy(rng, Hkv, L):
    pol = []
    for _ in range(Hkv):
        kind = int(rng.integers(0, 2))
        pol.append((kind, int(rng.integers(0, 7)), int(rng.integers(1, L + 3))))
    return pol


@pytest.mark.parametrize("trial", range(12))
def test_against_brute_force(trial):
    rng = np.random.default_rng(100 + trial)
    Hkv = int(rng.integers(1, 3))
    G = int(rng.choice([1, 2, 4]))
    D = int(rng.integers(2, 9))
    B = int(rng.integers(1, 4))
    ctx = [int(rng.integers(1, 49)) for _ in range(B)]
    ql = [int(rng.integers(1, c + 1)) for c in ctx]
    pol = _rand_policy(rng, Hkv, max(ctx))
    dtype = "f32" if trial % 2 else "bf16"
    scale = float(rng.choice([1.0 / math.sqrt(D), 1.0, 0.3]))
    c = custom_case(7 + trial, dtype=dtype, Hq=Hkv * G, Hkv=Hkv, D=D, P=16, ctx_len=ctx,
                    q_len=ql, policy=pol, scale=scale)
    out = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv, c.scale, c.dtype)
    from oracle import to_f64
    q = to_f64(c.q, dtype).tolist()
    k = to_f64(c.k, dtype).tolist()
    v = to_f64(c.v, dtype).tolist()
    q0 = kv0 = 0
    for b in range(B):
        L, nq = ctx[b], ql[b]
        for t in range(nq):
            p = L - nq + t
            for hq in range(c.Hq):
                h = hq // G
                kind, s, w = pol[h]
                krows = [k[kv0 + j][h] for j in range(L)]
                vrows = [v[kv0 + j][h] for j in range(L)]
                ref = brute.attention_row(q[q0 + t][hq], krows, vrows, p, kind, s, w, scale)
                np.testing.assert_allclose(out[q0 + t, hq], ref, rtol=1e-12, atol=1e-12)
        q0 += nq
        kv0 += L


def _closed_form_count(kind, S, W, p):
    if kind == GLOBAL:
        return p + 1
    lo = max(0, p - W + 1)
    return (p - lo + 1) + min(S, lo)


@pytest.mark.parametrize("kind", [GLOBAL, LOCAL])
def test_visible_count_closed_form(kind):
    for S in range(0, 6):
        for W in range(1, 40, 3):
            for p in range(0, 60):
                j = np.arange(0, 80)
                n = int(visible(kind, S, W, p, j).sum())
                assert n == _closed_form_count(kind, S, W, p), (kind, S, W, p)


def test_one_hot_support_and_row_sums():
    # With V[j] = e_j (D >= L), O[p] is the row of attention probabilities itself: its support
    # must be exactly the visible set and it must sum to 1.
    L, nq, Hkv, G = 40, 40, 2, 2
    pol = [(GLOBAL, 0, 1), (LOCAL, 3, 9)]
    c = custom_case(3, dtype="f32", Hq=Hkv * G, Hkv=Hkv, D=L, P=16, ctx_len=[L], q_len=[nq],
                    policy=pol)
    eye = np.eye(L, dtype=np.float32)
    c.v = np.repeat(eye[:, None, :], Hkv, axis=1)
    out = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv, c.scale, c.dtype)
    for t in range(nq):
        p = L - nq + t
        for hq in range(c.Hq):
            kind, s, w = pol[hq // G]
            row = out[t, hq]
            support = sorted(np.nonzero(row > 0)[0].tolist())
            assert support == brute.visible_set(kind, s, w, p)
            assert abs(row.sum() - 1.0) < 1e-12


def test_zero_query_closed_form():
    # Q = 0 makes attention uniform over the visible set; with V[j, 0] = j, O[p, 0] is the mean
    # visible position: p/2 for GLOBAL, and for LOCAL
    # (sum_{j < min(S, lo)} j + sum_{j=lo}^{p} j) / |vis|, lo = max(0, p - W + 1).
    L, nq = 70, 50
    pol = [(GLOBAL, 0, 1), (LOCAL, 4, 16), (LOCAL, 0, 5), (LOCAL, 30, 8)]
    c = custom_case(4, dtype="f32", Hq=4, Hkv=4, D=3, P=16, ctx_len=[L], q_len=[nq], policy=pol)
    c.q[:] = 0
    c.v[:, :, 0] = np.arange(L, dtype=np.float32)[:, None]
    out = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv, c.scale, c.dtype)
    for t in range(nq):
        p = L - nq + t
        assert abs(out[t, 0, 0] - p / 2.0) < 1e-9
        for h in (1, 2, 3):
            _, S, W = pol[h]
            lo = max(0, p - W + 1)
            m = min(S, lo)
            tot = m * (m - 1) / 2.0 + (lo + p) * (p - lo + 1) / 2.0
            cnt = m + (p - lo + 1)
            assert abs(out[t, h, 0] - tot / cnt) < 1e-9


def _sdpa_reference(case, mask_fn):
    """torch SDPA in float64 on the CPU with an explicitly built boolean mask."""
    from oracle import to_f64
    q = torch.from_numpy(to_f64(case.q, case.dtype))
    k = torch.from_numpy(to_f64(case.k, case.dtype))
    v = torch.from_numpy(to_f64(case.v, case.dtype))
    G = case.Hq // case.Hkv
    outs = []
    q0 = kv0 = 0
    for b in range(case.B):
        L, nq = int(case.ctx_len[b]), int(case.q_len[b])
        qb = q[q0:q0 + nq].permute(1, 0, 2)  # [Hq, nq, D]
        kb = k[kv0:kv0 + L].permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        vb = v[kv0:kv0 + L].permute(1, 0, 2).repeat_interleave(G, dim=0).contiguous()
        mask = mask_fn(nq, L)
        o = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=mask,
                                                             scale=case.scale)
        outs.append(o.permute(1, 0, 2))
        q0 += nq
        kv0 += L
    return torch.cat(outs, 0).numpy()


def test_all_global_is_causal_sdpa():
    c = custom_case(5, dtype="bf16", Hq=6, Hkv=3, D=16, P=16, ctx_len=[37, 64, 5],
                    q_len=[37, 20, 1], policy=[(GLOBAL, 4, 8)] * 3)
    out = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv, c.scale, c.dtype)
    ref = _sdpa_reference(c, lambda nq, L: torch.ones(nq, L, dtype=torch.bool).tril(L - nq))
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_local_without_sink_is_sliding_window_sdpa():
    W = 7
    c = custom_case(6, dtype="f32", Hq=4, Hkv=2, D=8, P=16, ctx_len=[50, 23], q_len=[30, 23],
                    policy=[(LOCAL, 0, W)] * 2)
    out = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv, c.scale, c.dtype)

    def band(nq, L):
        ones = torch.ones(nq, L, dtype=torch.bool)
        return ones.tril(L - nq) & ones.triu(L - nq - W + 1)

    ref = _sdpa_reference(c, band)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_local_with_wide_window_equals_global():
    L = 45
    base = dict(dtype="bf16", Hq=2, Hkv=1, D=8, P=16, ctx_len=[L], q_len=[30])
    a = custom_case(9, policy=[(LOCAL, 3, L)], **base)
    b = custom_case(9, policy=[(GLOBAL, 0, 1)], **base)
    oa = attention(a.q, a.k, a.v, a.ctx_len, a.q_len, a.policy, 2, 1, a.scale, a.dtype)
    ob = attention(b.q, b.k, b.v, b.ctx_len, b.q_len, b.policy, 2, 1, b.scale, b.dtype)
    np.testing.assert_array_equal(oa, ob)


def test_local_window_one_sees_sink_and_itself():
    # W = 1: each query sees the sink and its own position only; checked against a two-line
    # softmax written from that statement.
    from oracle import to_f64
    L, nq, S = 30, 20, 3
    c = custom_case(10, dtype="f32", Hq=1, Hkv=1, D=4, P=16, ctx_len=[L], q_len=[nq],
                    policy=[(LOCAL, S, 1)])
    out = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, 1, 1, c.scale, c.dtype)
    q, k, v = (to_f64(x, "f32")[:, 0, :] for x in (c.q, c.k, c.v))
    for t in range(nq):
        p = L - nq + t
        idx = [0, 1, 2, p]
        s = np.array([c.scale * q[t] @ k[j] for j in idx])
        w = np.exp(s - s.max())
        ref = (w[:, None] * v[idx]).sum(0) / w.sum()
        np.testing.assert_allclose(out[t, 0], ref, rtol=1e-12, atol=1e-12)


def test_gqa_isolation():
    # Zero every V head except h*: only query heads hq with hq // G == h* may be non-zero.
    Hkv, G = 4, 3
    c = custom_case(11, dtype="bf16", Hq=Hkv * G, Hkv=Hkv, D=8, P=16, ctx_len=[33],
                    q_len=[9], policy=[(GLOBAL, 0, 1), (LOCAL, 2, 5), (LOCAL, 0, 3),
                                       (GLOBAL, 0, 1)])
    for hstar in range(Hkv):
        v = c.v.copy()
        for h in range(Hkv):
            if h != hstar:
                v[:, h, :] = 0
        out = attention(c.q, c.k, v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv, c.scale,
                        c.dtype)
        for hq in range(c.Hq):
            nz = np.abs(out[:, hq, :]).max() > 0
            assert nz == (hq // G == hstar), (hstar, hq)


def test_rows_subset_matches_full():
    c = custom_case(12, dtype="bf16", Hq=4, Hkv=2, D=8, P=16, ctx_len=[40, 17],
                    q_len=[11, 17], policy=[(LOCAL, 2, 6), (GLOBAL, 0, 1)])
    full = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, 4, 2, c.scale, c.dtype)
    sub = attention_rows(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, 4, 2, c.scale, c.dtype,
                         b=1, hq=3, tokens=[0, 5, 16])
    np.testing.assert_array_equal(sub, full[11 + np.array([0, 5, 16]), 3])


def test_adaptive_window_against_brute_force():
    # Adaptive LOCAL heads (window = L // d per request) against the pure-Python loops, which
    # take the window the page's rule gives for each request, computed here by hand.
    from oracle import LOCAL_ADAPTIVE
    ctx, ql = [40, 23, 9], [9, 23, 1]
    pol = [(LOCAL_ADAPTIVE, 2, 4), (LOCAL_ADAPTIVE, 0, 2), (GLOBAL, 0, 1)]
    windows = {0: [10, 5, 2], 1: [20, 11, 4]}  # 40 // 4, 23 // 4, 9 // 4; 40 // 2, ...
    c = custom_case(77, dtype="f32", Hq=6, Hkv=3, D=5, P=16, ctx_len=ctx, q_len=ql, policy=pol)
    out = attention(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, 6, 3, c.scale, c.dtype)
    q0 = kv0 = 0
    for b in range(3):
        L, nq = ctx[b], ql[b]
        for hq in range(6):
            h = hq // 2
            kind, sink = (LOCAL, pol[h][1]) if h < 2 else (GLOBAL, 0)
            W = windows[h][b] if h < 2 else 1
            k_rows = [list(map(float, r)) for r in c.k[kv0:kv0 + L, h]]
            v_rows = [list(map(float, r)) for r in c.v[kv0:kv0 + L, h]]
            for t in range(nq):
                ref = brute.attention_row(list(map(float, c.q[q0 + t, hq])), k_rows, v_rows,
                                          L - nq + t, kind, sink, W, c.scale)
                np.testing.assert_allclose(out[q0 + t, hq], ref, rtol=1e-12, atol=1e-14)
        q0 += nq
        kv0 += L


def test_adaptive_window_divisor_one_equals_global():
    from oracle import LOCAL_ADAPTIVE
    base = dict(dtype="bf16", Hq=2, Hkv=1, D=8, P=16, ctx_len=[45, 12], q_len=[30, 12])
    a = custom_case(10, policy=[(LOCAL_ADAPTIVE, 3, 1)], **base)
    b = custom_case(10, policy=[(GLOBAL, 0, 1)], **base)
    oa = attention(a.q, a.k, a.v, a.ctx_len, a.q_len, a.policy, 2, 1, a.scale, a.dtype)
    ob = attention(b.q, b.k, b.v, b.ctx_len, b.q_len, b.policy, 2, 1, b.scale, b.dtype)
    np.testing.assert_array_equal(oa, ob)


def test_bf16_conversion_every_bit_pattern():
    """oracle.to_f64 against torch's own bf16 -> float64 conversion on all 65,536 bf16 bit
    patterns (NaN patterns must stay NaN). Every bf16 pin above converts its inputs and its
    reference through to_f64, so this is what ties those pins to the bf16 format itself."""
    from oracle import to_f64

    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = to_f64(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127  # exponent all ones with a non-zero 7-bit mantissa, both signs
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros and infinities keep their sign
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # a few values worked out by hand from the format (sign, 8-bit exponent, 7-bit mantissa)
    assert got[0x3F80] == 1.0 and got[0xC000] == -2.0 and got[0x3F40] == 0.75
    assert got[0x0001] == 2.0 ** -133  # smallest subnormal: 2^-126 * 2^-7
    assert got[0x7F7F] == (2.0 - 2.0 ** -7) * 2.0 ** 127  # largest finite
    assert np.isinf(got[0x7F80]) and got[0xFF80] < 0


def test_group_rows_equal_per_head_rows():
    """attention_group_rows (one K/V conversion for a whole GQA group) returns exactly the rows
    attention_rows computes per query head, for every head kind (bitwise: same arithmetic)."""
    from oracle import attention_group_rows
    from workloads import LOCAL_ADAPTIVE, RETRIEVAL
    rng = np.random.default_rng(77)
    pol = [(GLOBAL, 0, 1), (LOCAL, 4, 40), (LOCAL_ADAPTIVE, 2, 3), (RETRIEVAL, 4, 300)]
    c = custom_case(77, dtype="bf16", Hq=8, Hkv=4, D=64, P=16, ctx_len=[300, 97],
                    q_len=[50, 97], policy=pol)
    imp = rng.standard_normal((int(np.sum(c.ctx_len)), c.Hkv)).astype(np.float32)
    for b in range(c.B):
        toks = np.sort(rng.choice(int(c.q_len[b]), 9, replace=False))
        for h in range(c.Hkv):
            grp = attention_group_rows(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv,
                                       c.scale, c.dtype, b, h, toks, importance=imp)
            for g in range(c.Hq // c.Hkv):
                one = attention_rows(c.q, c.k, c.v, c.ctx_len, c.q_len, c.policy, c.Hq, c.Hkv,
                                     c.scale, c.dtype, b, h * 2 + g, toks, importance=imp)
                assert np.array_equal(grp[g], one)
