"""GPU parity of decode-time growth: the growable build, segpaged_append and the table-driven
segpaged_decode, through the C ABI, against oracle/append.py and the dense oracle (needs gfx950).

A case is one seeded sequence per request of final length L + N. The layout is built from its
first L tokens (with a prefill chunk of q tokens), then N decode steps each append token L + t
and run decode with the query at that position; the case's last N query rows are exactly those
queries, so one oracle call gives every step's expected output. Bars: tables, v2p and pool rows
bit-exact; O within the same bounds as the other parity tests.
"""

import numpy as np
import pytest
import torch

import oracle
from head_aware_paged_segpaged_amd import SP_ERR_SEGMENT_FULL, SegPagedDecoder, SegPagedLayer
from tests.helpers import COS_MIN, DEV, MAXABS, group_parity, head_major, to_device, to_f64
from workloads import GLOBAL, LOCAL, RETRIEVAL, custom_case, free_list, importance_scores

pytestmark = pytest.mark.gpu


def _split_rows(x, lengths, keep):
    """Rows of the first keep[b] tokens of each request from [sum(lengths), ...]."""
    out, r = [], 0
    for n, k in zip(lengths, keep):
        out.append(x[r:r + k])
        r += n
    return np.ascontiguousarray(np.concatenate(out))


def _token_rows(x, lengths, pos):
    """[B, ...]: row of token pos[b] of each request."""
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    return np.ascontiguousarray(x[starts + np.asarray(pos)])


def _check_pool(dec, st, v2p, case, final_len, keeps=None):
    kp, vp = dec.k_pool.cpu(), dec.v_pool.cpu()
    starts = np.concatenate([[0], np.cumsum(final_len)[:-1]])
    kk = to_device(case.k, case.dtype).cpu()
    vv = to_device(case.v, case.dtype).cpu()
    for b in range(case.B):
        for h in range(case.Hkv):
            got = oracle.gather_positions(st, v2p, case.P, b, h, (keeps or {}).get((b, h)))
            pos = np.array([g[0] for g in got], dtype=np.int64)
            ph = torch.tensor([g[1] for g in got], dtype=torch.long)
            sl = torch.tensor([g[2] for g in got], dtype=torch.long)
            rows = torch.from_numpy(starts[b] + pos)
            assert torch.equal(kp[ph, sl], kk[rows, h]), (b, h)
            assert torch.equal(vp[ph, sl], vv[rows, h]), (b, h)


def _cos_maxabs(got, ref):
    maxabs = float(np.abs(got - ref).max())
    cos = 1.0
    for hq in range(got.shape[0]):
        a, b = got[hq].ravel(), ref[hq].ravel()
        cos = min(cos, float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b))))
    return maxabs, cos


def _run(seed, dtype, Hq, Hkv, D, P, ctx, qb, steps, policy, mask_seed=None, prefill_check=True):
    # The case's query chunk is the build's chunk followed by the decode steps' queries, so the
    # oracle sees the same prefix boundary as the build (it decides what RETRIEVAL heads keep).
    ctx, qb = np.asarray(ctx), np.asarray(qb)
    final = ctx + steps
    case = custom_case(seed, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, P=P, ctx_len=final,
                       q_len=qb + steps, policy=policy, name="append")
    print("case append seed", seed, dtype, "P", P, "ctx", ctx.tolist(), "q", qb.tolist(),
          "steps", steps, "policy", np.asarray(policy).tolist(), flush=True)
    retrieval = bool((case.policy[:, 0] == RETRIEVAL).any())
    imp = importance_scores(case) if retrieval else None
    ref = oracle.attention(case.q, case.k, case.v, final, qb + steps, case.policy, Hq, Hkv,
                           case.scale, dtype, importance=imp)
    k_build = to_device(_split_rows(case.k, final, ctx), dtype)
    v_build = to_device(_split_rows(case.v, final, ctx), dtype)
    reserve = np.full(len(ctx), steps)
    dec = SegPagedDecoder(dtype, Hq, Hkv, D, P, ctx, qb, reserve, policy, DEV)
    st, kl, nv = oracle.grow_tables(ctx, qb, reserve, case.policy, P)
    assert dec.n_virt == nv
    n_phys = nv + 7
    fl = free_list(seed, n_phys)
    imp_build = _split_rows(imp, final, ctx) if retrieval else None
    dec.build(k_build, v_build, fl, n_phys=n_phys, importance=head_major(imp_build))
    v2p = fl[:nv].copy()
    keeps, row0 = {}, 0
    for b in range(len(ctx)):
        for h in range(Hkv):
            kind, sink, window = (int(x) for x in case.policy[h])
            if kind == RETRIEVAL and ctx[b] - qb[b] > 0:
                keeps[(b, h)] = oracle.retrieval_keep(imp_build[row0:row0 + ctx[b], h], sink,
                                                      window, int(ctx[b]), int(qb[b]))
        row0 += int(ctx[b])
    np.testing.assert_array_equal(dec.seg_table.cpu().numpy(), st)
    np.testing.assert_array_equal(dec.kv_len.cpu().numpy(), kl)
    if prefill_check:
        # The build's own prefill chunk runs through segpaged_attention on the growable layout.
        pre = custom_case(seed + 1, dtype=dtype, Hq=Hq, Hkv=Hkv, D=D, P=P, ctx_len=ctx,
                          q_len=qb, policy=policy)
        layer = SegPagedLayer(dtype, Hq, Hkv, D, P, ctx, qb, policy, DEV)
        layer.k_pool, layer.v_pool, layer.n_phys = dec.k_pool, dec.v_pool, dec.n_phys
        layer.seg_table, layer.kv_len, layer.v2p = dec.seg_table, dec.kv_len, dec.v2p
        got = to_f64(layer.attention(to_device(pre.q, dtype), pre.scale))
        exp = oracle.attention(pre.q, _split_rows(case.k, final, ctx),
                               _split_rows(case.v, final, ctx), ctx, qb, case.policy, Hq, Hkv,
                               pre.scale, dtype, importance=imp_build)
        assert float(np.abs(got - exp).max()) <= MAXABS[dtype]
        assert layer.check() == 0
    dec.plan()
    rng = np.random.default_rng(mask_seed) if mask_seed is not None else None
    count = np.zeros(len(ctx), dtype=np.int64)
    q_rows = np.concatenate([[0], np.cumsum(qb + steps)[:-1]]) + qb
    worst = (0.0, 1.0)
    for t in range(steps):
        n_new = None
        if rng is not None and t > 0:
            n_new = (rng.random(len(ctx)) < 0.8).astype(np.int32)
        mask = np.ones(len(ctx), dtype=np.int32) if n_new is None else n_new
        pos = ctx + count
        k_new = to_device(_token_rows(case.k, final, np.minimum(pos, final - 1)), dtype)
        v_new = to_device(_token_rows(case.v, final, np.minimum(pos, final - 1)), dtype)
        dec.append(k_new, v_new, n_new)
        st, kl, v2p, _ = oracle.append_step(st, kl, v2p, case.policy, P, mask)
        count += mask
        rows = q_rows + count - 1
        q = to_device(np.ascontiguousarray(case.q[rows]), dtype)
        out = to_f64(dec.decode(q, case.scale))
        np.testing.assert_array_equal(dec.seg_table.cpu().numpy(), st, err_msg="step %d" % t)
        np.testing.assert_array_equal(dec.kv_len.cpu().numpy(), kl)
        np.testing.assert_array_equal(dec.v2p.cpu().numpy(), v2p)
        for b in range(len(ctx)):
            m, c = _cos_maxabs(out[b], ref[rows[b]])
            worst = (max(worst[0], m), min(worst[1], c))
    assert dec.check() == (0, 0)
    _check_pool(dec, st, v2p, case, final, keeps)
    print("append %s steps %d: maxabs=%.3e min_cos=%.8f" % (dtype, steps, *worst), flush=True)
    assert worst[0] <= MAXABS[dtype] and worst[1] > COS_MIN
    return dec


_POLICY = [(GLOBAL, 0, 1), (LOCAL, 0, 100), (LOCAL, 4, 60), (LOCAL, 20, 300)]


@pytest.mark.parametrize("P", [16, 64])
def test_append_and_decode_match_oracle(P):
    # request 0: one-segment LOCAL heads that split during decode; request 2: a 250-token
    # prefill chunk whose LOCAL rings drop many pages at the first append
    _run(700 + P, "bf16", 8, 4, 128, P, [40, 333, 900], [1, 33, 250], 150, _POLICY)


def test_append_with_idle_requests():
    _run(720, "bf16", 8, 4, 128, 16, [70, 500, 260], [1, 1, 60], 90, _POLICY, mask_seed=5)


def test_append_fp32_d64():
    _run(730, "f32", 4, 2, 64, 32, [50, 400], [1, 100], 70, [(LOCAL, 3, 40), (GLOBAL, 0, 1)])


@pytest.mark.parametrize("P", [16, 64])
def test_append_with_retrieval_heads(P):
    # RETRIEVAL heads grow through their query chunk while LOCAL rings recycle and GLOBAL heads
    # grow beside them; one request is built from a long prefill chunk, one from a decode query
    pol = [(RETRIEVAL, 4, 150), (LOCAL, 4, 60), (GLOBAL, 0, 1), (RETRIEVAL, 0, 1)]
    _run(790 + P, "bf16", 8, 4, 128, P, [700, 2500, 90], [200, 1, 90], 60, pol)


@pytest.mark.parametrize("dtype,Hq,Hkv,D,P", [("bf16", 64, 2, 128, 64), ("bf16", 128, 1, 128, 16),
                                              ("f32", 32, 1, 64, 32)])
def test_append_with_large_query_groups(dtype, Hq, Hkv, D, P):
    # more than 16 query heads per KV head: the table-driven decode runs the prefill kernel's
    # tiles (all G rows of a (request, KV head) against its KV once per split)
    pol = [(LOCAL, 4, 200), (GLOBAL, 0, 1)][:Hkv]
    _run(760 + Hq + P, dtype, Hq, Hkv, D, P, [300, 2000, 90], [1, 50, 90], 40, pol)


def _growth_cases(n=64, seed=6060):
    """Seeded random growth scenarios: GLOBAL, LOCAL and RETRIEVAL heads mixed, 1-32 query
    heads per KV head, page sizes 16-256, idle requests on random steps."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        Hkv = int(rng.integers(1, 4))
        G = int(rng.choice([1, 2, 4, 8, 16, 32]))
        B = int(rng.integers(1, 4))
        ctx = [int(rng.integers(1, 2500)) for _ in range(B)]
        qb = [min(c, int(rng.choice([1, 1, 5, 60]))) for c in ctx]
        pol = []
        for _ in range(Hkv):
            r = rng.random()
            pol.append((GLOBAL, 0, 1) if r < 0.3 else
                       (LOCAL, int(rng.choice([0, 4, 40])), int(rng.choice([1, 30, 64, 300])))
                       if r < 0.75 else (RETRIEVAL, int(rng.choice([0, 4])),
                                         int(rng.choice([100, 500, 1000]))))
        out.append((8000 + i, "f32" if i % 5 == 4 else "bf16", Hkv * G, Hkv,
                    int(rng.choice([64, 128])), int(rng.choice([16, 32, 64, 256])), ctx, qb,
                    int(rng.integers(3, 25)), pol, int(rng.integers(1, 99)) if i % 2 else None))
    return out


@pytest.mark.parametrize("args", _growth_cases(), ids=lambda a: "seed%d" % a[0])
def test_random_growth_sweep(args):
    seed, dtype, Hq, Hkv, D, P, ctx, qb, steps, pol, mask_seed = args
    _run(seed, dtype, Hq, Hkv, D, P, ctx, qb, steps, pol, mask_seed=mask_seed,
         prefill_check=seed % 3 == 0)


def test_append_long_ring_rotation():
    # A ring of 300 pages (window 4200, page 16, a 600-token prefill chunk): rotations go
    # through the three-reversal path; its first append drops 37 pages at once.
    _run(740, "bf16", 8, 2, 128, 16, [5000, 4300], [600, 1], 40,
         [(LOCAL, 0, 4200), (LOCAL, 8, 4100)], prefill_check=False)


@pytest.mark.parametrize("G", [4, 32])
def test_table_decode_is_bitwise_the_planned_decode(G):
    # On a layout written by segpaged_build, the table-driven decode takes the same splits and
    # ranges as the length-planned decode, so O is bitwise identical (G = 32: both run the
    # prefill kernel's tiles).
    rng = np.random.default_rng(750)
    ctx = rng.integers(100, 9000, size=7)
    pol = [(GLOBAL, 0, 1), (LOCAL, 4, 512), (LOCAL, 0, 300), (GLOBAL, 0, 1),
           (LOCAL, 4, 2000), (LOCAL, 16, 64), (LOCAL, 4, 512), (LOCAL, 0, 5000)]
    Hq = 8 * G
    case = custom_case(751, dtype="bf16", Hq=Hq, Hkv=8, D=128, P=64, ctx_len=ctx,
                       q_len=np.ones(7, dtype=np.int32), policy=pol)
    print("case table-decode G", G, ctx.tolist(), flush=True)
    layer = SegPagedLayer("bf16", Hq, 8, 128, 64, ctx, case.q_len, pol, DEV)
    layer.build(to_device(case.k, "bf16"), to_device(case.v, "bf16"),
                free_list(751, layer.n_virt))
    q = to_device(case.q, "bf16")
    a = layer.attention(q, case.scale)
    dec = SegPagedDecoder("bf16", Hq, 8, 128, 64, ctx, case.q_len, np.zeros(7), pol, DEV)
    dec.k_pool, dec.v_pool, dec.n_phys = layer.k_pool, layer.v_pool, layer.n_phys
    dec.seg_table, dec.kv_len, dec.v2p = layer.seg_table, layer.kv_len, layer.v2p
    b = dec.decode(q, case.scale)
    torch.cuda.synchronize()
    assert layer.check() == 0
    assert torch.equal(a, b)


def test_append_past_the_reserve_reports_segment_full():
    P = 16
    pol = [(GLOBAL, 0, 1), (LOCAL, 0, 20)]
    ctx, steps = np.array([30]), 2
    case = custom_case(760, dtype="bf16", Hq=2, Hkv=2, D=128, P=P, ctx_len=ctx + 3,
                       q_len=[3], policy=pol)
    print("case segment-full", flush=True)
    dec = SegPagedDecoder("bf16", 2, 2, 128, P, ctx, [1], [steps], pol, DEV)
    dec.build(to_device(_split_rows(case.k, ctx + 3, ctx), "bf16"),
              to_device(_split_rows(case.v, ctx + 3, ctx), "bf16"), free_list(760, dec.n_virt))
    for t in range(3):
        kn = to_device(_token_rows(case.k, ctx + 3, ctx + t), "bf16")
        vn = to_device(_token_rows(case.v, ctx + 3, ctx + t), "bf16")
        before = dec.seg_table.cpu().numpy().copy()
        dec.append(kn, vn)
        err, _ = dec.check()
        if t < 2:
            assert err == 0
        else:
            # the GLOBAL head owns ceil(32 / 16) = 2 pages: its 33rd token has no page
            assert err == SP_ERR_SEGMENT_FULL
            after = dec.seg_table.cpu().numpy()
            np.testing.assert_array_equal(after[0, 0], before[0, 0])
            assert after[0, 1, 0, 1] + after[0, 1, 1, 1] > 0


@pytest.mark.parametrize("index", [3, 5])
def test_full_size_decode_append_all_rows(index):
    # The full decode workload (64 requests, 4K-128K contexts, or its 32K+ slice) built into a
    # growable layout, then 16 decode steps, each appending a token per request: tables
    # bit-exact against the append oracle after every step, and every row of the last
    # step's output against the dense oracle over the grown contexts.
    from workloads import config_case, decode_tokens
    c = config_case(index)
    n = 16
    print("case full-size append", c.name, flush=True)
    kn, vn, qn = decode_tokens(c, n)
    reserve = np.full(c.B, n)
    dec = SegPagedDecoder(c.dtype, c.Hq, c.Hkv, c.D, c.P, c.ctx_len, c.q_len, reserve, c.policy,
                          DEV)
    dec.build(to_device(c.k, c.dtype), to_device(c.v, c.dtype), free_list(c.seed, dec.n_virt))
    st, kl, nv = oracle.grow_tables(c.ctx_len, c.q_len, reserve, c.policy, c.P)
    v2p = free_list(c.seed, nv)
    dec.plan()
    kd, vd, qd = to_device(kn, c.dtype), to_device(vn, c.dtype), to_device(qn, c.dtype)
    for i in range(n):
        dec.append(kd[i], vd[i])
        out = dec.decode(qd[i], c.scale)
        st, kl, v2p, _ = oracle.append_step(st, kl, v2p, c.policy, c.P)
        np.testing.assert_array_equal(dec.seg_table.cpu().numpy(), st)
        np.testing.assert_array_equal(dec.kv_len.cpu().numpy(), kl)
    np.testing.assert_array_equal(dec.v2p.cpu().numpy(), v2p)
    assert dec.check() == (0, 0)
    got = to_f64(out)
    # every row of the last step (one query per (request, query head)) against the dense
    # oracle over the grown contexts: each request's context followed by its n new tokens
    row0 = np.concatenate([[0], np.cumsum(c.ctx_len)[:-1]])
    k_all = np.concatenate([x for b in range(c.B) for x in
                            (c.k[row0[b]:row0[b] + c.ctx_len[b]], kn[:, b])])
    v_all = np.concatenate([x for b in range(c.B) for x in
                            (c.v[row0[b]:row0[b] + c.ctx_len[b]], vn[:, b])])
    groups = [(b, h, np.array([0])) for b in range(c.B) for h in range(c.Hkv)]
    worst_abs, worst_cos, rows = group_parity(
        c, got, groups, q=qn[n - 1], k=k_all, v=v_all, ctx_len=c.ctx_len + n,
        q_len=np.ones(c.B, dtype=np.int64), q_row0=np.arange(c.B), label="append, last step")
    assert rows == c.B * c.Hq
    assert worst_abs <= MAXABS[c.dtype] and worst_cos > COS_MIN


@pytest.mark.parametrize("Hq", [16, 128])
def test_decode_step_graph_replays_match_eager(Hq):
    # One decode step (append + table-driven decode) captured as a HIP graph and replayed with
    # new inputs copied into its buffers between replays, against the same steps run eagerly
    # on an identical layout: every replay's output and tables bitwise equal (Hq = 128: 32
    # query heads per KV head, the decode runs as prefill tiles).
    from workloads import decode_tokens
    pol = [(GLOBAL, 0, 1), (LOCAL, 0, 40), (LOCAL, 4, 100), (GLOBAL, 0, 1)]
    ctx, steps = np.array([300, 1200, 77]), 30
    c = custom_case(780, dtype="bf16", Hq=Hq, Hkv=4, D=128, P=16, ctx_len=ctx, q_len=[1, 1, 1],
                    policy=pol)
    print("case graph replay Hq", Hq, flush=True)
    kn, vn, qn = decode_tokens(c, steps)
    kd, vd, qd = to_device(kn, "bf16"), to_device(vn, "bf16"), to_device(qn, "bf16")
    decs = []
    for _ in range(2):
        d = SegPagedDecoder("bf16", Hq, 4, 128, 16, ctx, c.q_len, np.full(3, steps), pol, DEV)
        d.build(to_device(c.k, "bf16"), to_device(c.v, "bf16"), free_list(780, d.n_virt))
        d.plan()
        decs.append(d)
    eager, graphed = decs
    k_buf, v_buf, q_buf = kd[0].clone(), vd[0].clone(), qd[0].clone()
    out_buf = torch.empty_like(q_buf)
    g = graphed.capture_step(k_buf, v_buf, q_buf, out_buf, c.scale)
    for t in range(steps):
        k_buf.copy_(kd[t])
        v_buf.copy_(vd[t])
        q_buf.copy_(qd[t])
        g.replay()
        graphed.advance()
        eager.append(kd[t], vd[t])
        oe = eager.decode(qd[t], c.scale)
        torch.cuda.synchronize()
        assert torch.equal(out_buf, oe), t
        assert torch.equal(graphed.seg_table, eager.seg_table)
        assert torch.equal(graphed.v2p, eager.v2p)
    assert graphed.check() == (0, 0) and eager.check() == (0, 0)
